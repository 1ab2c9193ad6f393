"""MI355X-native orthonormalized optimizer step (Dion power iteration with error
feedback, and Muon Newton-Schulz) behind a C-ABI library, ``libortho.so``.

Importing the package does not load the library; ``api`` does, and fails loudly
if it has not been built.
"""

__all__ = ["api", "synth"]
