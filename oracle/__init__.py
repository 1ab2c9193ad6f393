"""Plain, slow, fp64 CPU oracle for the orthonormalized optimizer step.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and
the CPU-baseline leg of the benchmark may import it.  The product path (the HIP
library and its Python binding) never imports, links or calls anything here, and
nothing here imports the product package.

What it computes, and where each step comes from (page titles and sections of the
public pages about microsoft/dion):

* ``newton_schulz`` -- Muon's orthogonalization: repeated matrix products that
  push the singular values of the normalised gradient towards one, approximating
  the U V^T factor of the SVD.  MSR talk "Dion: The distributed orthonormal
  update revolution is here", passage contrasting SGD with orthonormal updates
  and the passage on Muon's dense Newton-Schulz matrix products.
* ``gram_newton_schulz`` -- the same iteration written on the small Gram side
  (X_k = Q_k X_0 with Q_k m x m), the optional Gram Newton-Schulz that hysenlabs
  "Microsoft Dion: orthonormal optimizers that assume DTensor parallelism" names
  in its section on installing with the optional kernels.  No formula is
  printed; the reading is this exact algebraic rewrite.
* ``dion_step`` -- Dion's amortised power iteration (one power-iteration step
  per optimizer step, warm-started from the previous right factor), the low-rank
  fraction, error feedback, and the SGD-form weight update.  Same talk, passages
  on amortised power iteration and on low-rank fraction with error feedback;
  agentlenshq "microsoft/dion", section "How it works"; paper page "Dion:
  Distributed Orthonormalized Updates", abstract.

* ``normuon_step`` -- the Muon step with neuron-wise (row) normalisation of the
  orthogonalised momentum before the update (``row_normalize``).  agentlenshq
  "microsoft/dion", section "How it works"; hysenlabs "Microsoft Dion:
  orthonormal optimizers that assume DTensor parallelism", section "Dion3 is not
  a retuning of Dion2, and the README says so".  The
  pages print no formula: the reading is a stateless rescale of every row to
  the common norm ||U||_F / sqrt(m), which keeps the total norm; "parity
  unpinned" as to fidelity, pinned against its own definition.

* ``dion2_step`` -- Dion2: the k rows of B = M + G with the largest norm are
  orthonormalised with Newton-Schulz and applied; error feedback keeps mu times
  the applied rows and every other row whole.  agentlenshq "microsoft/dion",
  sections "How it works" and "Highlights"; hysenlabs, section "Dion3 is not a
  retuning of Dion2, and the README says so".  The selection rule is not
  printed; largest row norm is the reading, "parity unpinned" as to fidelity.

* ``muon_step`` -- the Muon step around the Newton-Schulz path: a heavy-ball
  momentum buffer, its Newton-Schulz orthogonalisation, and the SGD-form update.
  Same talk, same passages.  The momentum form is the plainest reading and
  "parity unpinned" as to fidelity: the pages name Muon's momentum but print no
  formula; the pins check the step against its own definition.

Where the pages leave a step open, the oracle takes the plainest reading they
support: mu is the error-feedback decay (B = M + G, M' = B - (1 - mu) P R^T);
P is the Q-factor of the thin QR with a positive diagonal in R; the new right
factor is R with unit-norm columns; the update scale is 1; Newton-Schulz uses
Muon's quintic (3.4445, -4.7750, 2.0315), eps = 1e-7, and works on the wide
orientation; Muon's momentum is the heavy-ball buffer mu M + G.

Pins: ``tests/test_oracle_pins.py`` checks these functions against closed forms
(SVD), invariants of the definitions, and an independent brute-force
implementation (``oracle.brute``) on tiny inputs.  The fidelity of the readings
themselves to the real method is "parity unpinned": the pages print no update
equation and no worked example.
"""

from .dion_ref import (  # noqa: F401
    MUON_ABC,
    NS_EPS,
    round_bf16,
    round_to_dtype,
    qr_positive,
    dion_step,
    newton_schulz,
    gram_newton_schulz,
    muon_step,
    row_normalize,
    normuon_step,
    select_rows,
    dion2_step,
)
