"""Parity of the HIP path (through the C-ABI) with the fp64 oracle on the same
seeded inputs.  Tolerances are relative Frobenius errors: 1e-4 for fp32 inputs
(Dion and Newton-Schulz), 2e-2 for bf16 inputs with fp32 accumulation."""

import numpy as np
import pytest
import torch

import oracle
from orthonormal_optimizer_update_amd import api, synth

from parity_util import TOL, gpu_dion_step, gpu_ns, note, rel, run_dion_parity, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.lib()   # the HIP library must load; there is no fallback
    torch.cuda.set_device(0)


# ----------------------------------------------------------------------------
# Newton-Schulz
# ----------------------------------------------------------------------------

NS_SHAPES = [(64, 64), (100, 300), (300, 100), (257, 513), (1, 50), (128, 4096), (520, 520),
             (128, 1000), (64, 333), (333, 128)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", NS_SHAPES)
def test_ns_small(shape, dtype):
    X, G, _ = synth.small_case(1, shape[0], shape[1], 1, dtype, x_scale=1.0)
    note(f"ns {shape} {dtype}")
    got = gpu_ns(G, dtype)
    want = oracle.newton_schulz(G)
    assert rel(got, want) <= TOL[dtype]


def test_ns_zero_steps0_and_custom_coefficients():
    _, G, _ = synth.small_case(2, 96, 160, 1, "bf16")
    note("ns zero input")
    assert np.all(gpu_ns(np.zeros((96, 160), np.float32), "bf16") == 0)
    note("ns steps=0")
    assert rel(gpu_ns(G, "f32", steps=0), oracle.newton_schulz(G, steps=0)) <= 1e-6
    note("ns cubic coefficients")
    cubic = (1.5, -0.5, 0.0)
    assert rel(gpu_ns(G, "bf16", steps=8, abc=cubic), oracle.newton_schulz(G, 8, cubic)) <= TOL["bf16"]
    # 64- and 128-row sides wide enough for the k-split Gram: with c = 0 the
    # split partials go through the plain reduce and the linear polynomial,
    # otherwise through the fused one-workgroup-per-member polynomial
    _, G2, _ = synth.small_case(4, 128, 1024, 1, "bf16", x_scale=1.0)
    note("ns cubic 128x1024 (split Gram, c = 0)")
    assert rel(gpu_ns(G2, "bf16", steps=8, abc=cubic), oracle.newton_schulz(G2, 8, cubic)) <= TOL["bf16"]
    _, G3, _ = synth.small_case(5, 64, 768, 1, "f32", x_scale=1.0)
    note("ns quintic 64x768 bf16 (split Gram, fused polynomial)")
    assert rel(gpu_ns(G3, "bf16"), oracle.newton_schulz(G3)) <= TOL["bf16"]
    # fp32 inputs take fp32-accurate products
    note("ns quintic 64x768 f32")
    assert rel(gpu_ns(G3, "f32"), oracle.newton_schulz(G3)) <= TOL["f32"]
    note("ns cubic 128x1024 f32")
    assert rel(gpu_ns(G2, "f32", steps=8, abc=cubic), oracle.newton_schulz(G2, 8, cubic)) <= TOL["f32"]


def test_ns_f32_planted_1024x1536():
    """fp32 input with a dominant rank-32 part: fp32-accurate products, both
    orientations."""
    S = synth.planted(22, 1024, 1536, 32, 10.0)
    G = synth.gradient(22, 1024, 1536, 1, "f32", planted_part=S)
    note("ns f32 planted 1024x1536")
    assert rel(gpu_ns(G, "f32"), oracle.newton_schulz(G)) <= TOL["f32"]
    note("ns f32 planted 1536x1024")
    Gt = np.ascontiguousarray(G.T)
    assert rel(gpu_ns(Gt, "f32"), oracle.newton_schulz(Gt)) <= TOL["f32"]


def test_ns_output_may_alias_input():
    _, G, _ = synth.small_case(3, 200, 136, 1, "bf16")
    g = to_dev(G, "bf16")
    note("ns aliased")
    api.newton_schulz(g, out=g)
    torch.cuda.synchronize()
    assert rel(to_host(g), oracle.newton_schulz(G)) <= TOL["bf16"]


def test_ns_planted_square_4096():
    """The 4096 x 4096 workload: G = E + S with a rank-32 part of 10x norm."""
    wl = synth.WORKLOADS[2]
    S = synth.planted(2, 4096, 4096, 32, wl["planted_ratio"])
    G = synth.gradient(2, 4096, 4096, 1, "bf16", planted_part=S)
    note("ns 4096 planted")
    got = gpu_ns(G, "bf16")
    assert rel(got, oracle.newton_schulz(G)) <= TOL["bf16"]


def test_ns_wide_2048x8192_deterministic():
    """A wide 2048 x 8192 matrix (Gram over 36 tiles on and above the
    diagonal, mirrored): matches the oracle and gives the same bits on a second
    run."""
    G = synth.gradient(11, 2048, 8192, 1, "bf16")
    note("ns 2048x8192")
    got = gpu_ns(G, "bf16")
    assert rel(got, oracle.newton_schulz(G)) <= TOL["bf16"]
    again = gpu_ns(G, "bf16")
    assert np.array_equal(got, again)


def test_ns_tall_4096x2048():
    """A tall 4096 x 2048 matrix: the iteration runs on the transpose (Gram side
    2048, the 256 x 256 products) and the last apply writes the bf16 output
    transposed, through the LDS-staged row pieces of the transposed tile."""
    G = synth.gradient(13, 4096, 2048, 1, "bf16")
    note("ns 4096x2048 tall")
    got = gpu_ns(G, "bf16")
    assert got.shape == (4096, 2048)
    assert rel(got, oracle.newton_schulz(G)) <= TOL["bf16"]


@pytest.mark.parametrize("members,side", [(5, 1792), (4, 2048)])
def test_ns_symmetric_tile_maps(members, side):
    """The symmetric Gram and polynomial kernels' two workgroup-to-tile maps,
    on batched groups large enough to take that kernel: 5 x 1792^2 (a 7 x 7
    tile grid, not a multiple of four: each XCD a run of the row-ordered walk)
    and 4 x 2048^2 (8 x 8: the XCD block partition with 2 x 2-tile blocks)."""
    Gs = [synth.gradient(15, side, side, 1, "bf16", index=i) for i in range(members)]
    note(f"ns batched {members} x {side}^2 symmetric tile maps")
    outs = api.newton_schulz_batched([to_dev(g, "bf16") for g in Gs], steps=5)
    torch.cuda.synchronize()
    for i in range(members):
        assert rel(to_host(outs[i]), oracle.newton_schulz(Gs[i])) <= TOL["bf16"], i


def test_ns_square_4096_deterministic():
    """Two runs of the 4096 x 4096 iteration give the same bits."""
    G = synth.gradient(12, 4096, 4096, 1, "bf16")
    note("ns 4096 deterministic")
    a = gpu_ns(G, "bf16", steps=2)
    b = gpu_ns(G, "bf16", steps=2)
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------------
# Dion
# ----------------------------------------------------------------------------

DION_SHAPES = [(96, 80, 16), (300, 200, 37), (513, 257, 64), (128, 1000, 128), (1000, 128, 100),
               (40, 30, 30), (7, 9, 1), (700, 900, 250),
               # bf16: the streaming update at r = 256 and (rows not 256-divisible)
               # r = 512; the 256 x 256 pair at r = 512; r = 1024 on the
               # two-accumulator kernel (1152 rows: not 256-divisible)
               (384, 352, 256), (640, 1056, 512), (768, 1024, 512), (1152, 2048, 1024)]

# bf16: the streaming sweeps (r = 64, 128, 256, 512 with both sides multiples
# of 64), with a last row tile of 64 rows, and r = m = n; at r = 512 with the
# orthonormalisation products on the 256 x 256 kernel (m a multiple of 256,
# 3 r <= n: the first reduce writes P~'s pieces, the last one P's transposed
# pieces k-blocked) and without them (576 rows).  (fp32 weights take the
# generic sweeps; on (256, 256, 256) and (1024, 512, 256) their P~ is
# conditioned badly enough that fp32-accurate products land at 1.1e-4 and
# 1.7e-4 against the fp64 oracle, above the fp32 bar.)
STREAM_SHAPES = [(384, 320, 64), (320, 448, 128), (576, 768, 256), (256, 256, 256),
                 (1024, 512, 256), (512, 1536, 512), (1024, 2048, 512), (576, 1024, 512)]


@pytest.mark.parametrize("shape", STREAM_SHAPES)
def test_dion_streaming_sweeps(shape):
    m, n, r = shape
    X, G1, Q0 = synth.small_case(10 + r, m, n, r, "bf16", planted_rank=min(4, r))
    Gs = [G1] + [synth.gradient(1010 + r, m, n, t, "bf16") for t in (2, 3)]
    worst, recs = run_dion_parity(X, Gs, Q0, mu=0.95, lr=0.01, dtype="bf16", label="stream")
    print(shape, worst)
    assert max(worst.values()) <= TOL["bf16"], recs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", DION_SHAPES)
def test_dion_small(shape, dtype):
    m, n, r = shape
    X, G1, Q0 = synth.small_case(10 + r, m, n, r, dtype, planted_rank=min(4, r))
    Gs = [G1] + [synth.gradient(1010 + r, m, n, t, dtype) for t in (2, 3)]
    worst, recs = run_dion_parity(X, Gs, Q0, mu=0.95, lr=0.01, dtype=dtype, label="small")
    print(shape, dtype, worst)
    assert max(worst.values()) <= TOL[dtype], recs


def test_dion_single_256_fp32_ten_steps():
    """Single 256 x 256 fp32 weight, r = 64, 10 steps."""
    wl = synth.WORKLOADS[1]
    X = synth.weight(1, 256, 256, "f32")
    Q0 = synth.right_factor0(1, 256, 64)
    Gs = [synth.gradient(1, 256, 256, t, "f32") for t in range(1, 11)]
    worst, recs = run_dion_parity(X, Gs, Q0, wl["mu"], wl["lr"], "f32", label="cfg1")
    print(worst)
    assert max(worst.values()) <= TOL["f32"], recs


@pytest.mark.parametrize("r", [256, 1024])
def test_dion_square_4096_planted(r):
    """4096 x 4096 bf16 weight, fp32 momentum, planted rank-32 gradient, 3 steps."""
    wl = synth.WORKLOADS[2]
    X = synth.weight(2, 4096, 4096, "bf16")
    Q0 = synth.right_factor0(2, 4096, r)
    S = synth.planted(2, 4096, 4096, 32, wl["planted_ratio"])
    Gs = [synth.gradient(2, 4096, 4096, t, "bf16", planted_part=S) for t in (1, 2, 3)]
    worst, recs = run_dion_parity(X, Gs, Q0, wl["mu"], wl["lr"], "bf16", label="cfg2")
    print(r, worst)
    assert max(worst.values()) <= TOL["bf16"], recs


def test_dion_scale_and_mu_edges():
    X, G, Q0 = synth.small_case(30, 160, 120, 24, "f32")
    M = np.zeros_like(X)
    for mu, lr, scale in [(1.0, 0.01, 1.0), (0.0, 0.05, 2.5), (0.5, 0.0, 1.0)]:
        note(f"dion edges mu={mu} lr={lr} scale={scale}")
        gpu = gpu_dion_step(X, G, M, Q0, mu, lr, "f32", scale)
        ref = oracle.dion_step(X, G, M, Q0, mu, lr, scale, x_dtype="f32")
        assert rel(gpu["M"], ref["M"]) <= TOL["f32"]
        assert rel(gpu["Q"], ref["Q"]) <= TOL["f32"]
        if lr == 0.0:
            assert np.array_equal(gpu["X"], X)
        else:
            assert rel(gpu["dX"], ref["dX"]) <= TOL["f32"]


def test_dion_deterministic():
    X, G, Q0 = synth.small_case(31, 600, 500, 64, "bf16", planted_rank=4)
    M = np.zeros_like(X)
    note("dion determinism")
    a = gpu_dion_step(X, G, M, Q0, 0.95, 0.01, "bf16")
    b = gpu_dion_step(X, G, M, Q0, 0.95, 0.01, "bf16")
    for k in ("X", "M", "Q", "P", "R", "dX"):
        assert np.array_equal(a[k], b[k]), k


def test_dion_rank_deficient_flags_status():
    """B Q exactly rank deficient (two identical columns of Q, so two bitwise
    identical columns of B Q): the Cholesky pivot shift bit is set and every
    output stays finite (outside the parity contract)."""
    m, n, r = 64, 48, 8
    X, G, Q0 = synth.small_case(5, m, n, r, "f32")
    Q0 = Q0.copy()
    Q0[:, 1] = Q0[:, 0]
    note("dion rank deficient")
    gpu = gpu_dion_step(X, G, np.zeros_like(X), Q0, 0.9, 0.1, "f32")
    assert gpu["status"] != 0
    for k in ("X", "M", "Q", "P", "R"):
        assert np.all(np.isfinite(gpu[k])), k


def test_dion_zero_gradient():
    m, n, r = 64, 48, 8
    X = synth.weight(1, m, n, "bf16")
    Q0 = synth.right_factor0(1006, n, r)
    note("dion zero gradient")
    gpu = gpu_dion_step(X, np.zeros((m, n), np.float32), np.zeros((m, n), np.float32), Q0, 0.9, 0.1, "bf16")
    assert gpu["status"] & api.DEV_ZERO_COLUMN
    assert np.all(gpu["M"] == 0) and np.all(gpu["Q"] == 0)
    assert np.array_equal(gpu["X"], X.astype(np.float64))


@pytest.mark.parametrize("shape", [(384, 352, 256), (768, 1024, 512), (300, 200, 37)])
def test_dion_padded_leading_dims(shape):
    """X, G and M as column views of wider buffers (ld > cols), bf16: the step
    matches the oracle and writes nothing outside the views."""
    m, n, r = shape
    X, G, Q0 = synth.small_case(40 + r, m, n, r, "bf16", planted_rank=4)
    pad = 64
    bufs = {}
    for name, a, dt in (("X", X, "bf16"), ("G", G, "bf16"), ("M", np.zeros_like(X), "f32")):
        full = np.full((m, n + pad), 7.0, np.float32)
        full[:, :n] = a
        bufs[name] = to_dev(full, dt)
    tQ = to_dev(Q0, "f32")
    P = torch.empty(m, r, dtype=torch.float32, device="cuda")
    note(f"dion padded ld {shape}")
    api.dion_step(bufs["X"][:, :n], bufs["G"][:, :n], bufs["M"][:, :n], tQ, 0.95, 0.01, P_out=P)
    torch.cuda.synchronize()
    ref = oracle.dion_step(X, G, np.zeros_like(X), Q0, 0.95, 0.01, x_dtype="bf16")
    for name in ("X", "G", "M"):
        assert np.all(to_host(bufs[name])[:, n:] == 7.0), f"{name} written outside its view"
    assert rel(to_host(bufs["M"])[:, :n], ref["M"]) <= TOL["bf16"]
    assert rel(to_host(tQ), ref["Q"]) <= TOL["bf16"]
    assert rel(to_host(P), ref["P"]) <= TOL["bf16"]
    assert rel(to_host(bufs["X"])[:, :n], ref["X_exact"]) <= TOL["bf16"]


# ----------------------------------------------------------------------------
# Gram Newton-Schulz: bf16 products, Gram side of at most 128 rows, long side
# at least four times longer (the iteration runs on the M x M side)
# ----------------------------------------------------------------------------

GRAM_NS_CASES = [(128, 4096), (64, 512), (100, 600), (1, 50), (37, 1000), (1000, 100),
                 (512, 128), (128, 1000)]


@pytest.mark.parametrize("shape", GRAM_NS_CASES)
def test_gram_ns_matches_oracle(shape):
    m, n = shape
    _, G, _ = synth.small_case(7, m, n, 1, "bf16", x_scale=1.0)
    note(f"gram ns {shape}")
    got = gpu_ns(G, "bf16")
    assert rel(got, oracle.gram_newton_schulz(G)) <= TOL["bf16"]
    assert rel(got, oracle.newton_schulz(G)) <= TOL["bf16"]


@pytest.mark.parametrize("kind", ["rank1", "rank8", "planted"])
def test_gram_ns_low_rank_inputs(kind):
    """Rank-deficient and planted 128 x 4096 inputs (small eigen-directions of the
    Gram matrix are where the side iteration loses precision)."""
    m, n = 128, 4096
    rng = np.random.default_rng({"rank1": 1, "rank8": 8, "planted": 32}[kind])
    if kind == "planted":
        S = synth.planted(23, m, n, 32, 10.0)
        G = synth.gradient(23, m, n, 1, "bf16", planted_part=S)
    else:
        k = 1 if kind == "rank1" else 8
        G = synth.to_storage(rng.standard_normal((m, k)) @ rng.standard_normal((k, n)), "bf16")
    note(f"gram ns {kind}")
    got = gpu_ns(G, "bf16")
    err = rel(got, oracle.gram_newton_schulz(G))
    print(kind, err)
    assert err <= TOL["bf16"]


def test_gram_ns_steps_and_coefficients():
    _, G, _ = synth.small_case(8, 96, 640, 1, "bf16", x_scale=1.0)
    for steps in (1, 2, 7):
        note(f"gram ns steps={steps}")
        assert rel(gpu_ns(G, "bf16", steps=steps), oracle.gram_newton_schulz(G, steps)) <= TOL["bf16"]
    cubic = (1.5, -0.5, 0.0)
    note("gram ns cubic")
    assert rel(gpu_ns(G, "bf16", steps=8, abc=cubic),
               oracle.gram_newton_schulz(G, 8, cubic)) <= TOL["bf16"]
    note("gram ns zero input")
    assert np.all(gpu_ns(np.zeros((96, 640), np.float32), "bf16") == 0)
