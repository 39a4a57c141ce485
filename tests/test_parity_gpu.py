"""Parity of the HIP path against the CPU oracle, through the C ABI (needs a gfx950 GPU).

Floating-point cases use the acceptance rule of oracle/tolerance.py (one FP16
ulp of the reference plus the summation-order allowance 16 * 2^-24 * sum|x*w|,
inside the rigorous outer band); integer-exact, closed-form and
structure-determined cases must match bit for bit.
"""
import numpy as np
import pytest
import torch

import linear_amd as la
from linear_amd import workloads
from oracle import tolerance

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def words(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def eq_words(a, b):
    a = np.asarray(a, np.uint16)
    b = np.asarray(b, np.uint16)
    fa, fb = a.view(np.float16), b.view(np.float16)
    return (a == b) | (np.isnan(fa) & np.isnan(fb)) | ((fa == 0) & (fb == 0))


def gpu_call(x, w, b, path=la.PATH_AUTO, out=None):
    xd, wd = x.to(DEV), w.to(DEV)
    bd = None if b is None else b.to(DEV)
    y = la.linear_f16_ex(xd, wd, bd, out=out, path=path)
    torch.cuda.synchronize()
    return y


def full_check(orc, x, w, b, path, exact=False):
    """Run the bias-less and the bias call on the GPU and compare everything with the oracle."""
    p_gpu = words(gpu_call(x, w, None, path))
    y_gpu = words(gpu_call(x, w, b, path))
    y_ref, p_ref = orc.linear(x, w, b)
    # y of the bias call is the epilogue of the bias-less call's projection, bit for bit
    bb = np.broadcast_to(words(b)[None, :], y_ref.shape).copy()
    assert eq_words(y_gpu, orc.bias_epilogue(p_gpu, bb)).all(), "y is not the epilogue of proj"
    if exact:
        assert eq_words(p_gpu, p_ref).all(), "proj differs (exact case): %d" % (~eq_words(p_gpu, p_ref)).sum()
        assert eq_words(y_gpu, y_ref).all(), "y differs (exact case)"
        return
    S, A = orc.band(x, w)
    ok, rep = tolerance.check_proj(p_gpu, p_ref, A)
    assert ok.all(), rep
    ok, rep = tolerance.check_y(y_gpu, y_ref, p_ref, A)
    assert ok.all(), rep
    assert tolerance.in_outer_band(p_gpu, S, A, x.shape[1]).all(), "outside the outer band"


PATHS = [la.PATH_GEMM, la.PATH_SKINNY]
PATH_IDS = ["gemm", "skinny"]


# --------------------------------------------------------------------- exact cases

@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (5, 9, 1), (17, 23, 300), (300, 257, 1000),
                                   (16, 4096, 512), (70, 130, 8), (3, 5, 7), (129, 66, 131)])
def test_small_integers_bit_exact(orc, path, M, N, K):
    x, w, b = workloads.small_integers(M, N, K, seed=M + N + K)
    full_check(orc, x, w, b, path, exact=True)


# Shapes whose 256 x 256 tiles leave a last wave at most half full: the call runs
# as two launches split by output columns (the second with 64 x 64 tiles here).
SPLIT_SHAPES = [(200, 66000, 64), (300, 34800, 72)]


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_column_split_bit_exact(orc, M, N, K):
    x, w, b = workloads.small_integers(M, N, K, seed=M + N)
    p = la.linear_f16_plan(x, w, b)
    assert p["split_n"] > 0 and p["grid2"] > 0, p
    full_check(orc, x, w, b, la.PATH_GEMM, exact=True)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_integer_ties_and_overflow_bit_exact(orc, path):
    """Sums that are odd integers in (2048, 4096), 2 mod 4 in (4096, 8192), and past
    65520 (overflow to inf): rounding of the projection decides, then the bias."""
    rows = []
    for s in (2049, 2051, 3001, 4098, 4102, 6002, 65519, 65520, 65535, 70000, -2049, -65520):
        v = [0.0] * 128
        rest = float(s)
        for k in range(128):
            step = max(min(rest, 1024.0), -1024.0)
            v[k] = step
            rest -= step
        assert rest == 0
        rows.append(v)
    x = torch.tensor(rows, dtype=torch.float16)
    w = torch.ones(40, 128, dtype=torch.float16)
    b = torch.tensor([(-1.0) ** i * (i % 5) for i in range(40)], dtype=torch.float16)
    full_check(orc, x, w, b, path, exact=True)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_subnormal_weights_bit_exact(orc, path):
    """Binary16 subnormal weights (integers times 2^-24): every partial sum is an
    exact multiple of 2^-24, so the result is unique; a flush to zero would show."""
    g = torch.Generator().manual_seed(21)
    x = torch.randint(-3, 4, (48, 256), generator=g).to(torch.float16)
    w = (torch.randint(-1023, 1024, (80, 256), generator=g).to(torch.float32) * 2.0 ** -24).to(torch.float16)
    b = (torch.randint(-50, 51, (80,), generator=g).to(torch.float32) * 2.0 ** -24).to(torch.float16)
    full_check(orc, x, w, b, path, exact=True)
    # and subnormal x against integer weights
    xs = (torch.randint(-1023, 1024, (48, 256), generator=g).to(torch.float32) * 2.0 ** -24).to(torch.float16)
    wi = torch.randint(-3, 4, (80, 256), generator=g).to(torch.float16)
    full_check(orc, xs, wi, b, path, exact=True)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_identity_weights(orc, path):
    x = workloads.random_words((40, 96), seed=30)
    w = torch.eye(96, dtype=torch.float16)
    b = workloads.random_words((96,), seed=31)
    full_check(orc, x, w, b, path, exact=True)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_one_hot_weights(orc, path):
    g = np.random.default_rng(32)
    M, N, K = 33, 70, 50
    x = workloads.random_words((M, K), seed=33)
    pi = g.integers(0, K, N)
    e = g.integers(-4, 5, N)
    w = torch.zeros(N, K, dtype=torch.float32)
    w[torch.arange(N), torch.from_numpy(pi)] = torch.from_numpy((2.0 ** e).astype(np.float32))
    full_check(orc, x, w.to(torch.float16), torch.zeros(N, dtype=torch.float16), path, exact=True)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_k1_unique_and_k2_within_rule(orc, path):
    """K = 1 is one exact product rounded once: unique, bit-exact.  K = 2 is one
    FP32 addition, but the matrix-core step may cut the smaller product below the
    guard bit, so it is held to the acceptance rule (the K = 2 results that are
    unique on the GPU too, ties on the guard grid, are checked bit for bit with
    the FP32-output tests)."""
    x = workloads.random_words((64, 1), seed=41)
    w = workloads.random_words((96, 1), seed=51)
    b = workloads.random_words((96,), seed=61)
    full_check(orc, x, w, b, path, exact=True)
    x = (torch.randn(64, 2, generator=torch.Generator().manual_seed(7)) * 8).to(torch.float16)
    w = (torch.randn(96, 2, generator=torch.Generator().manual_seed(8)) * 8).to(torch.float16)
    b = workloads.random_words((96,), seed=62)
    full_check(orc, x, w, b, path)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_k0_is_the_empty_sum(orc, path):
    b = workloads.random_words((37,), seed=70)
    x = torch.zeros(5, 0, dtype=torch.float16)
    w = torch.zeros(37, 0, dtype=torch.float16)
    y = words(gpu_call(x, w, b, path))
    assert eq_words(y, np.broadcast_to(words(b), (5, 37))).all()
    p = words(gpu_call(x, w, None, path))
    assert (p == 0).all()


def test_nan_and_inf_propagate(orc):
    x, w, b = workloads.make_inputs(40, 48, 64, 0.1, seed=71)
    x[3, 5] = float("nan")
    w[7, 9] = float("inf")
    for path in PATHS:
        y = words(gpu_call(x, w, b, path))
        y_ref, _ = orc.linear(x, w, b)
        assert eq_words(y, y_ref)[:, 7].all() and eq_words(y, y_ref)[3].all()
        assert np.isnan(y.view(np.float16)[3]).all()


# --------------------------------------------------------------------- random data

@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (1, 4096, 4096), (16, 4096, 4096), (7, 1000, 520),
                                   (33, 65, 100), (257, 129, 72), (200, 300, 520), (512, 384, 1024),
                                   (3, 5, 7), (130, 70, 333)])
def test_random_ragged_shapes(orc, path, M, N, K):
    x, w, b = workloads.make_inputs(M, N, K, 1.0 / np.sqrt(max(K, 1)), seed=M * 7 + N * 3 + K)
    full_check(orc, x, w, b, path)


def test_toy_workload_full(orc):
    """The pages' toy layer, every output, on the path the library picks."""
    x, w, b = workloads.workload_inputs("toy", seed=0)
    full_check(orc, x, w, b, la.PATH_AUTO)


@pytest.mark.parametrize("name", ["gemv1", "gemv16"])
def test_decode_workloads_full(orc, name):
    x, w, b = workloads.workload_inputs(name, seed=0)
    full_check(orc, x, w, b, la.PATH_AUTO)


@pytest.mark.parametrize("name", ["attn", "mlp_up", "down"])
def test_prefill_workloads_sampled(orc, name):
    """Full-size prefill shapes in the launch configuration the benchmark uses:
    sampled outputs against the oracle, and properties over every output."""
    x, w, b = workloads.workload_inputs(name, seed=0)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    p = la.linear_f16_nobias(xd, wd)
    y = la.linear_f16(xd, wd, bd)
    y2 = la.linear_f16(xd, wd, bd)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "rerun not bit-identical"
    pw, yw = words(p), words(y)
    assert np.isfinite(yw.view(np.float16)).all()
    # y is the epilogue of proj everywhere
    bb = np.broadcast_to(words(b)[None, :], yw.shape).copy()
    assert eq_words(yw, orc.bias_epilogue(pw, bb)).all()
    ms, ns = workloads.sample_points(x.shape[0], w.shape[0], 16384, seed=1)
    r = orc.points(x, w, b, ms, ns)
    ok, rep = tolerance.check_proj(pw[ms, ns], r["proj"], r["A"])
    assert ok.all(), rep
    ok, rep = tolerance.check_y(yw[ms, ns], r["y"], r["proj"], r["A"])
    assert ok.all(), rep
    assert tolerance.in_outer_band(pw[ms, ns], r["S"], r["A"], x.shape[1]).all()


# --------------------------------------------------------------------- layout, guards, streams

@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_strided_and_misaligned_operands_with_guard_band(orc, path):
    M, N, K = 67, 90, 200
    x, w, b = workloads.make_inputs(M, N, K, 0.07, seed=80)
    y_ref, _ = orc.linear(x, w, b)
    # x with row stride 216 starting one element in (misaligned: element-wise loader)
    xs = torch.full((M, 217), float("nan"), dtype=torch.float16, device=DEV)
    xv = xs[:, 1:1 + K]
    xv.copy_(x.to(DEV))
    ws = torch.full((N, 208), float("nan"), dtype=torch.float16, device=DEV)
    wv = ws[:, :K]
    wv.copy_(w.to(DEV))
    guard = torch.full((M + 2, 100), 12345.0, dtype=torch.float16, device=DEV)
    yv = guard[1:1 + M, 3:3 + N]
    la.linear_f16_ex(xv, wv, b.to(DEV), out=yv, path=path)
    torch.cuda.synchronize()
    g = words(guard)
    S, A = orc.band(x, w)
    _, p_ref = orc.linear(x, w, None)
    ok, rep = tolerance.check_y(g[1:1 + M, 3:3 + N], y_ref, p_ref, A)
    assert ok.all(), rep
    sentinel = np.float16(12345.0).view(np.uint16)
    mask = np.ones(g.shape, bool)
    mask[1:1 + M, 3:3 + N] = False
    assert (g[mask] == sentinel).all(), "wrote outside y"


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_aligned_padded_strides_match_contiguous(orc, path):
    M, N, K = 100, 144, 256
    x, w, b = workloads.make_inputs(M, N, K, 0.06, seed=81)
    y0 = words(gpu_call(x, w, b, path))
    xs = torch.zeros(M, K + 64, dtype=torch.float16, device=DEV)
    xs[:, :K] = x.to(DEV)
    ws = torch.zeros(N, K + 8, dtype=torch.float16, device=DEV)
    ws[:, :K] = w.to(DEV)
    ys = torch.zeros(M, N + 4, dtype=torch.float16, device=DEV)
    la.linear_f16_ex(xs[:, :K], ws[:, :K], b.to(DEV), out=ys[:, :N], path=path)
    torch.cuda.synchronize()
    assert np.array_equal(words(ys[:, :N]), y0)


def test_nondefault_stream_and_determinism(orc):
    x, w, b = workloads.make_inputs(300, 500, 640, 0.04, seed=82)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1 = la.linear_f16(xd, wd, bd)
        y2 = la.linear_f16(xd, wd, bd, stream=s)
    s.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    y3 = la.linear_f16(xd, wd, bd)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))


def test_paths_agree_on_exact_data(orc):
    x, w, b = workloads.small_integers(40, 300, 700, seed=83)
    ya = words(gpu_call(x, w, b, la.PATH_GEMM))
    yb = words(gpu_call(x, w, b, la.PATH_SKINNY))
    assert np.array_equal(ya, yb)


def test_argument_errors_raise(orc):
    x = torch.zeros(4, 8, dtype=torch.float16, device=DEV)
    w = torch.zeros(6, 8, dtype=torch.float16, device=DEV)
    # one host tensor among device tensors is refused before any launch
    with pytest.raises(ValueError, match="on the GPU"):
        la.linear_f16(x, w, torch.zeros(6, dtype=torch.float16))
    with pytest.raises(ValueError, match="on the GPU"):
        la.linear_f16_nobias(x, w, out=torch.empty(4, 6, dtype=torch.float16))
    with pytest.raises(la.LinearArgumentError):
        la.linear_f16_ex(x, w, None, out=x[:, :6].contiguous().view(4, 6)[:, :6], path=7)
    with pytest.raises(ValueError):
        la.linear_f16(x, w[:, :7], torch.zeros(6, dtype=torch.float16, device=DEV))
