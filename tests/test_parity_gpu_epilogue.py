"""Parity of the multi-step epilogue entry points against the CPU oracle (gfx950 GPU).

"The Graph IR", op table, ContractionEpilogue: the projection keeps the element
type and every step (bias, residual, multiply, the SiLU / GeLU compositions of
"Tracing a Model") rounds through it.  The epilogue is deterministic given the
rounded projection, so:

  - where the projection is unique (K = 1 and K = 8 identity weights, integer
    data) y must equal the oracle's y bit for bit; every 16-bit input word goes
    through every activation this way, on both paths;
  - for random data, y must be the oracle's epilogue of one of the projections
    the acceptance rule admits (|p - p_ref| <= ulp(p_ref) + 16 u32 A); the
    candidate projections come from the oracle's p_ref and A alone.
"""
import numpy as np
import pytest
import torch

import linear_amd as la
import oracle
from linear_amd import workloads
from oracle import tolerance

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F16, BF = torch.float16, torch.bfloat16
PATHS = [la.PATH_GEMM, la.PATH_SKINNY]
PATH_IDS = ["gemm", "skinny"]
ACTS = [la.EPI_SILU, la.EPI_GELU_TANH, la.EPI_GELU_ERF]
ACT_IDS = ["silu", "gelu_tanh", "gelu_erf"]


def elem_of(dtype):
    return tolerance.BF16 if dtype == BF else tolerance.F16


def words(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_words(w, dtype):
    return torch.from_numpy(np.ascontiguousarray(w, np.uint16).view(np.int16)).view(dtype)


def eq_words(a, b, elem):
    fa, fb = tolerance.words_to_f64(a, elem), tolerance.words_to_f64(b, elem)
    return (np.asarray(a) == np.asarray(b)) | (np.isnan(fa) & np.isnan(fb)) | ((fa == 0) & (fb == 0))


def epi(dtype, x, w, ops, bias=None, residual=None, mul=None, path=la.PATH_AUTO, out=None):
    fn = la.linear_bf16_epilogue if dtype == BF else la.linear_f16_epilogue
    d = lambda t: None if t is None else t.to(DEV)
    y = fn(x.to(DEV), w.to(DEV), ops, bias=d(bias), residual=d(residual), mul=d(mul), path=path, out=out)
    torch.cuda.synchronize()
    return y


class Candidates:
    """Element-type values in sorted order, to enumerate the projections the
    acceptance rule admits around an oracle projection."""

    def __init__(self, elem):
        w = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
        v = tolerance.words_to_f64(w, elem)
        keep = np.isfinite(v) & ~((v == 0) & (w != 0))      # one zero (+0)
        order = np.argsort(v[keep], kind="stable")
        self.vals = v[keep][order]
        self.words = w[keep][order]
        self.elem = elem

    def around(self, p_ref, A):
        p = tolerance.words_to_f64(p_ref, self.elem)
        tol = tolerance.ulp(p_ref, self.elem) + tolerance.ORDER_ALLOWANCE * tolerance.U32 * np.asarray(A)
        lo = np.searchsorted(self.vals, p - tol, "left")
        hi = np.searchsorted(self.vals, p + tol, "right")
        return lo, hi


def check_in_admitted_set(orc, y_gpu, p_ref, A, ops, elem, bias=None, res=None, mul=None):
    """y_gpu (flat words) must be the oracle epilogue of some admitted projection.
    bias / res / mul: flat per-element words (or None)."""
    cand = Candidates(elem)
    lo, hi = cand.around(p_ref, A)
    finite_ref = np.isfinite(tolerance.words_to_f64(p_ref, elem))
    # non-finite projections are unique (overflow or NaN): compare directly
    if (~finite_ref).any():
        direct = orc.epilogue(ops, p_ref[~finite_ref], bias=None if bias is None else bias[~finite_ref],
                              res=None if res is None else res[~finite_ref],
                              mul=None if mul is None else mul[~finite_ref], elem=elem)
        assert eq_words(y_gpu[~finite_ref], direct, elem).all()
    idx = np.nonzero(finite_ref)[0]
    counts = hi[idx] - lo[idx]
    assert (counts >= 1).all()
    rep = np.repeat(idx, counts)
    offs = np.concatenate([np.arange(c) for c in counts]) if idx.size else np.zeros(0, np.int64)
    cwords = cand.words[np.repeat(lo[idx], counts) + offs]
    sel = lambda a: None if a is None else a[rep]
    outs = orc.epilogue(ops, cwords, bias=sel(bias), res=sel(res), mul=sel(mul), elem=elem)
    ok = eq_words(outs, y_gpu[rep], elem)
    hit = np.zeros(y_gpu.size, bool)
    np.logical_or.at(hit, rep, ok)
    bad = idx[~hit[idx]]
    assert bad.size == 0, "%d outputs are no admitted projection's epilogue (e.g. index %s, y %s, p_ref %s)" % (
        bad.size, bad[:3], y_gpu[bad[:3]], p_ref[bad[:3]])
    return counts


# --------------------------------------------------------------------- every input word

@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("act", ACTS, ids=ACT_IDS)
def test_activation_every_input_word_k1(orc, act, path, dtype):
    """x = every 16-bit word as a [65536, 1] column, weight = [[1]]: the projection is
    x itself (K = 1, unique), so y must be the oracle's composition, bit for bit."""
    elem = elem_of(dtype)
    wds = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    x = from_words(wds.reshape(-1, 1), dtype)
    w = torch.ones(1, 1, dtype=dtype)
    y = words(epi(dtype, x, w, [act], path=path)).ravel()
    want = orc.unary(act, wds, elem)
    ok = eq_words(y, want, elem)
    assert ok.all(), "%d of 65536 words differ, e.g. %s -> %s (oracle %s)" % (
        (~ok).sum(), wds[~ok][:4], y[~ok][:4], want[~ok][:4])


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_activation_finite_words_through_the_aligned_kernels(orc, path, dtype):
    """The same for every finite word on the 16-byte (streaming) kernels: x [8192, 8]
    holds the words, weight is the 8 x 8 identity, so proj = x exactly."""
    elem = elem_of(dtype)
    wds = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    fin = wds[np.isfinite(tolerance.words_to_f64(wds, elem))]
    pad = (-fin.size) % 8
    fin = np.concatenate([fin, np.zeros(pad, np.uint16)])
    x = from_words(fin.reshape(-1, 8), dtype)
    w = torch.eye(8, dtype=dtype)
    for act in ACTS:
        y = words(epi(dtype, x, w, [la.EPI_BIAS, act], bias=torch.zeros(8, dtype=dtype), path=path)).ravel()
        want = orc.unary(act, orc.epilogue([oracle.EPI_BIAS], fin, bias=np.zeros_like(fin), elem=elem), elem)
        ok = eq_words(y, want, elem)
        assert ok.all(), (act, (~ok).sum())


# --------------------------------------------------------------------- equivalences, exact data

@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_empty_and_bias_programs_match_the_plain_calls(path, dtype):
    x, w, b = workloads.make_inputs(130, 200, 264, 0.05, seed=90, dtype=dtype)
    ex = la.linear_bf16_ex if dtype == BF else la.linear_f16_ex
    p0 = ex(x.to(DEV), w.to(DEV), None, path=path)
    y0 = ex(x.to(DEV), w.to(DEV), b.to(DEV), path=path)
    torch.cuda.synchronize()
    assert np.array_equal(words(epi(dtype, x, w, [], path=path)), words(p0))
    assert np.array_equal(words(epi(dtype, x, w, [la.EPI_BIAS], bias=b, path=path)), words(y0))


PROGRAMS = [
    [la.EPI_BIAS, la.EPI_SILU],
    [la.EPI_BIAS, la.EPI_GELU_TANH, la.EPI_RESIDUAL],
    [la.EPI_SILU, la.EPI_MUL],
    [la.EPI_BIAS, la.EPI_GELU_ERF, la.EPI_RESIDUAL, la.EPI_MUL],
    [la.EPI_RESIDUAL, la.EPI_RESIDUAL, la.EPI_BIAS, la.EPI_MUL, la.EPI_SILU, la.EPI_GELU_TANH, la.EPI_GELU_ERF,
     la.EPI_BIAS],
]
PROG_IDS = ["bias_silu", "bias_gelut_res", "silu_mul", "bias_gelue_res_mul", "eight_steps"]


def extras(M, N, dtype, seed, ints=False):
    g = torch.Generator().manual_seed(seed)
    if ints:
        r = torch.randint(-4, 5, (M, N), generator=g).to(dtype)
        u = torch.randint(-2, 3, (M, N), generator=g).to(dtype)
    else:
        r = torch.randn(M, N, generator=g).to(dtype)
        u = (torch.rand(M, N, generator=g) * 2 - 1).to(dtype)
    return r, u


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("prog", PROGRAMS, ids=PROG_IDS)
def test_programs_on_integer_data_bit_exact(orc, prog, path, dtype):
    elem = elem_of(dtype)
    M, N, K = 67, 90, 136
    x, w, b = workloads.small_integers(M, N, K, seed=91, dtype=dtype)
    r, u = extras(M, N, dtype, 92, ints=True)
    y = words(epi(dtype, x, w, prog, bias=b, residual=r, mul=u, path=path))
    _, p_ref = orc.linear(x, w, None, elem=elem)
    bb = np.broadcast_to(words(b)[None, :], (M, N))
    want = orc.epilogue(prog, p_ref, bias=bb, res=words(r), mul=words(u), elem=elem)
    ok = eq_words(y, want, elem)
    assert ok.all(), (~ok).sum()


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
def test_program_through_a_column_split_bit_exact(orc, dtype):
    """A shape that runs as two launches split by columns: the second launch reads
    bias, residual and gate at the shifted columns and writes its own."""
    elem = elem_of(dtype)
    M, N, K = 300, 34800, 72
    prog = [la.EPI_BIAS, la.EPI_GELU_ERF, la.EPI_RESIDUAL, la.EPI_MUL]
    x, w, b = workloads.small_integers(M, N, K, seed=93, dtype=dtype)
    r, u = extras(M, N, dtype, 94, ints=True)
    assert la.linear_f16_plan(x, w, b)["split_n"] > 0
    y = words(epi(dtype, x, w, prog, bias=b, residual=r, mul=u, path=la.PATH_GEMM))
    _, p_ref = orc.linear(x, w, None, elem=elem)
    bb = np.broadcast_to(words(b)[None, :], (M, N))
    want = orc.epilogue(prog, p_ref, bias=bb, res=words(r), mul=words(u), elem=elem)
    ok = eq_words(y, want, elem)
    assert ok.all(), (~ok).sum()


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_k0_program_of_the_empty_sum(orc, path, dtype):
    elem = elem_of(dtype)
    M, N = 5, 37
    x = torch.zeros(M, 0, dtype=dtype)
    w = torch.zeros(N, 0, dtype=dtype)
    b = workloads.make_inputs(1, N, 8, 1.0, seed=93, dtype=dtype)[2]
    r, u = extras(M, N, dtype, 94)
    prog = [la.EPI_BIAS, la.EPI_GELU_TANH, la.EPI_RESIDUAL, la.EPI_MUL]
    y = words(epi(dtype, x, w, prog, bias=b, residual=r, mul=u, path=path))
    want = orc.epilogue(prog, np.zeros((M, N), np.uint16), bias=np.broadcast_to(words(b)[None, :], (M, N)),
                        res=words(r), mul=words(u), elem=elem)
    assert eq_words(y, want, elem).all()


# --------------------------------------------------------------------- random data

@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("prog", PROGRAMS, ids=PROG_IDS)
@pytest.mark.parametrize("M,N,K", [(7, 1000, 520), (257, 129, 72), (200, 300, 520), (16, 4096, 4096)])
def test_programs_random_within_admitted_projections(orc, M, N, K, prog, path, dtype):
    elem = elem_of(dtype)
    x, w, b = workloads.make_inputs(M, N, K, 1.0 / np.sqrt(K), seed=M + N + K, dtype=dtype)
    r, u = extras(M, N, dtype, M * N)
    y = words(epi(dtype, x, w, prog, bias=b, residual=r, mul=u, path=path)).ravel()
    _, p_ref = orc.linear(x, w, None, elem=elem)
    _, A = orc.band(x, w, elem=elem)
    bb = np.broadcast_to(words(b)[None, :], (M, N)).ravel()
    counts = check_in_admitted_set(orc, y, p_ref.ravel(), A.ravel(), prog, elem, bias=bb,
                                   res=words(r).ravel(), mul=words(u).ravel())
    assert counts.mean() < 8


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_in_place_residual(orc, path, dtype):
    """y = gelu(x W^T + b) + y, written over the residual itself."""
    elem = elem_of(dtype)
    M, N, K = 96, 160, 264
    x, w, b = workloads.make_inputs(M, N, K, 0.06, seed=95, dtype=dtype)
    r, _ = extras(M, N, dtype, 96)
    prog = [la.EPI_BIAS, la.EPI_GELU_TANH, la.EPI_RESIDUAL]
    r_host = words(r).copy()
    buf = r.to(DEV)
    epi(dtype, x, w, prog, bias=b, residual=buf, path=path, out=buf)
    y = words(buf).ravel()
    _, p_ref = orc.linear(x, w, None, elem=elem)
    _, A = orc.band(x, w, elem=elem)
    check_in_admitted_set(orc, y, p_ref.ravel(), A.ravel(), prog, elem,
                          bias=np.broadcast_to(words(b)[None, :], (M, N)).ravel(), res=r_host.ravel())


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
def test_strided_epilogue_inputs_with_guard_band(orc, dtype):
    elem = elem_of(dtype)
    M, N, K = 67, 90, 200
    x, w, b = workloads.make_inputs(M, N, K, 0.07, seed=97, dtype=dtype)
    r, u = extras(M, N, dtype, 98)
    rs = torch.full((M, N + 13), float("nan"), dtype=dtype, device=DEV)
    rs[:, 5:5 + N] = r.to(DEV)
    us = torch.full((M, N + 3), float("nan"), dtype=dtype, device=DEV)
    us[:, :N] = u.to(DEV)
    guard = torch.full((M + 2, N + 11), 7.0, dtype=dtype, device=DEV)
    yv = guard[1:1 + M, 3:3 + N]
    prog = [la.EPI_BIAS, la.EPI_SILU, la.EPI_RESIDUAL, la.EPI_MUL]
    fn = la.linear_bf16_epilogue if dtype == BF else la.linear_f16_epilogue
    fn(x.to(DEV), w.to(DEV), prog, bias=b.to(DEV), residual=rs[:, 5:5 + N], mul=us[:, :N], out=yv)
    torch.cuda.synchronize()
    g = words(guard)
    _, p_ref = orc.linear(x, w, None, elem=elem)
    _, A = orc.band(x, w, elem=elem)
    check_in_admitted_set(orc, g[1:1 + M, 3:3 + N].ravel(), p_ref.ravel(), A.ravel(), prog, elem,
                          bias=np.broadcast_to(words(b)[None, :], (M, N)).ravel(), res=words(r).ravel(),
                          mul=words(u).ravel())
    mask = np.ones(g.shape, bool)
    mask[1:1 + M, 3:3 + N] = False
    assert (g[mask] == words(torch.tensor([7.0], dtype=dtype))[0]).all(), "wrote outside y"


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("name,prog", [("mlp_up", [la.EPI_BIAS, la.EPI_GELU_TANH]),
                                       ("down", [la.EPI_BIAS, la.EPI_RESIDUAL]),
                                       ("gemv16", [la.EPI_BIAS, la.EPI_SILU])])
def test_full_size_sampled(orc, name, prog, dtype):
    """Full-size shapes in the launch configuration the benchmark times: sampled
    outputs against the oracle's admitted set, reruns bit-identical."""
    elem = elem_of(dtype)
    x, w, b = workloads.workload_inputs(name, seed=0, dtype=dtype)
    M, N = x.shape[0], w.shape[0]
    r = (torch.randn(M, N, generator=torch.Generator().manual_seed(99)) if la.EPI_RESIDUAL in prog
         else torch.zeros(1, 1)).to(dtype)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    rd = r.to(DEV) if la.EPI_RESIDUAL in prog else None
    fn = la.linear_bf16_epilogue if dtype == BF else la.linear_f16_epilogue
    y1 = fn(xd, wd, prog, bias=bd, residual=rd)
    y2 = fn(xd, wd, prog, bias=bd, residual=rd)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "rerun not bit-identical"
    yw = words(y1)
    ms, ns = workloads.sample_points(M, N, 8192, seed=3)
    pts = orc.points(x, w, None, ms, ns, elem=elem)
    bb = words(b)[ns]
    rr = words(r)[ms, ns] if la.EPI_RESIDUAL in prog else None
    check_in_admitted_set(orc, yw[ms, ns], pts["proj"], pts["A"], prog, elem, bias=bb, res=rr)
