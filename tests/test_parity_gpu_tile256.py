"""The 256 x 256 streaming tile (16 x 16 x 32 MFMAs) at ragged shapes, every
output, both element types, every output mode; K = 0 on every streaming tile
and every remainder tile of the column split; NaN, infinities and overflow on the
larger tiles (needs a gfx950 GPU).

The other streaming tiles multiply with 32 x 32 x 16 MFMAs.  Both shapes feed
each output the same 16-wide k groups in the same order, so a layer gives the
same bits whichever tile computes it: here the rows of a 256 x 256-tile call are
compared with the same rows computed alone (a 64 x 64-tile call).  Against the
oracle: the acceptance rule of oracle/tolerance.py on random data, bit for bit
on integer data ("tensor programs, part 1", section "One Program and One
Numerical Contract").
"""
import numpy as np
import pytest
import torch

import linear_amd as la
from linear_amd import workloads
from oracle import tolerance
from test_parity_gpu_variants import BF, F16, DEV, full_check, words, eq_words, elem_of

pytestmark = pytest.mark.gpu

# M and N ragged against 256, K ragged against the 64-wide slices
SHAPES = [(4000, 4000, 72), (4096, 4000, 200), (3900, 4096, 8)]


def inputs(M, N, K, dtype, seed, integers=False):
    if integers:
        x, w, b = workloads.small_integers(M, N, K, seed=seed)
        return x.to(dtype), w.to(dtype), b.to(dtype)
    return workloads.make_inputs(M, N, K, 1.0 / np.sqrt(K), seed=seed, dtype=dtype)


def assert_tile(x, w, b):
    p = la.linear_f16_plan(x.to(F16), w.to(F16), b.to(F16))
    assert (p["tile_m"], p["tile_n"], p["split_n"]) == (256, 256, 0), p


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", SHAPES, ids=["%dx%dx%d" % s for s in SHAPES])
def test_tile256_random_every_output(orc, M, N, K, dtype):
    x, w, b = inputs(M, N, K, dtype, seed=M + N + K)
    assert_tile(x, w, b)
    full_check(orc, x, w, b, la.PATH_AUTO, dtype)


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
def test_tile256_integers_bit_exact(orc, dtype):
    x, w, b = inputs(4000, 4000, 72, dtype, seed=5, integers=True)
    assert_tile(x, w, b)
    full_check(orc, x, w, b, la.PATH_AUTO, dtype, exact=True)


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
def test_tile256_rows_equal_the_small_tile_call(dtype):
    """Rows 0..63 and the last 37 rows of a 256 x 256-tile call against the same
    rows computed alone (64 x 64 tiles, 32 x 32 x 16 MFMAs): the same words, with
    and without the bias, and the same FP32 sums."""
    M, N, K = 4000, 4000, 200
    x, w, b = inputs(M, N, K, dtype, seed=11)
    assert_tile(x, w, b)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    lin = la.linear_bf16 if dtype == BF else la.linear_f16
    nob = la.linear_bf16_nobias if dtype == BF else la.linear_f16_nobias
    f32 = la.linear_bf16_f32out if dtype == BF else la.linear_f16_f32out
    y, p, s = lin(xd, wd, bd), nob(xd, wd), f32(xd, wd)
    for rows in (slice(0, 64), slice(M - 37, M)):
        xs = xd[rows].contiguous()
        plan = la.linear_f16_plan(xs.to(F16), wd.to(F16), bd.to(F16))
        assert (plan["tile_m"], plan["tile_n"]) != (256, 256), plan
        ys, ps, ss = lin(xs, wd, bd), nob(xs, wd), f32(xs, wd)
        torch.cuda.synchronize()
        assert np.array_equal(words(ys), words(y[rows]))
        assert np.array_equal(words(ps), words(p[rows]))
        assert np.array_equal(ss.cpu().numpy().view(np.uint32), s[rows].cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
def test_tile256_epilogue_program_equals_the_bias_call(dtype):
    """The epilogue-program kernel of the 256 x 256 tile with the bias step alone
    gives the bias call's words; with the bias, a residual and the gate multiply
    each step is applied to the rounded value of the step before."""
    M, N, K = 4000, 4000, 72
    x, w, b = inputs(M, N, K, dtype, seed=13)
    assert_tile(x, w, b)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    g = torch.Generator().manual_seed(14)
    r = torch.randn(M, N, generator=g).to(dtype).to(DEV)
    m = torch.randn(M, N, generator=g).to(dtype).to(DEV)
    lin = la.linear_bf16 if dtype == BF else la.linear_f16
    epi = la.linear_bf16_epilogue if dtype == BF else la.linear_f16_epilogue
    y = lin(xd, wd, bd)
    e1 = epi(xd, wd, [la.EPI_BIAS], bias=bd)
    e3 = epi(xd, wd, [la.EPI_BIAS, la.EPI_RESIDUAL, la.EPI_MUL], bias=bd, residual=r, mul=m)
    torch.cuda.synchronize()
    assert np.array_equal(words(e1), words(y))
    want = ((y.float() + r.float()).to(dtype).float() * m.float()).to(dtype)
    assert eq_words(words(e3), words(want), elem_of(dtype)).all()


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
def test_tile256_k0_is_the_empty_sum(dtype):
    """K = 0 at a shape that takes the 256 x 256 tile: no K slice runs, the sums
    are +0, the projection is +0 and y is the bias ("tensor programs, part 1",
    the layer's definition with an empty sum)."""
    M, N = 4096, 4096
    # zero-width views of 8-column matrices: row strides of 8 elements, so the
    # call takes the 16-byte streaming kernels (a bare [M, 0] tensor would not)
    x = torch.zeros(M, 8, dtype=dtype)[:, :0]
    w = torch.zeros(N, 8, dtype=dtype)[:, :0]
    b = workloads.make_inputs(1, N, 8, 0.5, seed=21, dtype=dtype)[2]
    assert_tile(x, w, b)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    lin = la.linear_bf16 if dtype == BF else la.linear_f16
    nob = la.linear_bf16_nobias if dtype == BF else la.linear_f16_nobias
    f32 = la.linear_bf16_f32out if dtype == BF else la.linear_f16_f32out
    epi = la.linear_bf16_epilogue if dtype == BF else la.linear_f16_epilogue
    y, p, s, e = lin(xd, wd, bd), nob(xd, wd), f32(xd, wd), epi(xd, wd, [la.EPI_BIAS], bias=bd)
    torch.cuda.synchronize()
    want = np.broadcast_to(words(b)[None, :], (M, N))
    assert eq_words(words(y), want, elem_of(dtype)).all()
    assert eq_words(words(e), want, elem_of(dtype)).all()
    assert (words(p) == 0).all()
    assert (s.cpu().numpy().view(np.uint32) == 0).all()


# shapes the host planner sends to each streaming tile and each remainder tile of
# the column split: (M, N, tile, split remainder tile or None)
K0_SHAPES = [(1282, 5377, (256, 128), None), (5428, 1281, (128, 256), None), (4612, 775, (128, 128), None),
             (605, 619, (64, 64), None), (3877, 4109, (256, 256), (64, 64)), (3986, 5010, (256, 256), (128, 128)),
             (4002, 5914, (256, 256), (128, 256)), (3896, 6060, (256, 256), (256, 128))]


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("M,N,tile,rest", K0_SHAPES, ids=["%dx%d" % s[:2] for s in K0_SHAPES])
def test_every_streaming_tile_k0_is_the_empty_sum(M, N, tile, rest, dtype):
    """K = 0 on each streaming tile: every output of the bias call and of the
    one-step bias program is the bias word, the projection and the FP32 sums +0
    (the layer's definition with an empty sum)."""
    x = torch.zeros(M, 8, dtype=dtype)[:, :0]
    w = torch.zeros(N, 8, dtype=dtype)[:, :0]
    b = workloads.make_inputs(1, N, 8, 0.5, seed=M + N, dtype=dtype)[2]
    p = la.linear_f16_plan(x.view(F16), w.view(F16), b.view(F16))
    assert (p["tile_m"], p["tile_n"]) == tile, p
    assert ((p["tile_m2"], p["tile_n2"]) if p["split_n"] else None) == rest, p
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    lin = la.linear_bf16 if dtype == BF else la.linear_f16
    nob = la.linear_bf16_nobias if dtype == BF else la.linear_f16_nobias
    f32 = la.linear_bf16_f32out if dtype == BF else la.linear_f16_f32out
    epi = la.linear_bf16_epilogue if dtype == BF else la.linear_f16_epilogue
    y, pr, s, e = lin(xd, wd, bd), nob(xd, wd), f32(xd, wd), epi(xd, wd, [la.EPI_BIAS], bias=bd)
    torch.cuda.synchronize()
    want = np.broadcast_to(words(b)[None, :], (M, N))
    assert eq_words(words(y), want, elem_of(dtype)).all()
    assert eq_words(words(e), want, elem_of(dtype)).all()
    assert (words(pr) == 0).all()
    assert (s.cpu().numpy().view(np.uint32) == 0).all()


SPECIAL_SHAPES = [(1282, 5377), (5428, 1281), (4612, 775), (4002, 5914)]


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("M,N", SPECIAL_SHAPES, ids=["%dx%d" % s for s in SPECIAL_SHAPES])
def test_specials_on_the_large_tiles(orc, M, N, dtype):
    """A NaN in x row 5 makes row 5 NaN; +inf in weight row 7 (against x values
    of 1) makes column 7 +inf; +inf and -inf in weight row 9 make column 9 NaN;
    x row 11 times a column of 4s at 60000 overflows binary16 (not bfloat16).
    The special class of every output equals the oracle's, and every finite
    output satisfies the acceptance rule ("tensor programs, part 1", section
    "One Program and One Numerical Contract": IEEE arithmetic throughout)."""
    K = 72
    elem = elem_of(dtype)
    x, w, b = inputs(M, N, K, dtype, seed=M + 3 * N)
    x[:, 10] = 1.0
    x[:, 20] = 1.0
    x[:, 21] = 1.0
    x[5, 3] = float("nan")
    w[7, 10] = float("inf")
    w[9, 20] = float("inf")
    w[9, 21] = float("-inf")
    x[11, 30] = 60000.0
    w[:, 30] = 4.0
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    lin = la.linear_bf16 if dtype == BF else la.linear_f16
    nob = la.linear_bf16_nobias if dtype == BF else la.linear_f16_nobias
    y, p = words(lin(xd, wd, bd)), words(nob(xd, wd))
    torch.cuda.synchronize()
    y_ref, p_ref = orc.linear(x, w, b, elem=elem)
    for got, ref in ((p, p_ref), (y, y_ref)):
        g, r = tolerance.words_to_f64(got, elem), tolerance.words_to_f64(ref, elem)
        assert np.array_equal(np.isnan(g), np.isnan(r)), "NaN outputs differ"
        assert np.array_equal(np.isposinf(g), np.isposinf(r)) and np.array_equal(np.isneginf(g), np.isneginf(r))
    r = tolerance.words_to_f64(p_ref, elem)
    assert np.isnan(r[5]).all() and np.isnan(r[:, 9]).all() and np.isposinf(r[np.arange(M) != 5, 7]).all()
    rest = np.ones(N, bool)
    rest[[7, 9]] = False
    # row 11 sums to about 240000: past binary16's range, inside bfloat16's
    assert (np.isposinf(r[11, rest]) if dtype == F16 else np.isfinite(r[11, rest])).all()
    fin = np.isfinite(r)
    _, A = orc.band(x, w, elem=elem)
    ok, rep = tolerance.check_proj(p[fin], p_ref[fin], A[fin], elem=elem)
    assert ok.all(), rep
    fy = fin & np.isfinite(tolerance.words_to_f64(y_ref, elem))
    ok, rep = tolerance.check_y(y[fy], y_ref[fy], p_ref[fy], A[fy], elem=elem)
    assert ok.all(), rep
