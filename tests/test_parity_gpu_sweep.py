"""A seeded random sweep of the plain entry points against the CPU oracle.

Each case draws a shape from one of four ranges (small; M <= 16 weight streams;
large M and N with short K, which reaches every streaming tile and the column
split; deep K), row strides with padding, pointer offsets of one or eight
elements (one element makes the operands misaligned, so the call takes the
register-staged kernels), a padded output whose padding holds a sentinel, the
element type and the path.  Every output of the bias call, the bias-less call
and the FP32-output call is held to the acceptance rule of oracle/tolerance.py
("tensor programs, part 1", section "One Program and One Numerical Contract"),
y must be the bias epilogue of the bias-less call's projection, the FP32 sums
must round to that projection, and no padding word may change.

The GPU test runs the cases; the CPU test checks, through the host planner,
that the seeded cases reach every kernel and tile the sweep is meant to cover.
"""
import numpy as np
import pytest
import torch

import linear_amd as la
from linear_amd import workloads
from oracle import tolerance

DEV = "cuda:0"
F16, BF = torch.float16, torch.bfloat16
SENTINEL16 = 0x7E5A          # a NaN pattern no call writes
SENTINEL32 = 0x7FC0A5A5

# (range, count): M, N, K are drawn uniformly within the range; K is rounded up
# to a multiple of 8 three times in four (16-byte rows: the streaming kernels)
RANGES = {
    "small": ((1, 300), (1, 300), (1, 700)),
    "skinny": ((1, 16), (1, 3000), (1, 3000)),
    "stream": ((600, 6200), (600, 6200), (1, 160)),
    "deep": ((17, 200), (17, 400), (2000, 9000)),
}
COUNTS = {"small": 12, "skinny": 10, "stream": 8, "deep": 6}
# shapes that the host planner sends to each streaming tile and to each
# remainder tile of the column split (K ragged against the 64-wide slices)
ANCHORS = [(1282, 5377, 56), (5428, 1281, 40), (4612, 775, 56), (3848, 3851, 40), (605, 619, 40),
           (3877, 4109, 64), (3986, 5010, 16), (4002, 5914, 56), (3896, 6060, 16)]
SEED = 20261202


def _layouts(g, aligned):
    """(padding, offset) of x and weight and the output's padding.  Aligned:
    paddings of whole 16-byte chunks and offsets of 0 or 8 elements only."""
    lay = []
    for _ in range(2):                               # x, weight
        r = g.random()
        if aligned:
            r = 0.25 + 0.75 * r                      # never the odd padding
        if r < 0.25:
            lay.append((int(g.choice([1, 3, 9])), 1))          # odd padding, offset 1
        elif r < 0.5:
            lay.append((int(g.choice([8, 24, 64])), 8))        # aligned padding, offset 8
        else:
            lay.append((int(g.choice([0, 0, 8, 16])), 0))
    return lay, int(g.choice([0, 0, 8, 3]))


def _cases():
    g = np.random.default_rng(SEED)
    draws = []
    for name, count in COUNTS.items():
        (m0, m1), (n0, n1), (k0, k1) = RANGES[name]
        for i in range(count):
            M, N, K = int(g.integers(m0, m1 + 1)), int(g.integers(n0, n1 + 1)), int(g.integers(k0, k1 + 1))
            if g.random() < 0.75:
                K = (K + 7) // 8 * 8
            draws.append(("%s%d" % (name, i), M, N, K, False))
    draws += [("anchor%d" % i, M, N, K, True) for i, (M, N, K) in enumerate(ANCHORS)]
    out = []
    for cid, M, N, K, aligned in draws:
        lay, ypad = _layouts(g, aligned)
        dtype = F16 if g.random() < 0.5 else BF
        paths = [la.PATH_AUTO, la.PATH_AUTO, la.PATH_GEMM] + ([la.PATH_SKINNY] if M <= 64 else [])
        path = int(g.choice(paths))
        out.append(dict(id=cid, M=M, N=N, K=K, x=lay[0], w=lay[1], ypad=ypad, dtype=dtype, path=path,
                        seed=SEED + 97 * len(out)))
    return out


CASES = _cases()


def _embed(t, pad, off, seed):
    """t [R, C] inside a [R, C + pad] buffer of random finite words, at column off."""
    R, C = t.shape
    full = workloads.random_words((R, C + pad), seed=seed, dtype=t.dtype)
    full[:, off:off + C] = t
    return full, full[:, off:off + C]


def _words(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _eq_words(a, b, elem):
    fa, fb = tolerance.words_to_f64(a, elem), tolerance.words_to_f64(b, elem)
    return (np.asarray(a) == np.asarray(b)) | (np.isnan(fa) & np.isnan(fb)) | ((fa == 0) & (fb == 0))


def _case_inputs(c):
    x, w, b = workloads.make_inputs(c["M"], c["N"], c["K"], 1.0 / np.sqrt(c["K"]), seed=c["seed"], dtype=c["dtype"])
    (px, ox), (pw, ow) = c["x"], c["w"]
    return x, w, b, _embed(x, px, min(ox, px), c["seed"] + 1), _embed(w, pw, min(ow, pw), c["seed"] + 2)


def _plan(c):
    x, w, b, (_, xv), (_, wv) = _case_inputs(c)
    y = torch.empty((c["M"], c["N"] + c["ypad"]), dtype=c["dtype"])[:, :c["N"]]
    return la.linear_f16_plan(xv.view(F16), wv.view(F16), b.view(F16), out=y.view(F16), path=c["path"])


def test_sweep_reaches_every_kernel():
    """Host planner only: the seeded cases take the one-row and 16-row weight
    streams, both register-staged tiles, all five streaming tiles and the
    column split."""
    seen = set()
    for c in CASES:
        p = _plan(c)
        if p["path"] == la.PATH_SKINNY:
            seen.add("gemv" if p["tile_m"] == 1 else "skinny")
        elif not p["vector_io"]:
            seen.add("regstaged%dx%d" % (p["tile_m"], p["tile_n"]))
        else:
            seen.add("stream%dx%d" % (p["tile_m"], p["tile_n"]))
            if p["split_n"]:
                seen.add("split")
    want = {"gemv", "skinny", "regstaged128x128", "regstaged64x64", "stream256x256", "stream256x128",
            "stream128x256", "stream128x128", "stream64x64", "split"}
    assert want <= seen, "not reached: %s" % sorted(want - seen)


@pytest.mark.gpu
@pytest.mark.parametrize("c", CASES, ids=[c["id"] for c in CASES])
def test_sweep_case(orc, c):
    dtype, M, N, K = c["dtype"], c["M"], c["N"], c["K"]
    elem = tolerance.BF16 if dtype == BF else tolerance.F16
    x, w, b, (xf, _), (wf, _) = _case_inputs(c)
    (px, ox), (pw, ow) = c["x"], c["w"]
    ox, ow = min(ox, px), min(ow, pw)
    print("sweep case", c["id"], (M, N, K), "x", c["x"], "w", c["w"], "ypad", c["ypad"], dtype, "path", c["path"],
          flush=True)
    xd = xf.to(DEV)[:, ox:ox + K]
    wd = wf.to(DEV)[:, ow:ow + K]
    bd = b.to(DEV)
    ex = la.linear_bf16_ex if dtype == BF else la.linear_f16_ex
    f32 = la.linear_bf16_f32out if dtype == BF else la.linear_f16_f32out
    # the sentinels go in as integer words (a float round trip would lose a NaN's payload)
    yfull = torch.empty((M, N + c["ypad"]), dtype=dtype, device=DEV)
    pfull = torch.empty((M, N + c["ypad"]), dtype=dtype, device=DEV)
    sfull = torch.empty((M, N + c["ypad"]), dtype=torch.float32, device=DEV)
    yfull.view(torch.int16).fill_(SENTINEL16)
    pfull.view(torch.int16).fill_(SENTINEL16)
    sfull.view(torch.int32).fill_(SENTINEL32)
    ex(xd, wd, bd, out=yfull[:, :N], path=c["path"])
    ex(xd, wd, None, out=pfull[:, :N], path=c["path"])
    f32(xd, wd, out=sfull[:, :N], path=c["path"])
    torch.cuda.synchronize()

    yw, pw_, sw = _words(yfull), _words(pfull), sfull.cpu().numpy()
    assert (yw[:, N:] == SENTINEL16).all() and (pw_[:, N:] == SENTINEL16).all(), "output padding written"
    assert (sw[:, N:].view(np.uint32) == SENTINEL32).all(), "FP32 output padding written"
    y_gpu, p_gpu, s_gpu = yw[:, :N], pw_[:, :N], np.ascontiguousarray(sw[:, :N])

    y_ref, p_ref, _ = orc.linear(x, w, b, elem=elem, sums=True)
    bb = np.broadcast_to(_words(b)[None, :], y_ref.shape).copy()
    assert _eq_words(y_gpu, orc.bias_epilogue(p_gpu, bb, elem=elem), elem).all(), "y is not the epilogue of proj"
    narrow = orc.f32_to_bf16 if dtype == BF else orc.f32_to_f16
    assert _eq_words(narrow(s_gpu), p_gpu, elem).all(), "FP32 sums do not round to the projection"
    S, A = orc.band(x, w, elem=elem)
    ok, rep = tolerance.check_sums(s_gpu, S, A, K)
    assert ok.all(), rep
    ok, rep = tolerance.check_proj(p_gpu, p_ref, A, elem=elem)
    assert ok.all(), rep
    ok, rep = tolerance.check_y(y_gpu, y_ref, p_ref, A, elem=elem)
    assert ok.all(), rep
    assert tolerance.in_outer_band(p_gpu, S, A, K, elem=elem).all(), "outside the outer band"
