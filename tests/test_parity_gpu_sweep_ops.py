"""A seeded random sweep of the epilogue-program, grouped and indexed entry points
against the CPU oracle.

"The Graph IR", op table: ContractionEpilogue (steps applied to the rounded
projection, each rounding to the element type), GroupedDenseContraction and
IndexedMatMul.  Every case draws its shape, layout (padded strides, pointers
one element off 16-byte alignment, padded outputs whose padding holds a
sentinel), element type and path from one seed.  Acceptance: an epilogue
program's output must be the oracle's program applied to one of the
projections the rule of oracle/tolerance.py admits; grouped and indexed
results follow that rule against the oracle's projection and band, their FP32
sums the FP32 bound; rows with no expert and every padding word keep the
sentinel.

The CPU test checks, through the host planner, that the epilogue cases reach
the kernels they are meant to: the 16-row weight stream, both register-staged
tiles and the streaming tiles.
"""
import numpy as np
import pytest
import torch

import linear_amd as la
from linear_amd import workloads
from oracle import tolerance

DEV = "cuda:0"
F16, BF = torch.float16, torch.bfloat16
SENTINEL16 = 0x7E5A
SENTINEL32 = 0x7FC0A5A5
SEED = 20261203
STEPS = [la.EPI_BIAS, la.EPI_RESIDUAL, la.EPI_MUL, la.EPI_SILU, la.EPI_GELU_TANH, la.EPI_GELU_ERF]


def _k8(g, K):
    """K rounded up to a multiple of 8 three times in four (16-byte rows)."""
    return (K + 7) // 8 * 8 if g.random() < 0.75 else K


def _lay(g, aligned=False):
    """(padding, offset) of a matrix: odd padding with offset 1 (misaligned) one
    time in four unless aligned, else whole 16-byte chunks."""
    r = g.random()
    if aligned:
        r = 0.25 + 0.75 * r
    if r < 0.25:
        return int(g.choice([1, 3, 9])), 1
    if r < 0.5:
        return int(g.choice([8, 24, 64])), 8
    return int(g.choice([0, 0, 8, 16])), 0


def _epi_cases():
    g = np.random.default_rng(SEED)
    draws = []
    for i in range(6):
        draws.append(("small%d" % i, int(g.integers(1, 301)), int(g.integers(1, 301)), _k8(g, int(g.integers(1, 701))), False))
    for i in range(5):
        draws.append(("skinny%d" % i, int(g.integers(1, 17)), int(g.integers(1, 2001)), _k8(g, int(g.integers(1, 2001))), False))
    for i in range(5):
        draws.append(("stream%d" % i, int(g.integers(600, 2601)), int(g.integers(600, 2601)), _k8(g, int(g.integers(1, 161))), False))
    # the 256 x 128 and 128 x 128 streaming tiles; the 128 x 128 register-staged
    # tile (x one element off alignment)
    draws += [("anchor0", 1282, 5377, 56, True), ("anchor1", 4612, 775, 56, True),
              ("anchor2", 2400, 2100, 36, "misaligned")]
    out = []
    for cid, M, N, K, aligned in draws:
        nsteps = int(g.integers(1, 9))
        ops = [int(s) for s in g.choice(STEPS, nsteps)]
        paths = [la.PATH_AUTO, la.PATH_AUTO, la.PATH_GEMM] + ([la.PATH_SKINNY] if M <= 64 else [])
        xl = (3, 1) if aligned == "misaligned" else _lay(g, aligned)
        aligned = aligned is True
        out.append(dict(id=cid, M=M, N=N, K=K, x=xl, w=_lay(g, aligned), r=_lay(g, aligned),
                        u=_lay(g, aligned), ypad=int(g.choice([0, 8, 3])), ops=ops,
                        alias=bool(g.random() < 0.25), dtype=F16 if g.random() < 0.5 else BF,
                        path=int(g.choice(paths)), seed=SEED + 131 * len(out)))
    return out


def _grouped_cases():
    g = np.random.default_rng(SEED + 1)
    out = []
    shapes = [(int(g.integers(1, 10)), int(g.integers(1, 601)), int(g.integers(1, 601)), _k8(g, int(g.integers(1, 601))))
              for _ in range(10)]
    # whole-chip tile counts: 256 x 128 and 256 x 256 tiles over the groups
    shapes += [(4, 1024, 2048, 40), (4, 2048, 2048, 24)]
    for i, (G, M, N, K) in enumerate(shapes):
        aligned = i >= 10
        paths = [la.PATH_AUTO, la.PATH_GEMM] + ([la.PATH_SKINNY] if M <= 64 else [])
        out.append(dict(id="grouped%d" % i, G=G, M=M, N=N, K=K, x=_lay(g, aligned), w=_lay(g, aligned),
                        gpad=int(g.choice([0, 1, 5])), ypad=int(g.choice([0, 8, 3])),
                        dtype=F16 if g.random() < 0.5 else BF, path=int(g.choice(paths)),
                        seed=SEED + 1 + 137 * i))
    return out


def _indexed_cases():
    g = np.random.default_rng(SEED + 2)
    shapes = [(int(g.integers(1, 41)), int(g.integers(1, 3001)), _k8(g, int(g.integers(1, 1201))),
               _k8(g, int(g.integers(1, 701)))) for _ in range(10)]
    # the 256-row routed kernel and the 16-row decode kernel, on aligned operands
    shapes += [(4, 2000, 512, 72), (8, 48, 1024, 256), (3, 900, 264, 520)]
    out = []
    for i, (E, M, N, K) in enumerate(shapes):
        aligned = i >= 10
        out.append(dict(id="indexed%d" % i, E=E, M=M, N=N, K=K, x=_lay(g, aligned), w=_lay(g, aligned),
                        epad=int(g.choice([0, 2])), ypad=int(g.choice([0, 8, 3])),
                        skew=bool(g.random() < 0.4), drop=float(g.choice([0.0, 0.0, 0.1])),
                        dtype=F16 if g.random() < 0.5 else BF, seed=SEED + 2 + 139 * i))
    return out


EPI_CASES, GROUPED_CASES, INDEXED_CASES = _epi_cases(), _grouped_cases(), _indexed_cases()


def _words(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _eq_words(a, b, elem):
    fa, fb = tolerance.words_to_f64(a, elem), tolerance.words_to_f64(b, elem)
    return (np.asarray(a) == np.asarray(b)) | (np.isnan(fa) & np.isnan(fb)) | ((fa == 0) & (fb == 0))


def _elem(dtype):
    return tolerance.BF16 if dtype == BF else tolerance.F16


def _embed(t, lay, seed):
    """t [R, C] inside a [R, C + pad] buffer of random finite words at column
    offset off; returns (buffer, view) on the CPU."""
    pad, off = lay
    off = min(off, pad)
    R, C = t.shape
    full = workloads.random_words((R, C + pad), seed=seed, dtype=t.dtype)
    full[:, off:off + C] = t
    return full, (off, C)


def _to_dev(full, where):
    off, C = where
    return full.to(DEV)[:, off:off + C]


def _sentinel(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    if dtype == torch.float32:
        t.view(torch.int32).fill_(SENTINEL32)
    else:
        t.view(torch.int16).fill_(SENTINEL16)
    return t


def _epi_inputs(c):
    x, w, b = workloads.make_inputs(c["M"], c["N"], c["K"], 1.0 / np.sqrt(c["K"]), seed=c["seed"], dtype=c["dtype"])
    gen = torch.Generator().manual_seed(c["seed"] + 5)
    r = torch.randn(c["M"], c["N"], generator=gen).to(c["dtype"])
    u = (torch.rand(c["M"], c["N"], generator=gen) * 2 - 1).to(c["dtype"])
    return x, w, b, r, u


def test_epilogue_sweep_reaches_every_gemm_kernel():
    """Host planner only: the 16-row weight stream, both register-staged tiles
    and the streaming tiles 64 x 64, 256 x 128 and 128 x 128."""
    seen = set()
    for c in EPI_CASES:
        x, w, b, _, _ = _epi_inputs(c)
        (xf, xw), (wf, ww) = _embed(x, c["x"], 1), _embed(w, c["w"], 2)
        xv, wv = xf[:, xw[0]:xw[0] + xw[1]], wf[:, ww[0]:ww[0] + ww[1]]
        p = la.linear_f16_plan(xv.view(F16), wv.view(F16), b.view(F16), path=c["path"])
        if p["path"] == la.PATH_SKINNY:
            seen.add("skinny%d" % p["tile_m"])
        else:
            seen.add("%s%dx%d" % ("stream" if p["vector_io"] else "regstaged", p["tile_m"], p["tile_n"]))
    want = {"skinny16", "regstaged64x64", "regstaged128x128", "stream64x64", "stream256x128", "stream128x128"}
    assert want <= seen, "not reached: %s" % sorted(want - seen)


@pytest.mark.gpu
@pytest.mark.parametrize("c", EPI_CASES, ids=[c["id"] for c in EPI_CASES])
def test_epilogue_sweep_case(orc, c):
    from test_parity_gpu_epilogue import check_in_admitted_set
    dtype, M, N, K, ops = c["dtype"], c["M"], c["N"], c["K"], c["ops"]
    elem = _elem(dtype)
    print("epilogue case", c["id"], (M, N, K), ops, "alias", c["alias"], dtype, "path", c["path"], flush=True)
    x, w, b, r, u = _epi_inputs(c)
    xd = _to_dev(*_embed(x, c["x"], c["seed"] + 1))
    wd = _to_dev(*_embed(w, c["w"], c["seed"] + 2))
    rd = _to_dev(*_embed(r, c["r"], c["seed"] + 3))
    ud = _to_dev(*_embed(u, c["u"], c["seed"] + 4))
    fn = la.linear_bf16_epilogue if dtype == BF else la.linear_f16_epilogue
    if c["alias"]:
        # the output is the residual itself: every element reads its residual before the store
        out, guard = rd, None
    else:
        guard = _sentinel((M, N + c["ypad"]), dtype)
        out = guard[:, :N]
    fn(xd, wd, ops, bias=b.to(DEV), residual=rd, mul=ud, out=out, path=c["path"])
    torch.cuda.synchronize()
    if guard is not None:
        assert (_words(guard)[:, N:] == SENTINEL16).all(), "output padding written"
    y = _words(out)
    _, p_ref = orc.linear(x, w, None, elem=elem)
    _, A = orc.band(x, w, elem=elem)
    bb = np.broadcast_to(_words(b)[None, :], (M, N))
    check_in_admitted_set(orc, y.ravel(), p_ref.ravel(), A.ravel(), ops, elem, bias=bb.ravel(),
                          res=_words(r).ravel(), mul=_words(u).ravel())


@pytest.mark.gpu
@pytest.mark.parametrize("c", GROUPED_CASES, ids=[c["id"] for c in GROUPED_CASES])
def test_grouped_sweep_case(orc, c):
    dtype, G, M, N, K = c["dtype"], c["G"], c["M"], c["N"], c["K"]
    elem = _elem(dtype)
    print("grouped case", c["id"], (G, M, N, K), "x", c["x"], "w", c["w"], dtype, "path", c["path"], flush=True)
    x, w, b = workloads.make_grouped_inputs(G, M, N, K, 1.0 / np.sqrt(K), seed=c["seed"], dtype=dtype)
    # x: groups gpad rows apart, rows padded and offset as the layout says
    (xpad, xoff), gp = c["x"], c["gpad"]
    xoff = min(xoff, xpad)
    xfull = workloads.random_words((G, M + gp, K + xpad), seed=c["seed"] + 1, dtype=dtype)
    xfull[:, :M, xoff:xoff + K] = x
    xd = xfull.to(DEV)[:, :M, xoff:xoff + K]
    wd = _to_dev(*_embed(w, c["w"], c["seed"] + 2))
    fy = la.linear_bf16_grouped if dtype == BF else la.linear_f16_grouped
    fs = la.linear_bf16_grouped_f32out if dtype == BF else la.linear_f16_grouped_f32out
    gy = _sentinel((G, M, N + c["ypad"]), dtype)
    gp_ = _sentinel((G, M, N + c["ypad"]), dtype)
    gs = _sentinel((G, M, N + c["ypad"]), torch.float32)
    fy(xd, wd, b.to(DEV), out=gy[:, :, :N], path=c["path"])
    fy(xd, wd, None, out=gp_[:, :, :N], path=c["path"])
    fs(xd, wd, out=gs[:, :, :N], path=c["path"])
    torch.cuda.synchronize()
    yw, pw, sw = _words(gy), _words(gp_), gs.cpu().numpy()
    assert (yw[:, :, N:] == SENTINEL16).all() and (pw[:, :, N:] == SENTINEL16).all(), "output padding written"
    assert (sw[:, :, N:].view(np.uint32) == SENTINEL32).all(), "FP32 output padding written"
    y_ref, p_ref, _ = orc.grouped(x, w, b, elem=elem)
    narrow = orc.f32_to_bf16 if dtype == BF else orc.f32_to_f16
    for gi in range(G):
        S, A = orc.band(x[gi], w[gi * N:(gi + 1) * N], elem=elem)
        p, y, s = pw[gi, :, :N], yw[gi, :, :N], np.ascontiguousarray(sw[gi, :, :N])
        ok, rep = tolerance.check_proj(p, p_ref[gi], A, elem=elem)
        assert ok.all(), (gi, rep)
        ok, rep = tolerance.check_y(y, y_ref[gi], p_ref[gi], A, elem=elem)
        assert ok.all(), (gi, rep)
        ok, rep = tolerance.check_sums(s, S, A, K)
        assert ok.all(), (gi, rep)
        assert _eq_words(narrow(s), p, elem).all(), "group %d: FP32 sums do not round to the projection" % gi
        assert tolerance.in_outer_band(p, S, A, K, elem=elem).all(), "group %d outside the outer band" % gi


def _idx(c):
    """Expert per row: uniform, or skewed (expert e drawn with weight 1 / (e + 1));
    a fraction drop of the rows gets -1 or E (no expert)."""
    g = np.random.default_rng(c["seed"] + 3)
    E, M = c["E"], c["M"]
    if c["skew"]:
        p = 1.0 / np.arange(1, E + 1)
        idx = g.choice(E, M, p=p / p.sum())
    else:
        idx = g.integers(0, E, M)
    drop = g.random(M) < c["drop"]
    idx[drop] = np.where(g.random(drop.sum()) < 0.5, -1, E)
    return torch.from_numpy(idx.astype(np.int32))


@pytest.mark.gpu
@pytest.mark.parametrize("c", INDEXED_CASES, ids=[c["id"] for c in INDEXED_CASES])
def test_indexed_sweep_case(orc, c):
    dtype, E, M, N, K = c["dtype"], c["E"], c["M"], c["N"], c["K"]
    elem = _elem(dtype)
    print("indexed case", c["id"], (E, M, N, K), "x", c["x"], "w", c["w"], "skew", c["skew"], "drop", c["drop"],
          dtype, flush=True)
    x, w, _ = workloads.make_indexed_inputs(E, M, N, K, 1.0 / np.sqrt(K), seed=c["seed"], dtype=dtype)
    idx = _idx(c)
    xd = _to_dev(*_embed(x, c["x"], c["seed"] + 1))
    # tables: k rows padded and offset as the layout says, experts epad k rows apart
    (wpad, woff), ep = c["w"], c["epad"]
    woff = min(woff, wpad)
    wfull = workloads.random_words((E, K + ep, N + wpad), seed=c["seed"] + 2, dtype=dtype)
    wfull[:, :K, woff:woff + N] = w
    wd = wfull.to(DEV)[:, :K, woff:woff + N]
    fy = la.linear_bf16_indexed if dtype == BF else la.linear_f16_indexed
    fs = la.linear_bf16_indexed_f32out if dtype == BF else la.linear_f16_indexed_f32out
    gy = _sentinel((M, N + c["ypad"]), dtype)
    gs = _sentinel((M, N + c["ypad"]), torch.float32)
    fy(xd, wd, idx.to(DEV), out=gy[:, :N])
    fs(xd, wd, idx.to(DEV), out=gs[:, :N])
    torch.cuda.synchronize()
    yw, sw = _words(gy), gs.cpu().numpy()
    valid = (idx.numpy() >= 0) & (idx.numpy() < E)
    assert (yw[:, N:] == SENTINEL16).all() and (sw[:, N:].view(np.uint32) == SENTINEL32).all(), "padding written"
    assert (yw[~valid] == SENTINEL16).all() and (sw[~valid].view(np.uint32) == SENTINEL32).all(), \
        "a row with no expert was written"
    y, s = yw[valid, :N], np.ascontiguousarray(sw[valid, :N])
    y_ref, _ = orc.indexed(x, w, idx.numpy(), elem=elem)
    S, A = orc.indexed_band(x, w, idx.numpy(), elem=elem)
    y_ref, S, A = y_ref[valid], S[valid], A[valid]
    ok, rep = tolerance.check_proj(y, y_ref, A, elem=elem)
    assert ok.all(), rep
    assert tolerance.in_outer_band(y, S, A, K, elem=elem).all(), "outside the outer band"
    ok, rep = tolerance.check_sums(s, S, A, K)
    assert ok.all(), rep
    narrow = orc.f32_to_bf16 if dtype == BF else orc.f32_to_f16
    assert _eq_words(narrow(s), y, elem).all(), "FP32 sums do not round to y"
