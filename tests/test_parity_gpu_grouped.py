"""Parity of the grouped and indexed contractions against the CPU oracle (gfx950 GPU).

"The Graph IR", op table: GroupedDenseContraction (a [G*N, K] weight read as G
blocks of N rows against a [G, M, K] activation) and IndexedMatMul (x [M, K]
against expert tables W [E, K, N], row m against expert idx[m]).  Acceptance as
for the layer: bit for bit on integer data (unique sums), otherwise the rule of
oracle/tolerance.py against the oracle's projection and band.
"""
import numpy as np
import pytest
import torch

import linear_amd as la
from linear_amd import workloads
from oracle import tolerance

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F16, BF = torch.float16, torch.bfloat16
PATHS = [la.PATH_GEMM, la.PATH_SKINNY]
PATH_IDS = ["gemm", "skinny"]


def elem_of(dtype):
    return tolerance.BF16 if dtype == BF else tolerance.F16


def words(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def eq_words(a, b, elem):
    fa, fb = tolerance.words_to_f64(a, elem), tolerance.words_to_f64(b, elem)
    return (np.asarray(a) == np.asarray(b)) | (np.isnan(fa) & np.isnan(fb)) | ((fa == 0) & (fb == 0))


def grouped(dtype, x, w, b, path, f32=False, out=None):
    if f32:
        fn = la.linear_bf16_grouped_f32out if dtype == BF else la.linear_f16_grouped_f32out
        y = fn(x.to(DEV), w.to(DEV), out=out, path=path)
    else:
        fn = la.linear_bf16_grouped if dtype == BF else la.linear_f16_grouped
        y = fn(x.to(DEV), w.to(DEV), None if b is None else b.to(DEV), out=out, path=path)
    torch.cuda.synchronize()
    return y


def indexed(dtype, x, w, idx, f32=False, out=None):
    if f32:
        fn = la.linear_bf16_indexed_f32out if dtype == BF else la.linear_f16_indexed_f32out
    else:
        fn = la.linear_bf16_indexed if dtype == BF else la.linear_f16_indexed
    y = fn(x.to(DEV), w.to(DEV), idx.to(DEV), out=out)
    torch.cuda.synchronize()
    return y


def ints(shape, r, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(-r, r + 1, shape, generator=g).to(dtype)


# --------------------------------------------------------------------- grouped

@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("G,M,N,K", [(3, 9, 11, 37), (4, 16, 256, 512), (2, 130, 70, 264), (5, 1, 33, 8)])
def test_grouped_integers_bit_exact(orc, G, M, N, K, path, dtype):
    elem = elem_of(dtype)
    r = 40 if dtype == F16 else 6
    x, w, b = ints((G, M, K), r, 1, dtype), ints((G * N, K), r, 2, dtype), ints((G * N,), 40, 3, dtype)
    y_ref, p_ref, s_ref = orc.grouped(x, w, b, elem=elem)
    assert eq_words(words(grouped(dtype, x, w, b, path)), y_ref, elem).all()
    assert eq_words(words(grouped(dtype, x, w, None, path)), p_ref, elem).all()
    s = grouped(dtype, x, w, None, path, f32=True).cpu().numpy()
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("G,M,N,K", [(3, 33, 65, 100), (4, 16, 512, 1024), (2, 257, 129, 72)])
def test_grouped_random_within_rule_and_each_group_is_the_plain_call(orc, G, M, N, K, path, dtype):
    elem = elem_of(dtype)
    x, w, b = workloads.make_grouped_inputs(G, M, N, K, 1.0 / np.sqrt(K), seed=G + M + N + K, dtype=dtype)
    y = words(grouped(dtype, x, w, b, path))
    p = words(grouped(dtype, x, w, None, path))
    y_ref, p_ref, _ = orc.grouped(x, w, b, elem=elem)
    ex = la.linear_bf16_ex if dtype == BF else la.linear_f16_ex
    for g in range(G):
        xs, ws, bs = x[g], w[g * N:(g + 1) * N], b[g * N:(g + 1) * N]
        S, A = orc.band(xs, ws, elem=elem)
        ok, rep = tolerance.check_proj(p[g], p_ref[g], A, elem=elem)
        assert ok.all(), (g, rep)
        ok, rep = tolerance.check_y(y[g], y_ref[g], p_ref[g], A, elem=elem)
        assert ok.all(), (g, rep)
        assert tolerance.in_outer_band(p[g], S, A, K, elem=elem).all()
        one = ex(xs.to(DEV), ws.to(DEV), bs.to(DEV), path=path)
        torch.cuda.synchronize()
        assert np.array_equal(words(one), y[g]), "group %d differs from the plain call on its slices" % g


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_grouped_strided_layout_shared_activation_and_guard_band(orc, path, dtype):
    """Padded group strides, every group reading one shared activation (sx = 0), and
    nothing written outside the groups' outputs."""
    elem = elem_of(dtype)
    G, M, N, K = 3, 20, 40, 96
    x1, w, b = workloads.make_grouped_inputs(1, M, G * N, K, 0.1, seed=7, dtype=dtype)
    xs = x1.expand(G, M, K)
    xs_dev = x1.to(DEV).expand(G, M, K)         # group stride 0: every group reads one slice
    assert xs_dev.stride(0) == 0
    guard = torch.full((G, M + 3, N + 5), 9.0, dtype=dtype, device=DEV)
    yv = guard[:, 1:1 + M, 2:2 + N]
    fn = la.linear_bf16_grouped if dtype == BF else la.linear_f16_grouped
    fn(xs_dev, w.to(DEV), b.to(DEV), out=yv, path=path)
    torch.cuda.synchronize()
    y_ref, p_ref, _ = orc.grouped(xs.contiguous(), w, b, elem=elem)
    g = words(guard)
    for gi in range(G):
        _, A = orc.band(x1[0], w[gi * N:(gi + 1) * N], elem=elem)
        ok, rep = tolerance.check_y(g[gi, 1:1 + M, 2:2 + N], y_ref[gi], p_ref[gi], A, elem=elem)
        assert ok.all(), rep
    mask = np.ones(g.shape, bool)
    mask[:, 1:1 + M, 2:2 + N] = False
    assert (g[mask] == words(torch.tensor([9.0], dtype=dtype))[0]).all(), "wrote outside the groups"


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
def test_grouped_workload_sampled(orc, dtype):
    """The grouped workload at full size (8 groups of 512 x 4096 x 4096), sampled."""
    elem = elem_of(dtype)
    wl = workloads.GROUPED["grouped"]
    x, w, b = workloads.make_grouped_inputs(wl.G, wl.M, wl.N, wl.K, wl.a, seed=0, dtype=dtype)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    fn = la.linear_bf16_grouped if dtype == BF else la.linear_f16_grouped
    y1, y2 = fn(xd, wd, bd), fn(xd, wd, bd)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    # every GEMM tile feeds each output the same k order, so a group equals the
    # plain call on its slices even where the two pick different tiles (here
    # 256 x 256 for the grouped call against 64 x 64 for one group alone)
    plain = la.linear_bf16 if dtype == BF else la.linear_f16
    plan_g = la.linear_f16_plan(xd[0], wd[:wl.N], bd[:wl.N])
    assert (plan_g["tile_m"], plan_g["tile_n"]) == (64, 64)
    for g in (0, wl.G - 1):
        yp = plain(xd[g], wd[g * wl.N:(g + 1) * wl.N], bd[g * wl.N:(g + 1) * wl.N])
        torch.cuda.synchronize()
        assert torch.equal(yp.view(torch.int16), y1[g].view(torch.int16)), g
    yw = words(y1)
    for g in (0, wl.G // 2, wl.G - 1):
        ms, ns = workloads.sample_points(wl.M, wl.N, 2048, seed=g)
        pts = orc.points(x[g], w[g * wl.N:(g + 1) * wl.N], b[g * wl.N:(g + 1) * wl.N], ms, ns, elem=elem)
        ok, rep = tolerance.check_y(yw[g][ms, ns], pts["y"], pts["proj"], pts["A"], elem=elem)
        assert ok.all(), (g, rep)


# --------------------------------------------------------------------- indexed

IDX_CASES = {
    "mixed": lambda M, E, g: torch.randint(0, E, (M,), generator=g),
    "one_expert": lambda M, E, g: torch.full((M,), E - 1),
    "own_expert": lambda M, E, g: torch.arange(M) % E,
    "some_unused": lambda M, E, g: torch.randint(0, max(1, E // 2), (M,), generator=g) * 2,
    "invalid_rows": lambda M, E, g: torch.where(torch.rand(M, generator=g) < 0.3,
                                                torch.tensor(E + 5), torch.randint(-1, E, (M,), generator=g)),
    "no_expert": lambda M, E, g: torch.full((M,), -1),      # every workgroup finds no tile
}


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("case", list(IDX_CASES))
@pytest.mark.parametrize("M,E,N,K", [
    (13, 5, 19, 29), (700, 3, 130, 72), (64, 5000, 16, 16),        # row-scan kernel: unaligned, many experts
    (40, 4, 64, 256), (32, 8, 200, 520), (50, 4096, 24, 24),         # decode tiles, routed in the workgroup
    (4500, 300, 136, 40),                                            # decode tiles after the routing pass
    (96, 3, 384, 64), (700, 3, 136, 72), (1100, 2, 264, 520),        # 256-row tiles, ragged N and K
    (200, 2, 200, 64), (1300, 3, 520, 136),                          # 256-row tiles: short last tiles
    (33, 1, 64, 64), (600, 1, 128, 128),                             # a single expert
])
def test_indexed_integers_bit_exact(orc, M, E, N, K, case, dtype):
    elem = elem_of(dtype)
    r = 30 if dtype == F16 else 6
    x, w = ints((M, K), r, M + K, dtype), ints((E, K, N), r, E + N, dtype)
    g = torch.Generator().manual_seed(M * E)
    idx = IDX_CASES[case](M, E, g).to(torch.int32)
    sentinel = torch.full((M, N), 5.0, dtype=dtype)
    out = sentinel.to(DEV)
    y = words(indexed(dtype, x, w, idx, out=out))
    y_ref, s_ref = orc.indexed(x, w, idx.numpy(), elem=elem, y_init=words(sentinel))
    ok = eq_words(y, y_ref, elem)
    assert ok.all(), (~ok).sum()
    s = indexed(dtype, x, w, idx, f32=True, out=torch.zeros(M, N, device=DEV)).cpu().numpy()
    valid = (idx.numpy() >= 0) & (idx.numpy() < E)
    assert np.array_equal(s[valid].view(np.uint32), s_ref[valid].view(np.uint32))
    assert (s[~valid] == 0).all()


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("M,E,N,K", [(32, 8, 4096, 4096), (300, 5, 200, 520), (17, 2, 70, 130)])
def test_indexed_random_within_rule(orc, M, E, N, K, dtype):
    elem = elem_of(dtype)
    x, w, idx = workloads.make_indexed_inputs(E, M, N, K, 1.0 / np.sqrt(K), seed=M + N, dtype=dtype)
    y = words(indexed(dtype, x, w, idx))
    s = indexed(dtype, x, w, idx, f32=True).cpu().numpy()
    y_ref, _ = orc.indexed(x, w, idx.numpy(), elem=elem)
    S, A = orc.indexed_band(x, w, idx.numpy(), elem=elem)
    ok, rep = tolerance.check_proj(y, y_ref, A, elem=elem)
    assert ok.all(), rep
    assert tolerance.in_outer_band(y, S, A, K, elem=elem).all()
    ok, rep = tolerance.check_sums(s, S, A, K)
    assert ok.all(), rep
    narrow = BF if dtype == BF else F16
    assert np.array_equal(words(torch.from_numpy(s).to(narrow)), y), "FP32 sums do not round to y"
    y2 = words(indexed(dtype, x, w, idx))
    assert np.array_equal(y, y2), "rerun not bit-identical"


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
def test_indexed_strided_tables_and_unaligned_x(orc, dtype):
    """Expert tables with padded k rows and padded expert stride, x rows starting
    at an odd element (the element-wise x loader), y with a padded stride."""
    elem = elem_of(dtype)
    M, E, K, N = 45, 3, 100, 50
    x, w, idx = workloads.make_indexed_inputs(E, M, N, K, 0.1, seed=11, dtype=dtype)
    wpad = torch.full((E + 1, K + 2, N + 6), float("nan"), dtype=dtype, device=DEV)
    wv = wpad[:E, 1:1 + K, 3:3 + N]
    wv.copy_(w.to(DEV))
    xpad = torch.full((M, K + 3), float("nan"), dtype=dtype, device=DEV)
    xv = xpad[:, 1:1 + K]
    xv.copy_(x.to(DEV))
    guard = torch.full((M, N + 7), 3.0, dtype=dtype, device=DEV)
    yv = guard[:, 2:2 + N]
    fn = la.linear_bf16_indexed if dtype == BF else la.linear_f16_indexed
    fn(xv, wv, idx.to(DEV), out=yv)
    torch.cuda.synchronize()
    g = words(guard)
    y_ref, _ = orc.indexed(x, w, idx.numpy(), elem=elem)
    _, A = orc.indexed_band(x, w, idx.numpy(), elem=elem)
    ok, rep = tolerance.check_proj(g[:, 2:2 + N], y_ref, A, elem=elem)
    assert ok.all(), rep
    mask = np.ones(g.shape, bool)
    mask[:, 2:2 + N] = False
    assert (g[mask] == words(torch.tensor([3.0], dtype=dtype))[0]).all()


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("f32", [False, True], ids=["rounded", "sums"])
@pytest.mark.parametrize("M,E,N,K", [(600, 3, 264, 72), (40, 4, 136, 64)], ids=["rows256", "rows16"])
def test_indexed_routed_misaligned_output_with_guard_band(orc, M, E, N, K, f32, dtype):
    """Aligned x and tables (the routed kernels) with y starting one element into
    a guard band and an odd row stride: the element-wise stores of the row-order
    epilogue, bit for bit on integer data; the band and rows without an expert
    keep their contents."""
    elem = elem_of(dtype)
    r = 30 if dtype == F16 else 6
    x, w = ints((M, K), r, M + K, dtype), ints((E, K, N), r, E + N, dtype)
    g = torch.Generator().manual_seed(M + 7)
    idx = torch.where(torch.rand(M, generator=g) < 0.1, torch.tensor(-1), torch.randint(0, E, (M,), generator=g))
    idx = idx.to(torch.int32)
    out_dtype = torch.float32 if f32 else dtype
    guard = torch.full((M, N + 13), 3.0, dtype=out_dtype, device=DEV)
    yv = guard[:, 1:1 + N]
    indexed(dtype, x, w, idx, f32=f32, out=yv)
    y_ref, s_ref = orc.indexed(x, w, idx.numpy(), elem=elem)
    valid = (idx.numpy() >= 0) & (idx.numpy() < E)
    gh = guard.cpu()
    if f32:
        got = gh[:, 1:1 + N].numpy()
        assert np.array_equal(got[valid].view(np.uint32), s_ref[valid].view(np.uint32))
        assert (got[~valid] == 3.0).all()
        band = np.ones(gh.shape, bool)
        band[:, 1:1 + N] = False
        assert (gh.numpy()[band] == 3.0).all()
    else:
        gw = words(gh)
        ok = eq_words(gw[:, 1:1 + N][valid], y_ref[valid], elem)
        assert ok.all(), (~ok).sum()
        three = words(torch.tensor([3.0], dtype=dtype))[0]
        assert (gw[:, 1:1 + N][~valid] == three).all()
        band = np.ones(gw.shape, bool)
        band[:, 1:1 + N] = False
        assert (gw[band] == three).all()


# Rows of each expert, with the row tiles the routing pass cuts them into when it
# spreads leftover rows over an expert's full tiles (up to 32 more rows each) and
# when it does not: (rows, tiles absorbing, tiles plain).
ABSORB_COUNTS = [
    (532, 2, 3),     # 512 + 20: two tiles of 266 rows
    (576, 2, 3),     # 512 + 64: two tiles of 288, the most a tile takes
    (288, 1, 2),     # 256 + 32: one tile of 288
    (289, 2, 2),     # 256 + 33: one row too many, kept as a tile of 33
    (496, 2, 2),     # 256 + 240
    (800, 3, 4),     # 768 + 32: tiles of 267, 267 and 266 rows
    (100, 1, 1),     # no full tile
    (0, 0, 0),       # an expert without rows
]
# The routed workspace: a 64-word header (word 0: the tile count), the M-word row
# list, then the tile table of {first list position, expert, rows, 0} from the
# next multiple of 4 words.
WS_HEADER_WORDS = 64


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("N", [4096, 3848, 520], ids=["absorbing", "absorbing_ragged", "plain"])
def test_indexed_absorbed_rows_bit_exact(orc, N, dtype):
    """Experts whose leftover rows the routing pass spreads over their full tiles
    (tiles of up to 288 rows: the extra 32-row block of the 256-row kernel) when
    that saves a round of workgroups on the CUs (N = 4096: 16 column tiles), and
    the same rows in tiles of at most 256 when it does not (N = 520): every output
    bit for bit on integer data, rounded and FP32 sums, rows without an expert
    untouched, and the tile table read back from the caller's workspace."""
    elem = elem_of(dtype)
    E, K = len(ABSORB_COUNTS), 72
    g = torch.Generator().manual_seed(N)
    idx = torch.cat([torch.full((c,), e) for e, (c, _, _) in enumerate(ABSORB_COUNTS)] + [torch.full((37,), -1)])
    idx = idx[torch.randperm(idx.numel(), generator=g)].to(torch.int32)
    M = idx.numel()
    r = 30 if dtype == F16 else 6
    x, w = ints((M, K), r, M + K, dtype), ints((E, K, N), r, E + N, dtype)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles_n = (N + 255) // 256

    def rounds(t):
        return (t * tiles_n + cus - 1) // cus

    t_abs = sum(a for _, a, _ in ABSORB_COUNTS)
    t_plain = sum(p for _, _, p in ABSORB_COUNTS)
    absorb = rounds(t_abs) < rounds(t_plain)
    if N >= 3848 and cus == 256:
        assert absorb, "13 tiles fit one round of 256 workgroups, 17 do not"
    ws = torch.zeros(la.indexed_workspace_bytes(E, M), dtype=torch.uint8, device=DEV)
    sentinel = torch.full((M, N), 5.0, dtype=dtype)
    fn = la.linear_bf16_indexed if dtype == BF else la.linear_f16_indexed
    y = fn(x.to(DEV), w.to(DEV), idx.to(DEV), out=sentinel.to(DEV), workspace=ws)
    torch.cuda.synchronize()
    table = ws.view(torch.int32).cpu().numpy()
    ntiles = int(table[0])
    assert ntiles == (t_abs if absorb else t_plain), (ntiles, absorb)
    t0 = (WS_HEADER_WORDS + M + 3) & ~3
    tiles = table[t0:t0 + 4 * ntiles].reshape(ntiles, 4)
    per_expert = [sorted(tiles[tiles[:, 1] == e, 2].tolist()) for e in range(E)]
    for e, (c, _, _) in enumerate(ABSORB_COUNTS):
        assert sum(per_expert[e]) == c, (e, per_expert[e])
    assert max(tiles[:, 2]) == (288 if absorb else 256)
    if absorb:
        assert per_expert[5] == [266, 267, 267] and per_expert[3] == [33, 256]
    y_ref, s_ref = orc.indexed(x, w, idx.numpy(), elem=elem, y_init=words(sentinel))
    ok = eq_words(words(y), y_ref, elem)
    assert ok.all(), (~ok).sum()
    s = (la.linear_bf16_indexed_f32out if dtype == BF else la.linear_f16_indexed_f32out)(
        x.to(DEV), w.to(DEV), idx.to(DEV), out=torch.zeros(M, N, device=DEV), workspace=ws)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    valid = (idx.numpy() >= 0) & (idx.numpy() < E)
    assert np.array_equal(s[valid].view(np.uint32), s_ref[valid].view(np.uint32))
    assert (s[~valid] == 0).all()


def test_indexed_absorbed_rows_many_experts(orc):
    """64 experts of 257 to 288 rows each at N = 4096: every expert's leftover rows
    go into its one full tile (64 row tiles, 4 rounds of workgroups on 256 CUs,
    instead of 128 tiles and 8 rounds), every tile holds between 257 and 288 rows,
    and every output matches the oracle bit for bit on integer data."""
    E, N, K = 64, 4096, 64
    g = torch.Generator().manual_seed(64)
    counts = torch.randint(257, 289, (E,), generator=g).tolist()
    idx = torch.cat([torch.full((c,), e) for e, c in enumerate(counts)])
    idx = idx[torch.randperm(idx.numel(), generator=g)].to(torch.int32)
    M = idx.numel()
    x, w = ints((M, K), 30, M + K, F16), ints((E, K, N), 30, E + N, F16)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    absorb = (E * 16 + cus - 1) // cus < (2 * E * 16 + cus - 1) // cus
    ws = torch.zeros(la.indexed_workspace_bytes(E, M), dtype=torch.uint8, device=DEV)
    y = la.linear_f16_indexed(x.to(DEV), w.to(DEV), idx.to(DEV), workspace=ws)
    torch.cuda.synchronize()
    table = ws.view(torch.int32).cpu().numpy()
    ntiles = int(table[0])
    assert ntiles == (E if absorb else 2 * E), ntiles
    if absorb:
        t0 = (WS_HEADER_WORDS + M + 3) & ~3
        tiles = table[t0:t0 + 4 * ntiles].reshape(ntiles, 4)
        assert sorted(tiles[:, 2].tolist()) == sorted(counts)
    y_ref, _ = orc.indexed(x, w, idx.numpy(), elem=tolerance.F16)
    ok = eq_words(words(y), y_ref, tolerance.F16)
    assert ok.all(), (~ok).sum()


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
def test_indexed_reused_workspace(orc, dtype):
    """One caller-owned workspace through calls of different sizes and both row
    tiles: each call rebuilds the binning it needs."""
    elem = elem_of(dtype)
    E, N, K = 4, 136, 200
    ws = torch.empty(la.indexed_workspace_bytes(E, 900), dtype=torch.uint8, device=DEV)
    ws.fill_(0xAB)
    for M, seed in ((900, 1), (40, 2), (300, 3), (7, 4)):
        x, w, idx = workloads.make_indexed_inputs(E, M, N, K, 0.1, seed=seed, dtype=dtype)
        fn = la.linear_bf16_indexed if dtype == BF else la.linear_f16_indexed
        y = words(fn(x.to(DEV), w.to(DEV), idx.to(DEV), workspace=ws))
        y_ref, _ = orc.indexed(x, w, idx.numpy(), elem=elem)
        _, A = orc.indexed_band(x, w, idx.numpy(), elem=elem)
        ok, rep = tolerance.check_proj(y, y_ref, A, elem=elem)
        assert ok.all(), (M, rep)
    with pytest.raises(ValueError):
        fn(x.to(DEV), w.to(DEV), idx.to(DEV), workspace=ws[:16])


def test_indexed_empty_cases(orc):
    x = torch.zeros(6, 0, dtype=F16)
    w = torch.zeros(3, 0, 10, dtype=F16)
    idx = torch.tensor([0, 1, 2, 2, 7, -3], dtype=torch.int32)
    out = torch.full((6, 10), 2.0, dtype=F16, device=DEV)
    y = words(indexed(F16, x, w, idx, out=out))
    assert (y[:4] == 0).all(), "K = 0: the empty sum"
    assert (y[4:] == words(torch.tensor([2.0], dtype=F16))[0]).all()
    # no experts: nothing happens
    y2 = la.linear_f16_indexed(torch.zeros(4, 8, dtype=F16, device=DEV), torch.zeros(0, 8, 4, dtype=F16, device=DEV),
                               torch.zeros(4, dtype=torch.int32, device=DEV),
                               out=torch.full((4, 4), 1.0, dtype=F16, device=DEV))
    torch.cuda.synchronize()
    assert (words(y2) == words(torch.tensor([1.0], dtype=F16))[0]).all()


@pytest.mark.parametrize("E,M,N,K", [(8, 4800, 4096, 4096), (16, 4096, 4096, 4096), (64, 8192, 2048, 2048)],
                         ids=["8x4800", "16x4096", "64x8192"])
def test_indexed_multi_round_sampled(orc, E, M, N, K):
    """Routings that need more than one round of 256-row workgroups (24, about 24
    and 64+ row tiles), walked per XCD: 48 rows (the first 8 and 40 at random)
    against the oracle over every column, within the rule."""
    x, w, idx = workloads.make_indexed_inputs(E, M, N, K, 1.0 / np.sqrt(K), seed=E + M, dtype=F16)
    y = words(indexed(F16, x, w, idx))
    rows = np.unique(np.concatenate([np.arange(8), np.random.default_rng(E).integers(0, M, 40)]))
    y_ref, _ = orc.indexed(x[rows], w, idx.numpy()[rows], elem=tolerance.F16)
    _, A = orc.indexed_band(x[rows], w, idx.numpy()[rows], elem=tolerance.F16)
    ok, rep = tolerance.check_proj(y[rows], y_ref, A, elem=tolerance.F16)
    assert ok.all(), rep


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("name", ["moe_decode", "moe_prefill"])
def test_indexed_workloads_sampled(orc, name, dtype):
    elem = elem_of(dtype)
    wl = workloads.INDEXED[name]
    x, w, idx = workloads.make_indexed_inputs(wl.E, wl.M, wl.N, wl.K, wl.a, seed=0, dtype=dtype)
    y = words(indexed(dtype, x, w, idx))
    rows = np.unique(np.concatenate([np.arange(min(wl.M, 8)), np.random.default_rng(0).integers(0, wl.M, 24)]))
    y_ref, _ = orc.indexed(x[rows], w, idx.numpy()[rows], elem=elem)
    _, A = orc.indexed_band(x[rows], w, idx.numpy()[rows], elem=elem)
    ok, rep = tolerance.check_proj(y[rows], y_ref, A, elem=elem)
    assert ok.all(), rep
