"""Every output of the full-size prefill shapes against the oracle, and every
streaming tile over every output (needs a gfx950 GPU).

The full-size shapes run in the launch configuration the benchmark times
(contiguous operands, the automatic path).  The oracle computes every output;
the comparison is strict first (|p_gpu - p_ref| <= ulp(p_ref), and for y
ulp(y_ref) + ulp(p_ref)), and only outputs outside that get band data (S, A)
from the oracle's points interface for the acceptance rule and the rigorous
outer band of oracle/tolerance.py.  Each case prints its strict-violation count,
its largest deviation in units of the reference's last place, and the oracle's
wall time on this host ("tensor programs, part 1", section "One Program and One
Numerical Contract": FP32 accumulation in any order, the projection rounded
before the bias).
"""
import time

import numpy as np
import pytest
import torch

import linear_amd as la
from linear_amd import workloads
from oracle import tolerance
from test_parity_gpu import full_check, words

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def compare_every_output(orc, name, x, w, b, p_gpu, y_gpu, elem=tolerance.F16):
    """Strict comparison of every output, band data for the rest; returns the report."""
    t0 = time.perf_counter()
    y_ref, p_ref = orc.linear(x, w, b, elem=elem)
    t_orc = time.perf_counter() - t0
    M, N = p_ref.shape
    K = x.shape[1]
    zero = np.zeros(1)
    okp, repp = tolerance.check_proj(p_gpu, p_ref, zero, elem=elem)
    oky, repy = tolerance.check_y(y_gpu, y_ref, p_ref, zero, elem=elem)
    bad = ~(okp & oky)
    ms, ns = np.nonzero(bad)
    report = {
        "case": name, "M": M, "N": N, "K": K, "outputs": int(M * N),
        "oracle_s": round(t_orc, 2), "oracle_threads": orc.max_threads(),
        "proj_strict_over_1ulp": repp["n_fail"], "proj_max_ulp": round(repp["max_ulp"], 3),
        "y_strict_over_rule_without_allowance": repy["n_fail"], "y_max_ulp": round(repy["max_ulp"], 3),
    }
    if ms.size:
        r = orc.points(x, w, b, ms, ns, elem=elem)
        pg, yg = p_gpu[ms, ns], y_gpu[ms, ns]
        assert np.array_equal(r["proj"], p_ref[ms, ns]) and np.array_equal(r["y"], y_ref[ms, ns]), \
            "points interface disagrees with the full oracle"
        okp2, repp2 = tolerance.check_proj(pg, r["proj"], r["A"], elem=elem)
        oky2, repy2 = tolerance.check_y(yg, r["y"], r["proj"], r["A"], elem=elem)
        report["rule_failures"] = int((~okp2).sum() + (~oky2).sum())
        report["strict_abs_proj_max"] = repp2.get("strict_abs_proj_max", 0.0)
        assert okp2.all(), (report, repp2)
        assert oky2.all(), (report, repy2)
        assert tolerance.in_outer_band(pg, r["S"], r["A"], K, elem=elem).all(), report
    print("every-output parity", report, flush=True)
    return report


@pytest.mark.parametrize("name", ["attn", "mlp_up", "down"])
def test_prefill_workload_every_output(orc, name):
    """attn (8192 x 4096 x 4096, 256 x 256 tiles), mlp_up (4096 x 14336 x 4096,
    256 x 256 tiles then the 256 x 128 column-split remainder) and down (2000 x
    4000 x 14336, ragged, 256 x 128 tiles): every output of the bias-less and the
    bias call, as the benchmark launches them."""
    x, w, b = workloads.workload_inputs(name, seed=0)
    print("case", name, la.linear_f16_plan(x, w, b), flush=True)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    p = la.linear_f16_nobias(xd, wd)
    y = la.linear_f16(xd, wd, bd)
    torch.cuda.synchronize()
    pw, yw = words(p), words(y)
    del p, y, xd, wd, bd
    torch.cuda.empty_cache()
    compare_every_output(orc, name, x, w, b, pw, yw)


def test_down_bf16_every_output(orc):
    """The bfloat16 form of the ragged deep-K shape, every output."""
    x, w, b = workloads.workload_inputs("down", seed=0, dtype=torch.bfloat16)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    p = la.linear_bf16_nobias(xd, wd)
    y = la.linear_bf16(xd, wd, bd)
    torch.cuda.synchronize()
    pw, yw = words(p), words(y)
    del p, y, xd, wd, bd
    torch.cuda.empty_cache()
    compare_every_output(orc, "down_bf16", x, w, b, pw, yw, elem=tolerance.BF16)


# Small-K shapes that make the tile chooser pick each streaming tile (ragged M,
# N and K where the tile allows), compared over every output: (M, N, K, tile,
# column split).
TILE_SHAPES = [
    (2000, 4000, 136, (256, 128), False),     # one wave of 256 x 128, ragged M and N
    (4096, 14336, 72, (256, 256), True),      # mlp_up's split: 256 x 256, then 256 x 128
    (3990, 1910, 40, (128, 256), False),
    (2000, 2000, 200, (128, 128), False),
    (1000, 1000, 104, (64, 64), False),
    (333, 900, 136, (64, 64), False),         # three slices, fewer than the ring's four slots
    (600, 520, 192, (64, 64), False),
    (1000, 1000, 1032, (64, 64), False),
    (77, 1100, 8, (64, 64), False),           # one K slice, most of it past K
    (8192, 4096, 24, (256, 256), False),      # attn's tile at a short K
]


@pytest.mark.parametrize("M,N,K,tile,split", TILE_SHAPES,
                         ids=["%dx%dx%d" % s[:3] for s in TILE_SHAPES])
def test_every_streaming_tile_every_output(orc, M, N, K, tile, split):
    x, w, b = workloads.make_inputs(M, N, K, 1.0 / np.sqrt(K), seed=M + N + K)
    p = la.linear_f16_plan(x, w, b)
    assert (p["tile_m"], p["tile_n"]) == tile, p
    assert (p["split_n"] > 0) == split, p
    if split:
        assert (p["tile_m2"], p["tile_n2"]) == (256, 128), p
    full_check(orc, x, w, b, la.PATH_AUTO)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
def test_moe_prefill_every_output(orc, dtype):
    """The indexed prefill (4096 rows over 8 experts of [4096, 4096], routed at
    random as the benchmark's inputs are) over every output: the rule of
    oracle/tolerance.py against the oracle's projection and band ("The Graph IR",
    op table, IndexedMatMul row).  On a 256-CU part the routing pass spreads the
    leftover rows of some experts over their full tiles here (16 row tiles rather
    than 19), so the extra-row blocks are among the outputs checked."""
    elem = tolerance.BF16 if dtype == torch.bfloat16 else tolerance.F16
    wl = workloads.INDEXED["moe_prefill"]
    x, w, idx = workloads.make_indexed_inputs(wl.E, wl.M, wl.N, wl.K, wl.a, seed=0, dtype=dtype)
    ws = torch.zeros(la.indexed_workspace_bytes(wl.E, wl.M), dtype=torch.uint8, device=DEV)
    fn = la.linear_bf16_indexed if dtype == torch.bfloat16 else la.linear_f16_indexed
    y = fn(x.to(DEV), w.to(DEV), idx.to(DEV), workspace=ws)
    torch.cuda.synchronize()
    yw = words(y)
    ntiles = int(ws.view(torch.int32)[0].item())
    del y, ws
    torch.cuda.empty_cache()
    t0 = time.perf_counter()
    y_ref, _ = orc.indexed(x, w, idx.numpy(), elem=elem)
    t_orc = time.perf_counter() - t0
    # strict first (within one unit in the last place of the oracle's projection);
    # band data (S, A) only for the rows holding outputs outside that
    okp, repp = tolerance.check_proj(yw, y_ref, np.zeros(1), elem=elem)
    rows = np.unique(np.nonzero(~okp)[0])
    report = {"case": "moe_prefill", "dtype": str(dtype), "row_tiles": ntiles, "outputs": int(yw.size),
              "proj_strict_over_1ulp": repp["n_fail"], "max_ulp": round(repp["max_ulp"], 3),
              "rows_with_band_data": int(rows.size), "oracle_s": round(t_orc, 2)}
    if rows.size:
        S, A = orc.indexed_band(x[rows], w, idx.numpy()[rows], elem=elem)
        ok, rep = tolerance.check_proj(yw[rows], y_ref[rows], A, elem=elem)
        report["rule_failures"] = int((~ok).sum())
        assert ok.all(), (report, rep)
        assert tolerance.in_outer_band(yw[rows], S, A, wl.K, elem=elem).all(), report
    print("every-output parity", report, flush=True)
