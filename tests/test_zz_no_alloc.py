"""The no-allocation indexed call against the workspace call (needs a gfx950 GPU).

linear_f16_indexed_noalloc keeps its routing in the library's per-GPU scratch
array instead of a caller workspace; its results must equal those of
linear_f16_indexed bit for bit (same kernels, same per-output summation order),
on two calls in a row through the C ABI, the second smaller than the first (the
array keeps the first call's contents), and past the array's size it must refuse
the call with LINEAR_E_SCRATCH and write nothing.
"""
import numpy as np
import pytest
import torch

import linear_amd as la
from linear_amd import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def words(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# (E, M, N, K): the 256-row kernel after the routing pass, then a smaller call
# on the 16-row kernel after the routing pass (its grid is too deep for the
# self-routed form), then a small self-routed one
CASES = [(64, 8192, 512, 256), (16, 200, 4096, 128), (4, 24, 64, 96)]


def test_noalloc_equals_workspace_call_on_consecutive_calls():
    for E, M, N, K in CASES:
        print("case", (E, M, N, K), flush=True)
        x, w, idx = workloads.make_indexed_inputs(E, M, N, K, 1.0 / np.sqrt(K), seed=E + M)
        xd, wd, idd = x.to(DEV), w.to(DEV), idx.to(DEV)
        y_ws = torch.full((M, N), 7.0, dtype=torch.float16, device=DEV)
        la.linear_f16_indexed(xd, wd, idd, out=y_ws)
        y_na = torch.full((M, N), 7.0, dtype=torch.float16, device=DEV)
        la.linear_f16_indexed_noalloc(xd, wd, idd, out=y_na)
        torch.cuda.synchronize()
        a, b = words(y_ws), words(y_na)
        assert np.array_equal(a, b), "case %s: %d outputs differ" % ((E, M, N, K), int((a != b).sum()))
        # a rerun on the same array gives the same bits
        la.linear_f16_indexed_noalloc(xd, wd, idd, out=y_na)
        torch.cuda.synchronize()
        assert np.array_equal(words(y_na), a)


def test_noalloc_rows_without_an_expert_and_guard_band():
    E, M, N, K = 8, 600, 256, 64
    x, w, idx = workloads.make_indexed_inputs(E, M, N, K, 0.1, seed=5)
    idx[::7] = -1            # rows without an expert stay untouched
    idx[3::11] = E
    xd, wd, idd = x.to(DEV), w.to(DEV), idx.to(DEV)
    guard = torch.full((M + 2, N + 16), 3.0, dtype=torch.float16, device=DEV)
    ref = guard.clone()
    la.linear_f16_indexed(xd, wd, idd, out=ref[1:1 + M, 8:8 + N])
    la.linear_f16_indexed_noalloc(xd, wd, idd, out=guard[1:1 + M, 8:8 + N])
    torch.cuda.synchronize()
    assert np.array_equal(words(guard), words(ref))


def test_noalloc_refuses_calls_beyond_its_scratch():
    E, N, K = 8, 64, 16
    M = 1
    while la.indexed_workspace_bytes(E, M) <= la.NOALLOC_SCRATCH_BYTES:
        M *= 2
    x = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    w = torch.zeros((E, K, N), dtype=torch.float16, device=DEV)
    idx = torch.zeros((M,), dtype=torch.int32, device=DEV)
    y = torch.full((M, N), 5.0, dtype=torch.float16, device=DEV)
    with pytest.raises(la.LinearError) as e:
        la.linear_f16_indexed_noalloc(x, w, idx, out=y)
    assert e.value.code == la.LINEAR_E_SCRATCH
    torch.cuda.synchronize()
    assert (y == 5.0).all().item()
