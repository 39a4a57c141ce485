"""The skinny path's one-row kernel (x a single row, 16-byte aligned operands: one
wave per weight row, four rows per workgroup, x staged in LDS) against the CPU
oracle, through the C ABI (gfx950 GPU).

Every output of the bias-less, the bias and the FP32-sum calls is compared, in
binary16 and bfloat16, from a single 512-wide load per row up to the largest K
the kernel stages (32768) and just past it (the 16-row kernel then runs), with N
ragged against the four rows of a workgroup.  The kernel adds its products in a
fixed order of IEEE FP32 operations (per lane, eight running sums, then a fixed
reduction over the lanes): the acceptance rule of oracle/tolerance.py for random
data, bit for bit where the sums are exact, and bit for bit against the 16-row
kernel on exact data.
"""
import numpy as np
import pytest
import torch

import linear_amd as la
from oracle import tolerance
from test_parity_gpu_variants import BF, F16, DEV, full_check, words, eq_words, f32, call_sums

pytestmark = pytest.mark.gpu


def one_row(N, K, dtype, seed, integers=False):
    g = torch.Generator().manual_seed(seed)
    if integers:
        x = torch.randint(-3, 4, (1, K), generator=g).to(dtype)
        w = torch.randint(-3, 4, (N, K), generator=g).to(dtype)
        b = torch.randint(-16, 17, (N,), generator=g).to(dtype)
    else:
        a = 1.0 / np.sqrt(max(K, 1))
        x = torch.randn(1, K, generator=g).to(dtype)
        w = ((2 * torch.rand(N, K, generator=g) - 1) * a).to(dtype)
        b = ((2 * torch.rand(N, generator=g) - 1) * a).to(dtype)
    return x, w, b


def plan(x, w, b):
    return la.linear_f16_plan(x.to(DEV).to(F16), w.to(DEV).to(F16), b.to(DEV).to(F16))


SHAPES = [(1, 8), (3, 520), (5, 1024), (4096, 512), (4097, 4096), (1000, 8200), (64, 32768), (70, 32776)]


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("N,K", SHAPES, ids=["%dx%d" % s for s in SHAPES])
def test_one_row_random(orc, N, K, dtype):
    x, w, b = one_row(N, K, dtype, seed=N * 31 + K)
    p = plan(x, w, b)
    assert p["tile_m"] == (1 if K <= 32768 else 16), p
    full_check(orc, x, w, b, la.PATH_AUTO, dtype)


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("N,K", [(4096, 4096), (130, 8200), (7, 32768)])
def test_one_row_integers_bit_exact(orc, N, K, dtype):
    x, w, b = one_row(N, K, dtype, seed=K + N, integers=True)
    full_check(orc, x, w, b, la.PATH_AUTO, dtype, exact=True)


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
def test_one_row_matches_the_sixteen_row_kernel_on_exact_data(orc, dtype):
    """An epilogue program (here the bias step alone) keeps an M = 1 call on the
    16-row MFMA kernel: on integer data both kernels give the same words."""
    x, w, b = one_row(1000, 4104, dtype, seed=7, integers=True)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    if dtype == BF:
        y1, y16 = la.linear_bf16(xd, wd, bd), la.linear_bf16_epilogue(xd, wd, [la.EPI_BIAS], bias=bd)
    else:
        y1, y16 = la.linear_f16(xd, wd, bd), la.linear_f16_epilogue(xd, wd, [la.EPI_BIAS], bias=bd)
    torch.cuda.synchronize()
    assert np.array_equal(words(y1), words(y16))


def test_one_row_deterministic_and_stream_ordered(orc):
    x, w, b = one_row(4096, 4096, F16, seed=11)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    s = torch.cuda.Stream()
    ys = []
    with torch.cuda.stream(s):
        for _ in range(3):
            ys.append(la.linear_f16(xd, wd, bd, stream=s))
    s.synchronize()
    assert all(np.array_equal(words(ys[0]), words(y)) for y in ys[1:])
    sums = [f32(call_sums(x, w, la.PATH_AUTO, F16)) for _ in range(2)]
    assert np.array_equal(sums[0].view(np.uint32), sums[1].view(np.uint32))
