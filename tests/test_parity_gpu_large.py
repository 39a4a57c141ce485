"""Large shapes (-m gpu): grids and offsets far past the workloads' sizes.

- A vocabulary-sized projection (N = 128259, ragged, a 1 GB weight) on both
  paths: 4020 skinny workgroups, sampled outputs against the oracle.
- K = 2^20 on both paths with ternary data, whose FP32 sums are exact: bit for
  bit against the oracle (long K loops, 32-bit buffer offsets near 2^21 bytes
  per row).
- M = 65536 rows (256 GEMM row tiles through the XCD remap).
- Indexed calls with 64 and 256 experts (the 256-row kernel and the 16-row
  kernel, both after the routing pass).
"""
import numpy as np
import pytest
import torch

import linear_amd as la
from linear_amd import workloads
from oracle import tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def words(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def sampled_check(orc, x, w, b, y, count=4096, seed=0):
    ms, ns = workloads.sample_points(x.shape[0], w.shape[0], count, seed=seed)
    r = orc.points(x, w, b, ms, ns)
    ok, rep = tolerance.check_y(words(y)[ms, ns], r["y"], r["proj"], r["A"])
    assert ok.all(), rep


@pytest.fixture(scope="module")
def vocab():
    """x [300, 4096], weight [128259, 4096] (1 GB), b: drawn once for the module."""
    x, w, b = workloads.make_inputs(300, 128259, 4096, 1.0 / 64, seed=11)
    return x, w, b, w.to(DEV), b.to(DEV)


@pytest.mark.parametrize("M,path", [(1, la.PATH_AUTO), (16, la.PATH_AUTO), (300, la.PATH_AUTO),
                                    (16, la.PATH_GEMM)], ids=["m1", "m16", "m300", "m16_gemm"])
def test_vocabulary_projection_sampled(orc, vocab, M, path):
    x, w, b, wd, bd = vocab
    y = la.linear_f16_ex(x[:M].to(DEV), wd, bd, path=path)
    torch.cuda.synchronize()
    sampled_check(orc, x[:M], w, b, y, seed=M)


def ternary(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(-1, 2, shape, generator=g).half()


@pytest.mark.parametrize("path", [la.PATH_SKINNY, la.PATH_GEMM], ids=["skinny", "gemm"])
def test_long_k_ternary_bit_exact(orc, path):
    M, N, K = 16, 64, 1 << 20
    x, w = ternary((M, K), 1), ternary((N, K), 2)
    b = ternary((N,), 3)
    y = la.linear_f16_ex(x.to(DEV), w.to(DEV), b.to(DEV), path=path)
    torch.cuda.synchronize()
    y_ref, _ = orc.linear(x, w, b)
    assert np.array_equal(words(y), y_ref)


def test_many_row_tiles_sampled(orc):
    M, N, K = 65536, 256, 1024
    x, w, b = workloads.make_inputs(M, N, K, 1.0 / 32, seed=5)
    y = la.linear_f16(x.to(DEV), w.to(DEV), b.to(DEV))
    torch.cuda.synchronize()
    sampled_check(orc, x, w, b, y, count=8192, seed=2)


@pytest.mark.parametrize("E,M,N,K", [(64, 8192, 512, 1024), (256, 2048, 256, 512)],
                         ids=["64_experts_256_row_tiles", "256_experts_16_row_tiles"])
def test_many_experts_sampled(orc, E, M, N, K):
    x, w, idx = workloads.make_indexed_inputs(E, M, N, K, 1.0 / 32, seed=E)
    y = words(la.linear_f16_indexed(x.to(DEV), w.to(DEV), idx.to(DEV)))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(16), np.arange(M - 16, M),
                                     np.random.default_rng(E).integers(0, M, 48)]))
    y_ref, _ = orc.indexed(x[rows], w, idx.numpy()[rows])
    _, A = orc.indexed_band(x[rows], w, idx.numpy()[rows])
    ok, rep = tolerance.check_proj(y[rows], y_ref, A)
    assert ok.all(), rep
