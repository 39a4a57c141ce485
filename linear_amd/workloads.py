"""Seeded synthetic inputs for the FP16 linear layer.

This module only draws random numbers and lays out tensors; it holds none of
the layer's arithmetic, so both the HIP path's tests and the CPU oracle's tests
take their inputs from here.

Recipe (one ``torch.Generator('cpu')`` per workload, seeded; draws in the order
x, weight, b, each drawn in float32 and converted to float16 with torch's
round-to-nearest-even conversion):

    x      ~ N(0, 1)                     shape [M, K]
    weight ~ U(-a, a) = (2u - 1) * a      shape [N, K]   ([out_features, in_features])
    b      ~ U(-a, a)                     shape [N]

The toy workload's shapes are the ones of "tensor programs, part 1" (the
PyTorch line that builds x [1024, 768], weight [1024, 768], b [1024]); its bound
a = 1/sqrt(768) is nn.Linear's default initialisation bound for 768 input
features (the page names nn.Linear(768, 1024)).  The other workloads are
decode- and prefill-shaped projections of a 4096-wide model.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    a: float          # half-width of the uniform law of weight and b
    note: str = ""

    @property
    def flops(self) -> int:
        """Algorithmic FLOPs of the contraction: one multiply and one add per (m, n, k)."""
        return 2 * self.M * self.N * self.K

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: x, weight and b read once, y written once (2 B each)."""
        return 2 * (self.M * self.K + self.N * self.K + self.N + self.M * self.N)


WORKLOADS = {
    "toy": Workload("toy", 1024, 1024, 768, 1.0 / math.sqrt(768.0),
                    "toy linear of the pages: x[1024,768] @ weight[1024,768].T + b[1024]"),
    "gemv1": Workload("gemv1", 1, 4096, 4096, 1.0 / 64.0, "decode GEMV, one row"),
    "gemv16": Workload("gemv16", 16, 4096, 4096, 1.0 / 64.0, "decode GEMV batch, 16 rows"),
    "attn": Workload("attn", 8192, 4096, 4096, 1.0 / 64.0, "prefill attention projection"),
    "mlp_up": Workload("mlp_up", 4096, 14336, 4096, 1.0 / 64.0, "prefill MLP up-projection"),
    "down": Workload("down", 2000, 4000, 14336, 1.0 / math.sqrt(14336.0),
                     "deep-K down-projection, M and N not multiples of a tile"),
}

# Grouped and indexed contractions ("The Graph IR", op table: GroupedDenseContraction,
# IndexedMatMul).  The pages give no shapes; these are a grouped projection of the
# same 4096-wide model and mixture-of-experts feed-forward shapes (8 experts,
# top-2 routing: 16 decode tokens -> 32 rows, 2048 prefill tokens -> 4096 rows).
@dataclass(frozen=True)
class GroupedWorkload:
    name: str
    G: int
    M: int
    N: int
    K: int
    a: float

    @property
    def flops(self) -> int:
        return 2 * self.G * self.M * self.N * self.K

    @property
    def bytes(self) -> int:
        return 2 * (self.G * self.M * self.K + self.G * self.N * self.K + self.G * self.N + self.G * self.M * self.N)


@dataclass(frozen=True)
class IndexedWorkload:
    name: str
    E: int
    M: int
    N: int
    K: int
    a: float

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


GROUPED = {"grouped": GroupedWorkload("grouped", 8, 512, 4096, 4096, 1.0 / 64.0)}
INDEXED = {
    "moe_decode": IndexedWorkload("moe_decode", 8, 32, 4096, 4096, 1.0 / 64.0),
    "moe_prefill": IndexedWorkload("moe_prefill", 8, 4096, 4096, 4096, 1.0 / 64.0),
}


def make_grouped_inputs(G: int, M: int, N: int, K: int, a: float, seed: int = 0, device: str = "cpu",
                        dtype: torch.dtype = torch.float16):
    """x [G, M, K] ~ N(0,1), weight [G*N, K] and b [G*N] ~ U(-a, a), drawn in that order."""
    x, w, b = make_inputs(G * M, G * N, K, a, seed=seed, device=device, dtype=dtype)
    return x.reshape(G, M, K), w, b


def make_indexed_inputs(E: int, M: int, N: int, K: int, a: float, seed: int = 0, device: str = "cpu",
                        dtype: torch.dtype = torch.float16):
    """x [M, K] ~ N(0,1), expert tables w [E, K, N] ~ U(-a, a), idx [M] uniform over the
    experts (int32), drawn in that order."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn((M, K), generator=g, dtype=torch.float32)
    w = torch.rand((E, K, N), generator=g, dtype=torch.float32).mul_(2.0).sub_(1.0).mul_(a)
    idx = torch.randint(0, max(E, 1), (M,), generator=g, dtype=torch.int64).to(torch.int32)
    x, w = x.to(dtype), w.to(dtype)
    if device != "cpu":
        x, w, idx = x.to(device), w.to(device), idx.to(device)
    return x, w, idx


# The decode batch: one step runs both decode shapes over the same weight size.
DECODE_STEP = ("gemv1", "gemv16")


def make_inputs(M: int, N: int, K: int, a: float, seed: int = 0, device: str = "cpu",
                dtype: torch.dtype = torch.float16):
    """Draw (x, weight, b) as contiguous float16 (or bfloat16) tensors, following the
    recipe above; the float32 draws are the same for both element types."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn((M, K), generator=g, dtype=torch.float32)
    w = torch.rand((N, K), generator=g, dtype=torch.float32).mul_(2.0).sub_(1.0).mul_(a)
    b = torch.rand((N,), generator=g, dtype=torch.float32).mul_(2.0).sub_(1.0).mul_(a)
    x16, w16, b16 = x.to(dtype), w.to(dtype), b.to(dtype)
    if device != "cpu":
        x16, w16, b16 = x16.to(device), w16.to(device), b16.to(device)
    return x16, w16, b16


def workload_inputs(name: str, seed: int = 0, device: str = "cpu", dtype: torch.dtype = torch.float16):
    wl = WORKLOADS[name]
    return make_inputs(wl.M, wl.N, wl.K, wl.a, seed=seed, device=device, dtype=dtype)


def small_integers(M: int, N: int, K: int, seed: int = 0, lo: int = -3, hi: int = 3,
                   blo: int = -8, bhi: int = 8, dtype: torch.dtype = torch.float16):
    """Integer-valued float16 (or bfloat16) tensors: x, weight in [lo, hi], b in [blo, bhi].

    With sum |x*w| < 2^24 every partial sum in every order is an exact FP32
    integer, so the result is unique whatever the summation order."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randint(lo, hi + 1, (M, K), generator=g).to(dtype)
    w = torch.randint(lo, hi + 1, (N, K), generator=g).to(dtype)
    b = torch.randint(blo, bhi + 1, (N,), generator=g).to(dtype)
    return x, w, b


def random_words(shape, seed: int = 0, finite: bool = True, dtype: torch.dtype = torch.float16):
    """Uniformly random 16-bit patterns (optionally finite only) as float16 or bfloat16."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    words = torch.randint(0, 1 << 16, shape, generator=g, dtype=torch.int32)
    if finite:
        # the all-ones exponent field is inf/NaN: clear its top bit
        # (binary16: field 31 -> 15; bfloat16: field 255 -> 127)
        emask, top = (0x7F80, 0x4000) if dtype == torch.bfloat16 else (0x7C00, 0x4000)
        eall = (words & emask) == emask
        words = torch.where(eall, words & ~top, words)
    return words.to(torch.int16).view(dtype)


def sample_points(M: int, N: int, count: int, seed: int = 0):
    """Output coordinates for full-size spot checks: the four corners, the last
    row and column (ragged edges), and uniform random (m, n) pairs."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 7919)
    ms = torch.randint(0, M, (count,), generator=g)
    ns = torch.randint(0, N, (count,), generator=g)
    edge_m = torch.tensor([0, 0, M - 1, M - 1] + [M - 1] * 64 + list(range(min(M, 64))))
    edge_n = torch.tensor([0, N - 1, 0, N - 1] + torch.randint(0, N, (64,), generator=g).tolist()
                          + [N - 1] * min(M, 64))
    return torch.cat([edge_m, ms]).numpy(), torch.cat([edge_n, ns]).numpy()
