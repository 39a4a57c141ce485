"""Calls from several host threads at once, each on its own stream (-m gpu).

The C ABI keeps per-device state that the first calls set up: the device check
and its compute-unit figures, the activation tables of an epilogue program
(built and waited for by the first activation call on a device), and the
no-allocation scratch address.  Those set-ups must be safe when they race, and
the kernels themselves are deterministic, so every call made from four threads
at once in a fresh process must give the same bits as the same call made again
afterwards from one thread.  The workload runs in a child interpreter so that
the threads are the first callers of every entry point.
"""
import os
import subprocess
import sys

import pytest

import linear_amd as la  # noqa: F401  (the GPU marker's library check)

pytestmark = pytest.mark.gpu

CHILD = r"""
import sys, threading
sys.path.insert(0, sys.argv[1])
import numpy as np
import torch
import linear_amd as la
from linear_amd import workloads

DEV = "cuda:0"
THREADS, ROUNDS = 4, 6
SHAPES = [(1, 1024, 768), (16, 512, 1024), (300, 520, 264), (5, 96, 40)]

def make(tid, j, M, N, K, dtype):
    x, w, b = workloads.make_inputs(M, N, K, 1.0 / np.sqrt(K), seed=1000 * tid + 10 * j + M, dtype=dtype)
    return x.to(DEV), w.to(DEV), b.to(DEV)

def calls(tid, stream):
    out = []
    for j, (M, N, K) in enumerate(SHAPES):
        x, w, b = make(tid, j, M, N, K, torch.float16)
        xb, wb, bb = make(tid, j, M, N, K, torch.bfloat16)
        out.append(la.linear_f16(x, w, b, stream=stream))
        out.append(la.linear_f16_nobias(x, w, stream=stream))
        out.append(la.linear_bf16(xb, wb, bb, stream=stream))
        out.append(la.linear_f16_epilogue(x, w, [la.EPI_BIAS, la.EPI_SILU], bias=b, stream=stream))
        out.append(la.linear_bf16_epilogue(xb, wb, [la.EPI_GELU_TANH], stream=stream))
    E, M, N, K = 4, 40, 64, 96
    xi, wi, idx = workloads.make_indexed_inputs(E, M, N, K, 0.1, seed=tid)
    out.append(la.linear_f16_indexed(xi.to(DEV), wi.to(DEV), idx.to(DEV), stream=stream))
    return out

def words(ts):
    return [t.detach().cpu().contiguous().view(torch.int16).numpy().copy() for t in ts]

results = {}
errors = []
start = threading.Barrier(THREADS)

def worker(tid):
    try:
        s = torch.cuda.Stream()
        start.wait()
        got = []
        with torch.cuda.stream(s):
            for r in range(ROUNDS):
                got.append(calls(tid, s))
        s.synchronize()
        results[tid] = [words(g) for g in got]
    except Exception as e:   # reported by the parent
        errors.append(repr(e))

ts = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
for t in ts:
    t.start()
for t in ts:
    t.join()
torch.cuda.synchronize()
assert not errors, errors
bad = 0
for tid in range(THREADS):
    ref = words(calls(tid, torch.cuda.current_stream()))
    torch.cuda.synchronize()
    for r in range(ROUNDS):
        for a, b in zip(results[tid][r], ref):
            if not np.array_equal(a, b):
                bad += 1
print("threads", THREADS, "rounds", ROUNDS, "calls per round", len(ref), "mismatches", bad, flush=True)
assert bad == 0
print("threads ok", flush=True)
"""


def test_calls_from_four_threads_on_their_own_streams_match_one_thread():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", CHILD, root], capture_output=True, text=True, timeout=300)
    print(r.stdout[-2000:])
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    assert "threads ok" in r.stdout
