"""HIP-graph capture of the C-ABI calls (-m gpu).

Every entry point enqueues only kernel launches on the caller's stream (no
allocation, no memset, no host synchronisation once an activation's tables
exist), so a captured call must replay to the same bits as an eager call on the
same inputs.  Each graph is replayed several times; between replays the inputs
are rewritten in place by eager work on the capture stream and the replay's
output is compared, bit for bit, with an eager call on the new inputs.
"""
import numpy as np
import pytest
import torch

import linear_amd as la
from linear_amd import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F16, BF = torch.float16, torch.bfloat16


def words(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy()


def replay_check(call, refill, outs, eager, replays=3):
    """Capture call() on a side stream, replay it `replays` times with refill(i)
    before each replay, and compare outs() against eager() after each."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call()                                  # eager warm-up on the capture stream
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for i in range(replays):
        with torch.cuda.stream(s):
            refill(i)
            g.replay()
        s.synchronize()
        got = [words(o).copy() for o in outs()]
        ref = [words(o) for o in eager()]
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), "replay %d differs from the eager call" % i
    del g


@pytest.mark.parametrize("dtype", [F16, BF], ids=["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(16, 4096, 4096), (1, 1024, 768), (300, 520, 264), (1024, 1024, 768),
                                   (300, 34800, 72)])   # the last one runs as two launches split by columns
def test_linear_graph_replays(M, N, K, dtype):
    x, w, b = (t.to(DEV) for t in workloads.make_inputs(M, N, K, 1.0 / np.sqrt(K), seed=M, dtype=dtype))
    fn = la.linear_bf16 if dtype == BF else la.linear_f16
    fn32 = la.linear_bf16_f32out if dtype == BF else la.linear_f16_f32out
    y = torch.empty(M, N, dtype=dtype, device=DEV)
    s32 = torch.empty(M, N, dtype=torch.float32, device=DEV)
    gen = torch.Generator(device="cpu").manual_seed(5)
    fresh = [torch.randn(M, K, generator=gen).to(dtype).to(DEV) for _ in range(3)]

    def call():
        fn(x, w, b, out=y)
        fn32(x, w, out=s32)

    replay_check(call, lambda i: x.copy_(fresh[i]), lambda: (y, s32),
                 lambda: (fn(x, w, b), fn32(x, w)))


def test_epilogue_graph_replays():
    M, N, K = 512, 1024, 512
    x, w, b = (t.to(DEV) for t in workloads.make_inputs(M, N, K, 1.0 / np.sqrt(K), seed=3))
    res = torch.randn(M, N, generator=torch.Generator().manual_seed(4)).half().to(DEV)
    ops = [la.EPI_BIAS, la.EPI_GELU_TANH, la.EPI_RESIDUAL]
    y = torch.empty(M, N, dtype=F16, device=DEV)
    la.linear_f16_epilogue(x, w, ops, bias=b, residual=res)   # builds the tables outside the capture
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(6)
    fresh = [torch.randn(M, K, generator=gen).half().to(DEV) for _ in range(3)]
    replay_check(lambda: la.linear_f16_epilogue(x, w, ops, bias=b, residual=res, out=y),
                 lambda i: x.copy_(fresh[i]), lambda: (y,),
                 lambda: (la.linear_f16_epilogue(x, w, ops, bias=b, residual=res),))


def test_grouped_graph_replays():
    G, M, N, K = 4, 64, 256, 512
    x, w, b = (t.to(DEV) for t in workloads.make_inputs(G * M, G * N, K, 0.05, seed=7))
    x = x.view(G, M, K)
    y = torch.empty(G, M, N, dtype=F16, device=DEV)
    gen = torch.Generator(device="cpu").manual_seed(8)
    fresh = [torch.randn(G, M, K, generator=gen).half().to(DEV) for _ in range(3)]
    replay_check(lambda: la.linear_f16_grouped(x, w, b, out=y), lambda i: x.copy_(fresh[i]), lambda: (y,),
                 lambda: (la.linear_f16_grouped(x, w, b),))


@pytest.mark.parametrize("E,M,N,K", [(8, 32, 1024, 512), (4, 1200, 520, 264), (300, 4500, 136, 64),
                                     (8, 4096, 4096, 64)],
                         ids=["decode_self_routed", "prefill_routed", "decode_routed", "prefill_absorbing"])
def test_indexed_graph_replays(E, M, N, K):
    """The routing (in the workgroup, or the routing pass into the workspace) is
    redone on every replay: idx changes between replays.  At 4096 rows over 8
    experts and 16 column tiles the routing pass usually spreads leftover rows
    over full tiles (one round of workgroups instead of two), so the tiles of
    288 rows and fewer are rebuilt on every replay too."""
    x, w, idx = workloads.make_indexed_inputs(E, M, N, K, 0.05, seed=9)
    x, w, idx = x.to(DEV), w.to(DEV), idx.to(DEV)
    y = torch.zeros(M, N, dtype=F16, device=DEV)
    ws = torch.empty(la.indexed_workspace_bytes(E, M), dtype=torch.uint8, device=DEV)
    gen = torch.Generator(device="cpu").manual_seed(10)
    fresh = [torch.randint(0, E, (M,), generator=gen, dtype=torch.int32).to(DEV) for _ in range(3)]

    def refill(i):
        idx.copy_(fresh[i])
        y.zero_()

    def eager():
        return (la.linear_f16_indexed(x, w, idx, out=torch.zeros(M, N, dtype=F16, device=DEV)),)

    replay_check(lambda: la.linear_f16_indexed(x, w, idx, out=y, workspace=ws), refill, lambda: (y,), eager)


def test_indexed_calls_on_two_streams_with_their_own_workspaces():
    """Two indexed calls in flight at once on two streams, each with its workspace,
    equal the same calls made one after the other."""
    E, M, N, K = 8, 600, 256, 512
    xa, w, ia = workloads.make_indexed_inputs(E, M, N, K, 0.05, seed=21)
    xb, _, ib = workloads.make_indexed_inputs(E, M, N, K, 0.05, seed=22)
    xa, xb, w, ia, ib = (t.to(DEV) for t in (xa, xb, w, ia, ib))
    ref_a = la.linear_f16_indexed(xa, w, ia)
    ref_b = la.linear_f16_indexed(xb, w, ib)
    torch.cuda.synchronize()
    wsa = torch.empty(la.indexed_workspace_bytes(E, M), dtype=torch.uint8, device=DEV)
    wsb = torch.empty_like(wsa)
    ya = torch.empty(M, N, dtype=F16, device=DEV)
    yb = torch.empty(M, N, dtype=F16, device=DEV)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(4):
        la.linear_f16_indexed(xa, w, ia, out=ya, stream=sa, workspace=wsa)
        la.linear_f16_indexed(xb, w, ib, out=yb, stream=sb, workspace=wsb)
    torch.cuda.synchronize()
    assert torch.equal(ya.view(torch.int16), ref_a.view(torch.int16))
    assert torch.equal(yb.view(torch.int16), ref_b.view(torch.int16))


CAPTURE_FIRST_ACTIVATION = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
import linear_amd as la
x = torch.randn(64, 64, device="cuda").half()
w = torch.randn(64, 64, device="cuda").half()
y = torch.zeros(64, 64, device="cuda").half()
s = torch.cuda.Stream()
g = torch.cuda.CUDAGraph()
code = None
with torch.cuda.graph(g, stream=s):
    try:
        la.linear_f16_epilogue(x, w, [la.EPI_SILU], out=y)
    except la.LinearError as e:
        code = e.code
torch.cuda.synchronize()
print("capture status", code)
la.linear_f16_epilogue(x, w, [la.EPI_SILU], out=y)   # eager: builds the tables
torch.cuda.synchronize()
print("eager ok")
"""


def test_first_activation_under_capture_is_refused():
    """The first activation call on a device builds its tables and waits for
    them, which stream capture cannot hold: it returns LINEAR_E_CAPTURE and
    enqueues nothing; the same call made eagerly afterwards works."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", CAPTURE_FIRST_ACTIVATION, root], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "capture status %d" % la.LINEAR_E_CAPTURE in r.stdout, r.stdout
    assert "eager ok" in r.stdout
