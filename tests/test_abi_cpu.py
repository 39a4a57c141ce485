"""The C ABI without a GPU: exported symbols, host-side validation, plans."""
import ctypes
import os
import re
import subprocess

import pytest
import torch  # noqa: F401  (load torch's HIP runtime before the library)

import linear_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linear_amd.h")

needs_lib = pytest.mark.skipif(not os.path.exists(la.LIB_PATH), reason="liblinear_amd.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(linear_[a-z0-9_]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert set(declared_functions()) == set(la.ENTRY_POINTS)


@needs_lib
def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", la.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(la._lib(), name)


@needs_lib
def test_status_strings():
    for code in range(0, 12):
        assert la.linear_status_string(code) != "unknown status"
    assert la.linear_status_string(99) == "unknown status"


# Fake device addresses: validation must reject these calls before touching memory.
X = 0x7F0000000000
W = 0x7F1000000000
B = 0x7F2000000000
Y = 0x7F3000000000


def call(x=X, ldx=64, w=W, ldw=64, b=B, y=Y, ldy=32, M=8, N=32, K=64, path=0):
    return la._lib().linear_f16_ex(x, ldx, w, ldw, b, y, ldy, M, N, K, path, None)


def call_bias(x=X, ldx=64, w=W, ldw=64, b=B, y=Y, ldy=32, M=8, N=32, K=64):
    return la._lib().linear_f16(x, ldx, w, ldw, b, y, ldy, M, N, K, None)


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), la.LINEAR_E_SHAPE),
    (dict(N=-5), la.LINEAR_E_SHAPE),
    (dict(K=-1), la.LINEAR_E_SHAPE),
    (dict(M=1 << 31), la.LINEAR_E_SHAPE),
    (dict(x=0), la.LINEAR_E_NULL),
    (dict(w=0), la.LINEAR_E_NULL),
    (dict(y=0), la.LINEAR_E_NULL),
    (dict(ldx=63), la.LINEAR_E_STRIDE),
    (dict(ldw=10), la.LINEAR_E_STRIDE),
    (dict(ldy=31), la.LINEAR_E_STRIDE),
    (dict(ldx=1 << 22, ldw=64), la.LINEAR_E_STRIDE),
    (dict(path=3), la.LINEAR_E_PATH),
    (dict(path=-1), la.LINEAR_E_PATH),
    (dict(y=X + 100), la.LINEAR_E_ALIAS),           # y starts inside x
    (dict(y=W - 10), la.LINEAR_E_ALIAS),            # y runs into w
    (dict(b=Y + 2 * 32 * 3), la.LINEAR_E_ALIAS),    # b inside y
])
def test_validation_errors_are_reported_before_any_device_work(kw, code):
    assert call(**kw) == code


@needs_lib
def test_bias_entry_point_requires_bias():
    assert call_bias(b=0) == la.LINEAR_E_NULL


@needs_lib
def test_empty_output_is_a_noop_even_with_null_pointers():
    assert call(x=0, w=0, b=0, y=0, M=0) == la.LINEAR_OK
    assert call(x=0, w=0, b=0, y=0, N=0) == la.LINEAR_OK


@needs_lib
def test_k0_allows_null_inputs_until_the_device_check():
    # K == 0: x and w are never read, so NULL is accepted; without a GPU the call then
    # stops at the device check.
    rc = call(x=0, w=0, K=0, ldx=0, ldw=0)
    assert rc in (la.LINEAR_E_DEVICE, la.LINEAR_OK)
    if not torch.cuda.is_available():
        assert rc == la.LINEAR_E_DEVICE


@needs_lib
@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_valid_call_without_a_device_reports_device_error():
    assert call() == la.LINEAR_E_DEVICE
    assert la._lib().linear_last_hip_error() != 0


R = 0x7F4000000000   # fake residual
U = 0x7F5000000000   # fake gate input


def call_epi(ops, bias=B, res=R, ldr=32, mul=U, ldm=32, y=Y, ldy=32, M=8, N=32, K=64, bf16=False, nsteps=None):
    ep = la._Epilogue()
    ep.nsteps = len(ops) if nsteps is None else nsteps
    for i, o in enumerate(ops[:la.EPI_MAX_STEPS]):
        ep.op[i] = o
    ep.bias, ep.residual, ep.ldr, ep.mul, ep.ldm = bias, res, ldr, mul, ldm
    fn = la._lib().linear_bf16_epilogue if bf16 else la._lib().linear_f16_epilogue
    return fn(X, 64, W, 64, ctypes.byref(ep), y, ldy, M, N, K, 0, None)


@needs_lib
@pytest.mark.parametrize("bf16", [False, True], ids=["f16", "bf16"])
@pytest.mark.parametrize("kw,code", [
    (dict(ops=[], nsteps=-1), la.LINEAR_E_EPILOGUE),
    (dict(ops=[1] * 9, nsteps=9), la.LINEAR_E_EPILOGUE),
    (dict(ops=[7]), la.LINEAR_E_EPILOGUE),
    (dict(ops=[0]), la.LINEAR_E_EPILOGUE),
    (dict(ops=[la.EPI_BIAS], bias=0), la.LINEAR_E_NULL),
    (dict(ops=[la.EPI_RESIDUAL], res=0), la.LINEAR_E_NULL),
    (dict(ops=[la.EPI_MUL], mul=0), la.LINEAR_E_NULL),
    (dict(ops=[la.EPI_RESIDUAL], ldr=31), la.LINEAR_E_STRIDE),
    (dict(ops=[la.EPI_MUL], ldm=31), la.LINEAR_E_STRIDE),
    (dict(ops=[la.EPI_RESIDUAL], res=Y + 64), la.LINEAR_E_ALIAS),              # residual offset inside y
    (dict(ops=[la.EPI_RESIDUAL], res=Y, ldr=40), la.LINEAR_E_ALIAS),           # same start, other stride
    (dict(ops=[la.EPI_MUL], mul=Y), la.LINEAR_E_ALIAS),                        # y may not be the gate input
    (dict(ops=[la.EPI_BIAS], bias=Y + 6), la.LINEAR_E_ALIAS),
    (dict(ops=[la.EPI_BIAS, la.EPI_SILU], y=0), la.LINEAR_E_NULL),
])
def test_epilogue_validation(kw, code, bf16):
    assert call_epi(bf16=bf16, **kw) == code


@needs_lib
def test_epilogue_unused_inputs_may_be_null_and_in_place_residual_is_accepted():
    # the inputs a program does not read are never checked; the residual may be y itself
    no_dev = not torch.cuda.is_available()
    for kw in (dict(ops=[la.EPI_SILU], bias=0, res=0, mul=0), dict(ops=[], bias=0, res=0, mul=0),
               dict(ops=[la.EPI_BIAS, la.EPI_RESIDUAL], res=Y, ldr=32, mul=0)):
        rc = call_epi(**kw)
        assert rc in (la.LINEAR_E_DEVICE, la.LINEAR_OK)
        if no_dev:
            assert rc == la.LINEAR_E_DEVICE
    assert la._lib().linear_f16_epilogue(X, 64, W, 64, None, Y, 32, 8, 32, 64, 0, None) == la.LINEAR_E_NULL


def call_grouped(x=X, ldx=64, sx=8 * 64, w=W, ldw=64, b=B, y=Y, ldy=32, sy=8 * 32, G=3, M=8, N=32, K=64,
                 path=0):
    return la._lib().linear_f16_grouped(x, ldx, sx, w, ldw, b, y, ldy, sy, G, M, N, K, path, None)


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(G=-1), la.LINEAR_E_SHAPE),
    (dict(G=65536), la.LINEAR_E_SHAPE),
    (dict(sy=7 * 32 + 31), la.LINEAR_E_STRIDE),      # groups would write overlapping outputs
    (dict(sx=-1), la.LINEAR_E_STRIDE),
    (dict(y=X + 2 * 64 * 8 * 2), la.LINEAR_E_ALIAS),  # y inside the third activation slice
    (dict(b=Y + 2 * 8 * 32 * 2), la.LINEAR_E_ALIAS),  # b inside the third output group
    (dict(path=9), la.LINEAR_E_PATH),
    (dict(x=0), la.LINEAR_E_NULL),
])
def test_grouped_validation(kw, code):
    assert call_grouped(**kw) == code


@needs_lib
def test_grouped_noops_and_device_check():
    assert call_grouped(G=0, x=0, w=0, y=0) == la.LINEAR_OK
    rc = call_grouped(sx=0)             # every group reading the same activation is allowed
    assert rc in (la.LINEAR_E_DEVICE, la.LINEAR_OK)
    if not torch.cuda.is_available():
        assert rc == la.LINEAR_E_DEVICE


I = 0x7F6000000000   # fake idx
WS = 0x7F7000000000  # fake workspace


def call_indexed(x=X, ldx=64, w=W, ldw=32, sw=64 * 32, idx=I, y=Y, ldy=32, E=4, M=8, N=32, K=64, f32=False,
                 ws=WS, ws_bytes=1 << 20):
    fn = la._lib().linear_f16_indexed_f32out if f32 else la._lib().linear_f16_indexed
    return fn(x, ldx, w, ldw, sw, idx, y, ldy, E, M, N, K, ws, ws_bytes, None)


@needs_lib
def test_indexed_workspace_bytes():
    f = la._lib().linear_indexed_workspace_bytes
    assert f(-1, 4) == -1 and f(4, -1) == -1 and f(65536, 4) == -1
    # header, row list, then one 16-byte tile record per possible tile
    for E, M in ((1, 1), (8, 32), (8, 4096), (256, 100), (4096, 1 << 20)):
        n = f(E, M)
        assert n % 16 == 0
        assert n >= 4 * (M + 1) + 16 * ((M + 15) // 16 + E)
        assert n < 4 * (M + 72) + 16 * ((M + 15) // 16 + E)
    assert la.indexed_workspace_bytes(8, 32) == f(8, 32)


@needs_lib
@pytest.mark.parametrize("f32", [False, True], ids=["round", "f32out"])
@pytest.mark.parametrize("kw,code", [
    (dict(E=-1), la.LINEAR_E_SHAPE),
    (dict(E=65536), la.LINEAR_E_SHAPE),
    (dict(M=-2), la.LINEAR_E_SHAPE),
    (dict(idx=0), la.LINEAR_E_NULL),
    (dict(w=0), la.LINEAR_E_NULL),
    (dict(ldw=31), la.LINEAR_E_STRIDE),
    (dict(sw=64 * 32 - 1), la.LINEAR_E_STRIDE),
    (dict(ldx=63), la.LINEAR_E_STRIDE),
    (dict(ldy=31), la.LINEAR_E_STRIDE),
    (dict(y=W + 3 * 64 * 32 * 2), la.LINEAR_E_ALIAS),   # y inside the last expert table
    (dict(idx=Y + 16), la.LINEAR_E_ALIAS),
    (dict(ws=0), la.LINEAR_E_NULL),
    (dict(ws_bytes=0), la.LINEAR_E_WORKSPACE),
    (dict(ws=WS + 8), la.LINEAR_E_WORKSPACE),           # misaligned
    (dict(ws=Y), la.LINEAR_E_ALIAS),                    # workspace over y
    (dict(ws=X + 64), la.LINEAR_E_ALIAS),               # workspace over x
    (dict(ws=I - 64), la.LINEAR_E_ALIAS),               # workspace over idx
])
def test_indexed_validation(kw, code, f32):
    assert call_indexed(f32=f32, **kw) == code


@needs_lib
def test_indexed_noops_and_device_check():
    assert call_indexed(E=0, x=0, w=0, idx=0, y=0, ws=0) == la.LINEAR_OK
    assert call_indexed(M=0, idx=0, ws=0) == la.LINEAR_OK
    rc = call_indexed()
    assert rc in (la.LINEAR_E_DEVICE, la.LINEAR_OK)
    if not torch.cuda.is_available():
        assert rc == la.LINEAR_E_DEVICE


@needs_lib
def test_indexed_noalloc_host_checks():
    """The no-allocation call: the workspace call's shape checks and no-ops, and
    LINEAR_E_SCRATCH (before any device work) when the routing would not fit the
    library's scratch array."""
    f = la._lib().linear_f16_indexed_noalloc
    ws_bytes = la._lib().linear_indexed_workspace_bytes

    def call(**kw):
        a = dict(x=X, ldx=64, w=W, ldw=32, sw=64 * 32, idx=I, y=Y, ldy=32, E=4, M=48, N=32, K=64)
        a.update(kw)
        return f(a["x"], a["ldx"], a["w"], a["ldw"], a["sw"], a["idx"], a["y"], a["ldy"], a["E"], a["M"], a["N"],
                 a["K"], None)
    assert call(E=-1) == la.LINEAR_E_SHAPE and call(M=-1) == la.LINEAR_E_SHAPE and call(E=65536) == la.LINEAR_E_SHAPE
    assert call(E=0, x=0, w=0, idx=0, y=0) == la.LINEAR_OK
    assert call(M=0, idx=0) == la.LINEAR_OK
    # the largest row count that fits at 8 experts, and one more
    m = 1
    while ws_bytes(8, 2 * m) <= la.NOALLOC_SCRATCH_BYTES:
        m *= 2
    lo, hi = m, 2 * m
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if ws_bytes(8, mid) <= la.NOALLOC_SCRATCH_BYTES else (lo, mid)
    assert lo > 150000
    assert call(E=8, M=hi, ldx=64) == la.LINEAR_E_SCRATCH
    rc = call(E=8, M=lo)
    assert rc in (la.LINEAR_E_DEVICE, la.LINEAR_E_ALIAS, la.LINEAR_OK)
    if not torch.cuda.is_available():
        assert call() == la.LINEAR_E_DEVICE


def plan(M, N, K, path=0, x=X, w=W, ldx=None, ldw=None):
    p = la._Plan()
    rc = la._lib().linear_f16_plan(x, ldx or K, w, ldw or K, B, Y, N, M, N, K, path, ctypes.byref(p))
    assert rc == la.LINEAR_OK
    return {f: getattr(p, f) for f, _ in la._Plan._fields_}


@needs_lib
def test_plans_for_the_workloads():
    from linear_amd.workloads import WORKLOADS
    for name, wl in WORKLOADS.items():
        p = plan(wl.M, wl.N, wl.K)
        if wl.M <= 16:
            assert p["path"] == la.PATH_SKINNY, name
        else:
            assert p["path"] == la.PATH_GEMM, name
            assert p["grid"] >= 256, (name, p)
        assert p["vector_io"] == 1
    # the toy runs 256 tiles of 64 x 64 through a 4-slice ring
    p = plan(1024, 1024, 768)
    assert (p["tile_m"], p["tile_n"], p["threads"], p["stages"], p["tile_k"], p["grid"]) == (64, 64, 256, 4, 64, 256)
    assert plan(8192, 4096, 4096)["stages"] == 2 and plan(2000, 4000, 14336)["stages"] == 3
    assert plan(16, 4096, 4096)["stages"] == 0                # the skinny path has no ring
    # a single x row: one wave per weight row, 4 rows per workgroup, 512 K per wave load
    p = plan(1, 4096, 4096)
    assert (p["path"], p["tile_m"], p["tile_n"], p["tile_k"], p["threads"], p["grid"]) == (la.PATH_SKINNY, 1, 4, 512,
                                                                                          256, 1024)
    assert plan(1, 4097, 32768)["grid"] == 1025
    assert plan(1, 64, 32776)["tile_m"] == 16                  # x too long to stage: the 16-row kernel
    assert plan(1, 64, 63)["tile_m"] == 16                     # no 16-byte loads
    assert plan(2, 4096, 4096)["tile_m"] == 16
    assert plan(1, 64, 64, path=la.PATH_SKINNY)["tile_m"] == 1


@needs_lib
def test_binding_refuses_host_tensors():
    """A host tensor handed to a kernel would fault the GPU: every entry point of
    the binding refuses it with ValueError before the library is called."""
    f16, bf = torch.float16, torch.bfloat16
    x, w, b = torch.zeros(4, 8, dtype=f16), torch.zeros(6, 8, dtype=f16), torch.zeros(6, dtype=f16)
    xb, wb, bb = x.to(bf), w.to(bf), b.to(bf)
    idx = torch.zeros(4, dtype=torch.int32)
    calls = [
        (la.linear_f16, (x, w, b)), (la.linear_f16_nobias, (x, w)), (la.linear_f16_ex, (x, w, b)),
        (la.linear_f16_f32out, (x, w)), (la.linear_bf16, (xb, wb, bb)), (la.linear_bf16_nobias, (xb, wb)),
        (la.linear_bf16_ex, (xb, wb, None)), (la.linear_bf16_f32out, (xb, wb)),
        (la.linear_f16_epilogue, (x, w, [la.EPI_BIAS], b)), (la.linear_bf16_epilogue, (xb, wb, [la.EPI_SILU])),
        (la.linear_f16_grouped, (x.view(1, 4, 8), w, b)), (la.linear_bf16_grouped, (xb.view(1, 4, 8), wb)),
        (la.linear_f16_grouped_f32out, (x.view(1, 4, 8), w)), (la.linear_bf16_grouped_f32out, (xb.view(1, 4, 8), wb)),
        (la.linear_f16_indexed, (x, w.view(1, 8, 6), idx)), (la.linear_bf16_indexed, (xb, wb.view(1, 8, 6), idx)),
        (la.linear_f16_indexed_f32out, (x, w.view(1, 8, 6), idx)),
        (la.linear_bf16_indexed_f32out, (xb, wb.view(1, 8, 6), idx)),
        (la.linear, (x, w, b)),
    ]
    for fn, args in calls:
        with pytest.raises(ValueError, match="on the GPU"):
            fn(*args)


@needs_lib
def test_column_split_rule():
    """A GEMM call whose 256 x 256 tiles leave a last wave at most half full over
    256 CUs is split by columns: whole waves first, the rest with its own tile."""
    p = plan(4096, 14336, 4096)                      # mlp_up: 896 tiles, 3.5 waves
    assert (p["tile_m"], p["tile_n"], p["grid"]) == (256, 256, 768)
    assert (p["split_n"], p["tile_m2"], p["tile_n2"], p["grid2"]) == (12288, 256, 128, 256)
    p = plan(4096, 4352, 512)                       # 272 tiles: the last 256 columns alone
    assert (p["grid"], p["split_n"], p["tile_m2"], p["tile_n2"], p["grid2"]) == (256, 4096, 64, 64, 256)
    p = plan(300, 34800, 72)                        # 2 x 136 tiles, ragged remainder
    assert (p["grid"], p["split_n"], p["tile_m2"], p["tile_n2"], p["grid2"]) == (256, 32768, 64, 64, 160)
    for M, N in [(8192, 4096), (2000, 4000), (4096, 27 * 256), (1024, 1024), (4096, 16128)]:
        # whole waves, a last wave more than half full, or another tile: one launch
        p = plan(M, N, 512)
        assert p["split_n"] == 0 and p["grid2"] == 0 and p["tile_m2"] == 0, (M, N, p)
    assert plan(4096, 14336, 4096, path=la.PATH_SKINNY)["split_n"] == 0


@needs_lib
def test_plan_falls_back_to_elementwise_loader():
    assert plan(64, 64, 63)["vector_io"] == 0          # K % 8 != 0
    assert plan(64, 64, 64, x=X + 2)["vector_io"] == 0  # misaligned x
    assert plan(64, 64, 64, ldx=72)["vector_io"] == 1   # padded stride, still aligned
    assert plan(64, 64, 64, ldw=66)["vector_io"] == 0


@needs_lib
def test_forced_paths():
    assert plan(1000, 64, 64, path=la.PATH_SKINNY)["path"] == la.PATH_SKINNY
    assert plan(1, 64, 64, path=la.PATH_GEMM)["path"] == la.PATH_GEMM


def test_product_package_does_not_import_the_oracle():
    for root, _, files in os.walk(os.path.join(ROOT, "linear_amd")):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(root, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "oracle.c" not in text and "liboracle" not in text, f


@needs_lib
def test_every_kernel_launch_stub_is_defined():
    """Each kernel the library launches must be defined in the library itself (the
    host compilation pass can silently drop a kernel's launch stub)."""
    out = subprocess.run(["nm", "-C", la.LIB_PATH], capture_output=True, text=True, check=True).stdout
    undefined = [l for l in out.splitlines() if " U " in l and "lin::" in l]
    assert not undefined, undefined[:5]
