"""C-ABI checks that need no GPU: the library loads, exports every declared entry point, and
every host-side validation path returns its error code without launching anything."""
import ctypes
import os
import re

import pytest

import grouped_gemm_expert_router_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return moe.load_library()


def test_header_declares_the_entry_points():
    assert header_functions() == sorted(moe.ENTRY_POINTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in (moe.MOE_OK, moe.MOE_ERR_NULL, moe.MOE_ERR_SHAPE, moe.MOE_ERR_DTYPE, moe.MOE_ERR_WORKSPACE,
               moe.MOE_ERR_ALIGN):
        assert len(moe.status_string(st)) >= 2
    assert moe.status_string(-99) == "unknown status"


def sz(lib, dm, which):
    out = ctypes.c_size_t(0)
    rc = lib.moe_workspace_bytes(ctypes.byref(dm), which, ctypes.byref(out))
    return rc, out.value


@pytest.mark.parametrize("bad", [
    dict(k=0), dict(k=9), dict(E=0), dict(E=1025, k=2), dict(k=65, E=128), dict(d=100), dict(f=64),
    dict(T=-1), dict(d=0), dict(T=(1 << 31) // 2, k=2),
])
def test_shape_errors(lib, bad):
    p = dict(T=64, d=128, f=256, E=8, k=2)
    p.update(bad)
    dm = moe.dims(**p)
    assert sz(lib, dm, moe.MOE_WS_FORWARD)[0] == moe.MOE_ERR_SHAPE


def test_dtype_and_reserved_errors(lib):
    dm = moe.dims(64, 128, 256, 8, 2, dtype=7)
    assert sz(lib, dm, moe.MOE_WS_FORWARD)[0] == moe.MOE_ERR_DTYPE
    dm = moe.dims(64, 128, 256, 8, 2)
    dm.reserved = 1
    assert sz(lib, dm, moe.MOE_WS_FORWARD)[0] == moe.MOE_ERR_SHAPE
    assert lib.moe_workspace_bytes(None, 0, None) == moe.MOE_ERR_NULL
    assert lib.moe_workspace_bytes(ctypes.byref(moe.dims(64, 128, 256, 8, 2)), 0, None) == moe.MOE_ERR_NULL
    assert sz(lib, moe.dims(64, 128, 256, 8, 2), 4)[0] == moe.MOE_ERR_SHAPE


def test_fp8_shape_rules(lib):
    # the fp8 tiles are 256 wide along d and f
    assert sz(lib, moe.dims(64, 128, 256, 8, 2, dtype=moe.MOE_FP8_E4M3), moe.MOE_WS_FORWARD)[0] == moe.MOE_ERR_SHAPE
    assert sz(lib, moe.dims(64, 256, 384, 8, 2, dtype=moe.MOE_FP8_E4M3), moe.MOE_WS_FORWARD)[0] == moe.MOE_ERR_SHAPE
    bf = moe.dims(64, 256, 256, 8, 2)
    f8 = moe.dims(64, 256, 256, 8, 2, dtype=moe.MOE_FP8_E4M3)
    # fp8 adds the e4m3 copies of As (forward) and of dy and dH, plus x dequantised to bf16 for the
    # bf16 weight gradients (backward)
    A, T, d, f = 128, 64, 256, 256
    # forward: the per-pair outputs Op [A, d] bf16 plus As in e4m3 with its 1x128 scales
    assert sz(lib, f8, moe.MOE_WS_FORWARD)[1] >= A * d * 2 + A * f + A * (f // 128) * 4
    assert sz(lib, f8, moe.MOE_WS_BACKWARD)[1] >= (sz(lib, bf, moe.MOE_WS_BACKWARD)[1] + T * d + A * 2 * f
                                                   + T * d * 2)


def test_workspace_sizes_scale_with_pairs_not_capacity(lib):
    small = sz(lib, moe.dims(64, 128, 256, 8, 2), moe.MOE_WS_FORWARD)[1]
    big = sz(lib, moe.dims(128, 128, 256, 8, 2), moe.MOE_WS_FORWARD)[1]
    assert 0 < small < big
    out = ctypes.c_size_t(0)
    assert lib.moe_saved_bytes(ctypes.byref(moe.dims(64, 128, 256, 8, 2)), ctypes.byref(out)) == 0
    # saved context = H [A, 2f] + As [A, f] in bf16, nothing sized by experts x capacity
    assert out.value == 64 * 2 * 2 * 256 * 2 + 64 * 2 * 256 * 2
    # zero tokens is a legal (empty) layer
    assert sz(lib, moe.dims(0, 128, 256, 8, 2), moe.MOE_WS_FORWARD)[0] == 0


FAKE = 1 << 20  # a non-null, 256-aligned address that is never dereferenced on error paths


def test_route_and_plan_argument_errors(lib):
    dm = moe.dims(64, 128, 256, 8, 2)
    rc, need = sz(lib, dm, moe.MOE_WS_ROUTE)
    assert rc == 0 and need > 0
    args = [FAKE] * 7
    assert lib.moe_route(ctypes.byref(dm), None, *args, need, None) == moe.MOE_ERR_NULL
    assert lib.moe_route(ctypes.byref(dm), FAKE, *args[:-1], None, need, None) == moe.MOE_ERR_NULL
    assert lib.moe_route(ctypes.byref(dm), FAKE, *args, need - 1, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(dm), FAKE, *args[:-1], FAKE + 8, need, None) == moe.MOE_ERR_ALIGN
    assert lib.moe_plan(ctypes.byref(dm), None, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == moe.MOE_ERR_NULL
    assert lib.moe_plan(ctypes.byref(dm), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == moe.MOE_ERR_WORKSPACE
    bad = moe.dims(64, 128, 256, 8, 9)
    assert lib.moe_route(ctypes.byref(bad), FAKE, *args, need, None) == moe.MOE_ERR_SHAPE


def test_forward_backward_argument_errors(lib):
    dm = moe.dims(64, 128, 256, 8, 2)
    _, wf = sz(lib, dm, moe.MOE_WS_FORWARD)
    _, wb = sz(lib, dm, moe.MOE_WS_BACKWARD)
    F = FAKE
    fwd = lambda **o: lib.moe_forward(ctypes.byref(o.get("dm", dm)), o.get("x", F), o.get("xs", None), F, None, F,
                                      None, F, F, F, F, o.get("y", F), F, F, o.get("ws", wf), None)
    assert fwd(x=None) == moe.MOE_ERR_NULL
    assert fwd(y=None) == moe.MOE_ERR_NULL
    assert fwd(xs=F) == moe.MOE_ERR_DTYPE                 # scales with bf16
    assert fwd(ws=wf - 1) == moe.MOE_ERR_WORKSPACE
    assert fwd(x=F + 2) == moe.MOE_ERR_ALIGN
    fp8 = moe.dims(64, 256, 256, 8, 2, dtype=moe.MOE_FP8_E4M3)
    rc, wf8 = sz(lib, fp8, moe.MOE_WS_FORWARD)
    assert rc == 0
    f8 = lambda *sc, ws=wf8: lib.moe_forward(ctypes.byref(fp8), F, sc[0], F, sc[1], F, sc[2], F, F, F, F, F, F, F,
                                             ws, None)
    assert f8(None, F, F) == moe.MOE_ERR_NULL              # fp8 needs every scale
    assert f8(F, F, None) == moe.MOE_ERR_NULL
    assert f8(F, F, F, ws=wf8 - 1) == moe.MOE_ERR_WORKSPACE
    assert f8(F + 4, F, F) == moe.MOE_ERR_ALIGN
    b8 = lambda *sc: lib.moe_backward(ctypes.byref(fp8), F, F, sc[0], F, sc[1], F, sc[2], F, F, F, F, F, F, F, F, F,
                                      F, F, F, sz(lib, fp8, moe.MOE_WS_BACKWARD)[1], None)
    assert b8(F, None, F) == moe.MOE_ERR_NULL
    bwd = lambda **o: lib.moe_backward(ctypes.byref(dm), F, F, None, F, None, F, None, o.get("ids", F), F, F, F, F, F,
                                       F, F, F, o.get("dtw", F), o.get("dl", F), F, o.get("ws", wb), None)
    assert bwd(dtw=None) == moe.MOE_ERR_NULL
    assert bwd(ids=None) == moe.MOE_ERR_NULL               # d_logits requested without ids
    assert bwd(ws=wb - 1) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_combine(ctypes.byref(dm), None, F, F, None) == moe.MOE_ERR_NULL
    assert lib.moe_permute(ctypes.byref(dm), F, F, None, None) == moe.MOE_ERR_NULL
    assert lib.moe_permute(ctypes.byref(dm), F + 4, F, F, None) == moe.MOE_ERR_ALIGN
    assert lib.moe_combine(ctypes.byref(dm), F + 4, F, F, None) == moe.MOE_ERR_ALIGN
    # an empty layer is legal with NULL buffers for the data-movement steps, as for the layer
    empty = moe.dims(0, 128, 256, 8, 2)
    assert lib.moe_combine(ctypes.byref(empty), None, None, None, None) == moe.MOE_OK
    assert lib.moe_permute(ctypes.byref(empty), None, None, None, None) == moe.MOE_OK
    assert lib.moe_forward(ctypes.byref(empty), *([None] * 13), 0, None) == moe.MOE_OK


def test_fused_forward_argument_errors(lib):
    dm = moe.dims(64, 128, 256, 8, 2)
    _, wf = sz(lib, dm, moe.MOE_WS_FORWARD)
    F = FAKE
    fused = lambda **o: lib.moe_forward_fused(ctypes.byref(o.get("dm", dm)), o.get("x", F), F, F, F, F, F, F,
                                              o.get("y", F), o.get("saved", F), F, o.get("ws", wf), None)
    assert fused(x=None) == moe.MOE_ERR_NULL
    assert fused(y=None) == moe.MOE_ERR_NULL
    assert fused(saved=None) == moe.MOE_ERR_NULL
    assert fused(ws=wf - 1) == moe.MOE_ERR_WORKSPACE
    assert fused(x=F + 2) == moe.MOE_ERR_ALIGN
    assert fused(saved=F + 16) == moe.MOE_ERR_ALIGN
    assert fused(dm=moe.dims(64, 128, 200, 8, 2)) == moe.MOE_ERR_SHAPE
    for dt in (moe.MOE_FP8_E4M3, moe.MOE_MXFP8):           # bf16 only
        assert fused(dm=moe.dims(64, 256, 256, 8, 2, dtype=dt)) == moe.MOE_ERR_DTYPE
    empty = moe.dims(0, 128, 256, 8, 2)
    assert lib.moe_forward_fused(ctypes.byref(empty), *([None] * 10), 0, None) == moe.MOE_OK


def test_mxfp8_argument_rules(lib):
    F = FAKE
    mx = moe.dims(64, 256, 256, 8, 2, dtype=moe.MOE_MXFP8)
    rc, wf = sz(lib, mx, moe.MOE_WS_FORWARD)
    assert rc == 0
    # MXFP8 takes bf16 inputs and quantises them itself: scales must be NULL
    assert lib.moe_forward(ctypes.byref(mx), F, F, F, None, F, None, F, F, F, F, F, F, F, wf, None) == moe.MOE_ERR_DTYPE
    # workspace holds the quantised copies: larger than the bf16 layer's
    bf = moe.dims(64, 256, 256, 8, 2)
    assert wf > sz(lib, bf, moe.MOE_WS_FORWARD)[1] + 8 * 256 * 512   # at least W1's e4m3 codes
    assert sz(lib, moe.dims(64, 128, 256, 8, 2, dtype=moe.MOE_MXFP8), moe.MOE_WS_FORWARD)[0] == moe.MOE_ERR_SHAPE
    q = lambda *a: lib.moe_mxfp8_quantize(*a, None)
    assert q(F, 1, 64, 100, 1, F, F) == moe.MOE_ERR_SHAPE      # row blocks need cols % 32 == 0
    assert q(F, 1, 40, 64, 0, F, F) == moe.MOE_ERR_SHAPE       # column blocks need rows % 32 == 0
    assert q(F, 1, 64, 60, 0, F, F) == moe.MOE_ERR_SHAPE       # ... and cols % 8 == 0
    assert q(F, 1, 64, 64, 2, F, F) == moe.MOE_ERR_SHAPE       # block_axis is 0 or 1
    assert q(None, 1, 64, 64, 1, F, F) == moe.MOE_ERR_NULL
    assert q(F, 1, 64, 64, 1, F + 8, F) == moe.MOE_ERR_ALIGN
    assert q(F, 0, 64, 64, 1, None, None) == moe.MOE_OK         # empty input: nothing to do
    assert q(F, 1 << 20, 1 << 12, 1 << 12, 1, F, F) == moe.MOE_ERR_SHAPE   # 2^44 elements
    w = lambda *a: lib.moe_mxfp8_quantize_weights(*a, None)
    assert w(F, 1, 64, 384, F, F, F, F) == moe.MOE_ERR_SHAPE    # cols % 256 == 0
    assert w(F, 1, 48, 256, F, F, F, F) == moe.MOE_ERR_SHAPE    # rows % 32 == 0
    assert w(F, -1, 64, 256, F, F, F, F) == moe.MOE_ERR_SHAPE
    assert w(F, 1 << 20, 1 << 12, 1 << 12, F, F, F, F) == moe.MOE_ERR_SHAPE
    assert w(F, 1, 64, 256, F, None, F, F) == moe.MOE_ERR_NULL
    assert w(F, 1, 64, 256, F, F + 4, F, F) == moe.MOE_ERR_ALIGN   # column exponents: 8-byte aligned
    assert w(F, 1, 64, 256, F, F, F, F + 2) == moe.MOE_ERR_ALIGN   # row exponent words: 4-byte aligned
    assert w(F, 0, 64, 256, None, None, None, None) == moe.MOE_OK


def test_mxfp8_padded_rows_rule(lib):
    # T*k = 2^31 - 1000 pairs is a legal bf16 (and blockwise fp8) layer; MXFP8 pads each expert's
    # rows to a multiple of 128 for the weight gradients, which would pass 2^31 with 1024 experts
    T, k, E = 268435331, 8, 1024
    assert sz(lib, moe.dims(T, 256, 256, E, k), moe.MOE_WS_FORWARD)[0] == moe.MOE_OK
    assert sz(lib, moe.dims(T, 256, 256, E, k, dtype=moe.MOE_FP8_E4M3), moe.MOE_WS_FORWARD)[0] == moe.MOE_OK
    mx = moe.MOE_MXFP8
    assert sz(lib, moe.dims(T, 256, 256, E, k, dtype=mx), moe.MOE_WS_FORWARD)[0] == moe.MOE_ERR_SHAPE
    assert sz(lib, moe.dims(T // 2, 256, 256, E, k, dtype=mx), moe.MOE_WS_FORWARD)[0] == moe.MOE_OK


def test_route_noalloc_host_rules(lib):
    # the fixed 4 MiB scratch holds the plan tables of every shape the ABI accepts: the largest
    # (1024 experts, T*k just under 2^31) needs exactly 2 * 1024 * 512 int32
    rc, need = sz(lib, moe.dims(268435455, 128, 128, 1024, 8), moe.MOE_WS_ROUTE)
    assert rc == 0 and need <= 4 << 20
    dm = moe.dims(64, 128, 256, 8, 2)
    outs = [FAKE] * 6       # topk_ids, topk_w, counts, offsets, perm, inv_perm
    assert lib.moe_route_noalloc(ctypes.byref(dm), None, *outs, None) == moe.MOE_ERR_NULL
    assert lib.moe_route_noalloc(ctypes.byref(dm), FAKE, *outs[:-1], None, None) == moe.MOE_ERR_NULL
    assert lib.moe_route_noalloc(ctypes.byref(moe.dims(64, 128, 256, 8, 9)), FAKE, *outs, None) == moe.MOE_ERR_SHAPE


def test_router_front_end_host_rules(lib):
    F = FAKE
    dm = moe.dims(4096, 256, 128, 64, 4)
    rc, need = sz(lib, dm, moe.MOE_WS_ROUTER)
    # dWg's token slices: fp32 partials of the whole [d, E] gradient per slice
    assert rc == 0 and need % 256 == 0 and need >= 2 * 256 * 64 * 4
    lg = lambda *a, d=dm: lib.moe_router_logits(ctypes.byref(d), *a, None)
    assert lg(None, F, F) == moe.MOE_ERR_NULL
    assert lg(F, F, F + 4) == moe.MOE_ERR_ALIGN
    assert lg(F, F, F, d=moe.dims(64, 256, 256, 8, 2, dtype=moe.MOE_FP8_E4M3)) == moe.MOE_ERR_DTYPE
    assert lg(None, None, None, d=moe.dims(0, 128, 128, 8, 2)) == moe.MOE_OK
    bw = lambda x, wg, dl, dx, dwg, ws, nb: lib.moe_router_backward(ctypes.byref(dm), x, wg, dl, dx, dwg, ws, nb, None)
    assert bw(F, F, None, F, F, F, need, ) == moe.MOE_ERR_NULL          # d_logits
    assert bw(None, F, F, None, F, F, need) == moe.MOE_ERR_NULL         # dWg needs x
    assert bw(F, None, F, F, None, F, need) == moe.MOE_ERR_NULL         # dx needs Wg
    assert bw(F, F, F, None, F, None, need) == moe.MOE_ERR_NULL         # dWg needs the workspace
    assert bw(F, F, F, None, F, F, need - 256) == moe.MOE_ERR_WORKSPACE
    assert bw(F, F, F, None, F, F + 16, need) == moe.MOE_ERR_ALIGN
    assert bw(None, None, None, None, None, None, 0) == moe.MOE_OK     # nothing requested
