"""GPU checks of the single-launch forward (moe_forward_fused) through the C ABI.

It runs the same per-tile arithmetic as moe_forward in one persistent launch, so y and the saved
H and As must equal moe_forward's bit for bit; y is also compared with the fp64 oracle, and the
backward run from the fused forward's `saved` must match the oracle as well.  The cases cover
more row tiles than compute units (every queue drained and stolen from), fewer, ragged tails,
empty experts, the 128-wide down tiles (d not a multiple of 256) and the full Qwen3 shape."""
import numpy as np
import pytest
import torch

import grouped_gemm_expert_router_amd as moe
import oracle
from workloads import make_config, make_inputs
from moe_testlib import GpuLayer, TOL_BF16, check_full_parity, oracle_full, rel_err, to_np

pytestmark = pytest.mark.gpu


def _fused(gl, y, saved):
    b = gl.b
    moe.moe_forward_fused(gl.dm, gl.x, gl.W1, gl.W2, b["topk_w"], b["offsets"], b["perm"], b["inv_perm"], y, saved,
                          b["ws_fwd"])


def _both(gl):
    """Two-launch and fused forwards on the same routing, from zeroed outputs."""
    b = gl.b
    gl.route()
    b["y"].zero_()
    b["saved"].zero_()
    gl.forward()
    y2 = torch.zeros_like(b["y"])
    s2 = torch.zeros_like(b["saved"])
    _fused(gl, y2, s2)
    torch.cuda.synchronize()
    return y2, s2


def _assert_same(gl, y2, s2):
    assert torch.equal(gl.b["y"].view(torch.int16), y2.view(torch.int16)), "y differs from moe_forward"
    assert torch.equal(gl.b["saved"], s2), "saved H / As differ from moe_forward"


CASES = {
    # name: (T, d, f, E, k, seed)
    "small": (64, 128, 256, 8, 2, 30),
    "ragged_tails": (77, 256, 384, 6, 3, 31),
    "down_tiles_128": (300, 384, 256, 4, 2, 32),          # d % 256 = 128: 256x128 down tiles
    "one_token": (1, 128, 128, 4, 2, 33),
    "max_experts": (96, 128, 128, 1024, 4, 34),          # most of the 1024 queues' experts empty
    # 8192 x 8 pairs over 64 experts: about 290 row tiles for 256 compute units, with full and
    # partial tiles in every queue
    "more_tiles_than_cus": (8192, 256, 256, 64, 8, 35),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_forward_equals_two_launch_forward(name):
    T, d, f, E, k, seed = CASES[name]
    print(f"[case] fused {name} T={T} d={d} f={f} E={E} k={k} seed={seed}", flush=True)
    inp = make_inputs(T, d, f, E, k, seed=seed)
    gl = GpuLayer(inp, backward=False)
    y2, s2 = _both(gl)
    _assert_same(gl, y2, s2)
    ids, w = oracle.route(inp.logits, k)
    x, W1, W2 = (oracle.bf16_to_f64(a) for a in (inp.x, inp.W1, inp.W2))
    assert rel_err(to_np(y2), oracle.forward(x, W1, W2, ids, w)) <= TOL_BF16


def test_fused_forward_feeds_the_backward():
    """moe_backward on the fused forward's saved context: full parity with the oracle."""
    inp = make_inputs(200, 256, 256, 8, 4, seed=36)
    print("[case] fused forward then backward", flush=True)
    gl = GpuLayer(inp)
    gl.route()
    b = gl.b
    _fused(gl, b["y"], b["saved"])
    gl.backward(with_logits=True)
    torch.cuda.synchronize()
    check_full_parity(gl, oracle_full(inp))


def test_fused_forward_skewed_and_empty_experts():
    E = 16
    bias = np.zeros(E, np.float32)
    bias[::2] = -100.0          # even experts never selected
    bias[3] = 4.0               # expert 3 takes most first slots: several queues steal its tiles
    inp = make_inputs(3000, 128, 256, E, 2, seed=37, logits_bias=bias)
    print("[case] fused skewed, empty experts", flush=True)
    gl = GpuLayer(inp, backward=False)
    y2, s2 = _both(gl)
    _assert_same(gl, y2, s2)


def test_fused_forward_twice_then_smaller():
    """The queue counters are rebuilt by every call: repeated and smaller calls stay exact."""
    big = make_inputs(2000, 128, 256, 8, 4, seed=38)
    small = make_inputs(70, 128, 256, 8, 4, seed=39)
    print("[case] fused repeated calls", flush=True)
    gl = GpuLayer(big, backward=False)
    y2, s2 = _both(gl)
    _fused(gl, y2, s2)          # second call on the same workspace
    torch.cuda.synchronize()
    _assert_same(gl, y2, s2)
    gs = GpuLayer(small, backward=False)
    gs.b["ws_fwd"] = gl.b["ws_fwd"]   # the big call's workspace, counters left past their ends
    y3, s3 = _both(gs)
    _assert_same(gs, y3, s3)


@pytest.mark.slow
def test_fused_forward_fullsize_qwen3():
    """The Qwen3-30B-A3B shape (T=16384, d=2048, f=768, E=128, top-8): 574 row tiles."""
    inp = make_config("qwen3")
    print(f"[case] fused full-size qwen3 T={inp.T}", flush=True)
    gl = GpuLayer(inp, backward=False)
    y2, s2 = _both(gl)
    _assert_same(gl, y2, s2)
