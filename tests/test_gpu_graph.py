"""The layer's calls captured in a HIP graph (torch.cuda.CUDAGraph over the C ABI) and replayed.

Every entry point only enqueues kernels on the caller's stream (no allocation, no host
synchronisation, no memset), so a whole step - routing, forward, backward - can be captured once
and replayed.  Each replay is checked bit for bit against the eager step on the same inputs, with
eager work and synchronisations between the replays, and the outputs are poisoned before each
replay so that stale values cannot pass."""
import pytest
import torch

import grouped_gemm_expert_router_amd as moe
from workloads import make_inputs, make_prerouted_fp8
from moe_testlib import GpuLayer

pytestmark = pytest.mark.gpu

ROUTE_OUTS = ("topk_ids", "topk_w")
OUTS = ("counts", "offsets", "perm", "inv_perm", "y", "dx", "dW1", "dW2", "d_topk_w")


def _poison(gl, outs):
    for name in outs:
        t = gl.b[name]
        if t.is_floating_point():
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


def _snapshot(gl, outs):
    return {name: gl.b[name].clone() for name in outs}


def _check(gl, ref, what, outs):
    A = int(ref["offsets"][-1].item())
    for name in outs:
        a, b = ref[name], gl.b[name]
        if name == "perm":  # entries past offsets[E] are unused (pairs routed elsewhere have none)
            a, b = a[:A], b[:A]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{what}: {name} differs from the eager step"


# bf16 routed from logits (also through the single-launch forward), bf16 inputs run as MXFP8,
# and the pre-routed blockwise-fp8 share (plan instead of route, no logits)
CASES = ["bf16", "bf16_fused", "mxfp8", "fp8"]


@pytest.mark.parametrize("case", CASES)
def test_step_graph_replays_match_eager(case):
    if case == "fp8":
        inp = make_prerouted_fp8(256, 16, 4, 256, 256, 4, 46, name="fp8_graph")
        gl = GpuLayer(inp)
    else:
        inp = make_inputs(300, 256, 256, 8, 2, seed=40)
        gl = GpuLayer(inp, dtype=moe.MOE_MXFP8 if case == "mxfp8" else None)
    print(f"[case] graph replay {case}", flush=True)
    b = gl.b
    routed = gl.logits is not None
    outs = OUTS + (ROUTE_OUTS + ("d_logits",) if routed else ())

    def step():
        gl.route()
        if case == "bf16_fused":
            moe.moe_forward_fused(gl.dm, gl.x, gl.W1, gl.W2, b["topk_w"], b["offsets"], b["perm"], b["inv_perm"],
                                  b["y"], b["saved"], b["ws_fwd"])
        else:
            gl.forward()
        gl.backward(with_logits=routed)

    step()
    torch.cuda.synchronize()
    ref = _snapshot(gl, outs)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream's kind of stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        _poison(gl, outs)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _check(gl, ref, f"replay {rep}", outs)
        # eager work between replays: the same step, checked too
        _poison(gl, outs)
        step()
        torch.cuda.synchronize()
        _check(gl, ref, f"eager step after replay {rep}", outs)
