"""The layer's calls captured in a HIP graph (torch.cuda.CUDAGraph over the C ABI) and replayed.

Every entry point only enqueues kernels on the caller's stream (no allocation, no host
synchronisation, no memset), so a whole step - routing, forward, backward - can be captured once
and replayed.  Each replay is checked bit for bit against the eager step on the same inputs, with
eager work and synchronisations between the replays, and the outputs are poisoned before each
replay so that stale values cannot pass."""
import pytest
import torch

import grouped_gemm_expert_router_amd as moe
from workloads import make_inputs
from moe_testlib import GpuLayer

pytestmark = pytest.mark.gpu

OUTS = ("topk_ids", "topk_w", "counts", "offsets", "perm", "inv_perm", "y", "dx", "dW1", "dW2", "d_topk_w",
        "d_logits")


def _poison(gl):
    for name in OUTS:
        t = gl.b[name]
        if t.is_floating_point():
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


def _snapshot(gl):
    return {name: gl.b[name].clone() for name in OUTS}


def _check(gl, ref, what):
    for name in OUTS:
        a, b = ref[name], gl.b[name]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{what}: {name} differs from the eager step"


@pytest.mark.parametrize("fused", [False, True])
def test_step_graph_replays_match_eager(fused):
    inp = make_inputs(300, 256, 256, 8, 2, seed=40)
    print(f"[case] graph replay fused={fused}", flush=True)
    gl = GpuLayer(inp)
    b = gl.b

    def step():
        gl.route()
        if fused:
            moe.moe_forward_fused(gl.dm, gl.x, gl.W1, gl.W2, b["topk_w"], b["offsets"], b["perm"], b["inv_perm"],
                                  b["y"], b["saved"], b["ws_fwd"])
        else:
            gl.forward()
        gl.backward(with_logits=True)

    step()
    torch.cuda.synchronize()
    ref = _snapshot(gl)

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
        _poison(gl)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _check(gl, ref, f"replay {rep}")
        # eager work between replays: the same step, checked too
        _poison(gl)
        step()
        torch.cuda.synchronize()
        _check(gl, ref, f"eager step after replay {rep}")
