"""GPU parity of the router front end (through the C ABI) against the fp64 oracle: the gate's
scores logits = x Wg, the routing that the layer then takes from those GPU logits (bit-exact:
the oracle routes the same fp32 array), and the backward through the gate, dWg = x^T d_logits and
the part of dx that flows through the logits, added to the expert path's dx.  The gate's backward
is compared with the oracle's on the layer's own d_logits; the whole input gradient is compared
end to end.

Small cases compare every element; the Qwen3-30B-A3B-shaped layer compares the whole logits and
dWg and sampled dx rows."""
import numpy as np
import pytest
import torch

import grouped_gemm_expert_router_amd as moe
import oracle
from workloads import make_config, make_inputs
from moe_testlib import GpuLayer, TOL_BF16, bf16_dev, check_routing_bitexact, rel_err, to_np

pytestmark = pytest.mark.gpu

CASES = {
    # name: (T, d, f, E, k, seed)
    "router_small": (200, 256, 128, 8, 2, 50),
    # T, E off every tile multiple; E = 100 rows of the gate are not 16-byte aligned
    "router_ragged_E100": (77, 384, 128, 100, 5, 51),
    "router_E128_k8": (1000, 512, 256, 128, 8, 52),
    "router_one_token": (1, 128, 128, 4, 2, 53),
    # the E = 128 / 256 kernels: E = 256 with a ragged token count; fewer tokens than one
    # 64-row block; d = 384 (three 128-column slices of dx); token slices of dWg whose length
    # (224) is not a whole number of 64-token steps
    "router_E256_ragged": (130, 384, 128, 256, 8, 55),
    "router_E128_T33": (33, 256, 128, 128, 4, 56),
    "router_E128_d384": (300, 384, 128, 128, 6, 57),
    "router_E128_T600": (600, 256, 128, 128, 8, 58),
    # one token and d = 128: a single x step, a single 128-column slice of dx, one dWg slice
    "router_E128_one_token": (1, 128, 128, 128, 8, 59),
}


class RouterLayer:
    """A GpuLayer whose logits come from the library's gate product instead of the inputs."""

    def __init__(self, inp):
        self.gl = GpuLayer(inp)
        self.Wg = bf16_dev(inp.Wg)
        self.dm = self.gl.dm
        T, d, E = inp.T, inp.d, inp.E
        self.gl.logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
        self.dWg = torch.full((d, E), 5.0, dtype=torch.bfloat16, device="cuda")
        nb = moe.moe_workspace_bytes(self.dm, moe.MOE_WS_ROUTER)
        self.ws = torch.empty((max(nb, 256),), dtype=torch.uint8, device="cuda")

    def run(self):
        gl = self.gl
        moe.moe_router_logits(self.dm, gl.x, self.Wg, gl.logits)
        gl.route()
        gl.forward()
        gl.backward(with_logits=True)
        self.dx_experts = gl.b["dx"].clone()
        moe.moe_router_backward(self.dm, gl.x, self.Wg, gl.b["d_logits"], gl.b["dx"], self.dWg, self.ws)
        torch.cuda.synchronize()
        return self


@pytest.mark.parametrize("name", list(CASES))
def test_router_front_end_parity(name):
    T, d, f, E, k, seed = CASES[name]
    print(f"[case] {name} T={T} d={d} f={f} E={E} k={k}", flush=True)
    inp = make_inputs(T, d, f, E, k, seed=seed)
    rl = RouterLayer(inp).run()
    gl, b = rl.gl, rl.gl.b
    x = oracle.bf16_to_f64(inp.x)
    Wg = oracle.bf16_to_f64(inp.Wg)
    W1, W2, dy = (oracle.bf16_to_f64(a) for a in (inp.W1, inp.W2, inp.dy))
    logits_gpu = to_np(gl.logits)
    errs = {"logits": rel_err(logits_gpu, oracle.router_logits(x, Wg))}
    # the layer routes the GPU's own fp32 logits; so does the oracle, and the plan must match bit for bit
    ids, w = oracle.route(logits_gpu, k)
    pl = oracle.plan(ids, E)
    check_routing_bitexact(gl, ids, pl)
    # the gate's backward against the oracle's on the layer's own d_logits (whose parity the layer
    # tests check; with one token and two slots d_logits = w0 w1 (dw0 - dw1) can cancel, so its
    # relative error is not the router's)
    dl_gpu = to_np(b["d_logits"]).astype(np.float64)
    dx_r_g, dWg_g = oracle.router_backward(x, Wg, dl_gpu)
    errs["dWg"] = rel_err(to_np(rl.dWg), dWg_g)
    dxr = torch.zeros_like(b["dx"])
    moe.moe_router_backward(rl.dm, gl.x, rl.Wg, b["d_logits"], dxr, None, rl.ws)
    torch.cuda.synchronize()
    errs["dx_router"] = rel_err(to_np(dxr), dx_r_g)
    # end to end: the whole input gradient of the routed layer (expert path + gate path)
    ref = oracle.backward(x, W1, W2, ids, w, dy)
    dx_r, _ = oracle.router_backward(x, Wg, ref["d_logits"])
    errs["dx_experts"] = rel_err(to_np(rl.dx_experts), ref["dx"])
    errs["dx"] = rel_err(to_np(b["dx"]), ref["dx"] + dx_r)
    print(f"[case] {name}: " + ", ".join(f"{n}={v:.2e}" for n, v in errs.items()), flush=True)
    bad = {n: v for n, v in errs.items() if not v <= TOL_BF16}
    assert not bad, bad


def test_router_backward_on_empty_layer_zeroes_dwg():
    inp = make_inputs(0, 128, 128, 8, 2, seed=54)
    print("[case] router T=0", flush=True)
    dm = moe.dims(0, 128, 128, 8, 2)
    Wg = bf16_dev(inp.Wg)
    dWg = torch.full((128, 8), 3.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((max(moe.moe_workspace_bytes(dm, moe.MOE_WS_ROUTER), 256),), dtype=torch.uint8, device="cuda")
    moe.moe_router_logits(dm, None, Wg, None)
    moe.moe_router_backward(dm, None, Wg, None, None, dWg, ws)
    torch.cuda.synchronize()
    assert torch.all(dWg == 0)


@pytest.mark.slow
def test_router_front_end_fullsize_qwen3():
    inp = make_config("qwen3")
    T, d, E, k = inp.T, inp.d, inp.E, inp.k
    print(f"[case] full-size router qwen3: T={T} d={d} E={E} k={k}", flush=True)
    rl = RouterLayer(inp).run()
    gl, b = rl.gl, rl.gl.b
    x = oracle.bf16_to_f64(inp.x)
    Wg = oracle.bf16_to_f64(inp.Wg)
    logits_gpu = to_np(gl.logits)
    errs = {"logits": rel_err(logits_gpu, oracle.router_logits(x, Wg))}
    ids, w = oracle.route(logits_gpu, k)
    check_routing_bitexact(gl, ids, oracle.plan(ids, E))
    # the gate's backward on the layer's own d_logits (their parity is checked by the layer tests)
    dl = to_np(b["d_logits"]).astype(np.float64)
    dx_r, dWg = oracle.router_backward(x, Wg, dl)
    errs["dWg"] = rel_err(to_np(rl.dWg), dWg)
    # the router's part of dx on its own: the same call into a zeroed dx (dWg skipped)
    dxr = torch.zeros((T, d), dtype=torch.bfloat16, device="cuda")
    moe.moe_router_backward(rl.dm, gl.x, rl.Wg, b["d_logits"], dxr, None, rl.ws)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(6).choice(T, 30, replace=False)]))
    errs["dx_router_rows"] = rel_err(to_np(dxr)[toks], dx_r[toks])
    errs["dx_rows"] = rel_err(to_np(b["dx"])[toks], to_np(rl.dx_experts)[toks] + dx_r[toks])
    print("[case] router qwen3: " + ", ".join(f"{n}={v:.2e}" for n, v in errs.items()), flush=True)
    bad = {n: v for n, v in errs.items() if not v <= TOL_BF16}
    assert not bad, bad
