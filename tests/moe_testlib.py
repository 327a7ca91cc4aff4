"""Shared helpers of the GPU parity tests: move seeded inputs to the device, run the library
through its C ABI, run the oracle, and compare.

The comparison metric for floating-point tensors is max|gpu - oracle| / max|oracle| (per
tensor, and per expert for weight gradients); integer outputs must be bitwise equal.
"""
from __future__ import annotations

import numpy as np
import torch

import grouped_gemm_expert_router_amd as moe
import oracle

TOL_BF16 = 2e-2      # max relative error for bf16 outputs and gradients (fp32 accumulation)
TOL_FP8 = 6e-2       # same for the fp8 path, against the oracle on dequantised values
TOL_TOPK_W = 1e-5    # routing weights are computed in fp32: absolute tolerance


def bf16_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    num = np.abs(gpu - ref).max()
    if den == 0:
        return float(num)
    return float(num / den)


class GpuLayer:
    """Device copies of one layer's inputs plus every buffer the library needs."""

    def __init__(self, inp, device="cuda", backward=True, dtype=None):
        """dtype: the layer's moe dtype; defaults to the inputs' format (bf16 inputs may also
        run as MOE_MXFP8, which quantises them inside the library)."""
        self.inp = inp
        self.fp8 = inp.dtype == "fp8"
        if dtype is None:
            dtype = moe.MOE_FP8_E4M3 if self.fp8 else moe.MOE_BF16
        self.dm = moe.dims(inp.T, inp.d, inp.f, inp.E, inp.k, dtype)
        if self.fp8:
            self.x, self.W1, self.W2 = (torch.from_numpy(np.ascontiguousarray(a)).to(device)
                                        for a in (inp.x, inp.W1, inp.W2))
            self.x_scale, self.W1_scale, self.W2_scale = (torch.from_numpy(np.ascontiguousarray(a)).to(device)
                                                          for a in (inp.x_scale, inp.W1_scale, inp.W2_scale))
        else:
            self.x = bf16_dev(inp.x, device)
            self.W1 = bf16_dev(inp.W1, device)
            self.W2 = bf16_dev(inp.W2, device)
            self.x_scale = self.W1_scale = self.W2_scale = None
        self.dy = bf16_dev(inp.dy, device) if (backward and inp.dy is not None) else None
        self.logits = torch.from_numpy(inp.logits).to(device) if inp.logits is not None else None
        self.b = moe.alloc_layer_buffers(self.dm, device, backward=backward and self.dy is not None)
        if inp.topk_ids is not None:
            self.b["topk_ids"].copy_(torch.from_numpy(inp.topk_ids))
            self.b["topk_w"].copy_(torch.from_numpy(inp.topk_w))

    def route(self):
        b = self.b
        if self.logits is not None:
            moe.moe_route(self.dm, self.logits, b["topk_ids"], b["topk_w"], b["counts"], b["offsets"], b["perm"],
                          b["inv_perm"], b["ws_route"])
        else:
            moe.moe_plan(self.dm, b["topk_ids"], b["counts"], b["offsets"], b["perm"], b["inv_perm"], b["ws_route"])

    def forward(self):
        b = self.b
        moe.moe_forward(self.dm, self.x, self.x_scale, self.W1, self.W1_scale, self.W2, self.W2_scale, b["topk_w"],
                        b["offsets"], b["perm"], b["inv_perm"], b["y"], b["saved"], b["ws_fwd"])

    def backward(self, with_logits=True):
        b = self.b
        moe.moe_backward(self.dm, self.dy, self.x, self.x_scale, self.W1, self.W1_scale, self.W2, self.W2_scale,
                         b["topk_ids"], b["topk_w"],
                         b["offsets"], b["perm"], b["inv_perm"], b["saved"], b["dx"], b["dW1"], b["dW2"],
                         b["d_topk_w"], b["d_logits"] if with_logits else None, b["ws_bwd"])

    def run(self, backward=True):
        self.route()
        self.forward()
        if backward and self.dy is not None:
            self.backward(with_logits=self.logits is not None)
        torch.cuda.synchronize()
        return self

    def routing_np(self):
        b = self.b
        A = int(b["offsets"][-1].item())
        return dict(ids=to_np(b["topk_ids"]), w=to_np(b["topk_w"]), counts=to_np(b["counts"]),
                    offsets=to_np(b["offsets"]), perm=to_np(b["perm"])[:A],
                    inv_perm=to_np(b["inv_perm"])[: self.inp.T * self.inp.k])


def oracle_inputs(inp):
    """fp64 copies of the layer inputs; fp8 operands are dequantised exactly (codes times scales)."""
    if inp.dtype == "fp8":
        x = oracle.dequant_rows_1x128(inp.x, inp.x_scale)
        W1 = oracle.dequant_blocks_128x128(inp.W1, inp.W1_scale)
        W2 = oracle.dequant_blocks_128x128(inp.W2, inp.W2_scale)
    else:
        x = oracle.bf16_to_f64(inp.x)
        W1 = oracle.bf16_to_f64(inp.W1)
        W2 = oracle.bf16_to_f64(inp.W2)
    dy = oracle.bf16_to_f64(inp.dy) if inp.dy is not None else None
    return x, W1, W2, dy


def oracle_full(inp):
    x, W1, W2, dy = oracle_inputs(inp)
    if inp.logits is not None:
        ids, w = oracle.route(inp.logits, inp.k)
    else:
        ids, w = inp.topk_ids, inp.topk_w.astype(np.float64)
    pl = oracle.plan(ids, inp.E)
    out = dict(ids=ids, w=w, plan=pl, y=oracle.forward(x, W1, W2, ids, w))
    if dy is not None:
        out.update(oracle.backward(x, W1, W2, ids, w, dy, logits_routed=inp.logits is not None))
    return out


def summarize_errs(errs: dict) -> dict:
    """Per-tensor maxima of an error dict (the per-expert dW entries folded into dW1, dW2)."""
    out = {}
    for k, v in errs.items():
        name = k.split("[")[0]
        out[name] = max(out.get(name, 0.0), v)
    return out


def check_routing_bitexact(gl: GpuLayer, ref_ids, ref_plan):
    r = gl.routing_np()
    assert np.array_equal(r["ids"], ref_ids), "topk ids differ"
    assert np.array_equal(r["counts"], ref_plan.counts), "counts differ"
    assert np.array_equal(r["offsets"], ref_plan.offsets), "offsets differ"
    assert np.array_equal(r["perm"], ref_plan.perm), "perm differs"
    assert np.array_equal(r["inv_perm"], ref_plan.inv_perm), "inv_perm differs"
    return r


def check_full_parity(gl: GpuLayer, ref, tol=TOL_BF16, backward=True):
    """Element-by-element comparison of every output against the full oracle."""
    r = check_routing_bitexact(gl, ref["ids"], ref["plan"])
    if gl.logits is not None:
        assert np.abs(r["w"] - ref["w"]).max() <= TOL_TOPK_W
    errs = {"y": rel_err(to_np(gl.b["y"]), ref["y"])}
    if backward and gl.dy is not None:
        b = gl.b
        errs["dx"] = rel_err(to_np(b["dx"]), ref["dx"])
        errs["d_topk_w"] = rel_err(to_np(b["d_topk_w"]), ref["d_topk_w"])
        if gl.logits is not None:
            errs["d_logits"] = rel_err(to_np(b["d_logits"]), ref["d_logits"])
        dW1, dW2 = to_np(b["dW1"]), to_np(b["dW2"])
        counts = ref["plan"].counts
        for e in range(gl.inp.E):
            if counts[e] == 0:
                assert np.all(dW1[e] == 0) and np.all(dW2[e] == 0), f"empty expert {e} has nonzero dW"
            else:
                errs[f"dW1[{e}]"] = rel_err(dW1[e], ref["dW1"][e])
                errs[f"dW2[{e}]"] = rel_err(dW2[e], ref["dW2"][e])
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, f"tolerance {tol} exceeded: {bad}"
    return errs
