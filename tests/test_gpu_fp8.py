"""GPU parity of the blockwise-fp8 path (OCP e4m3 operands with fp32 scales per 1x128 block of
activations and per 128x128 block of weights, bf16 outputs) against the plain fp64 oracle run on
the exactly dequantised inputs and the bf16 dy, for every output including the weight gradients
(the layer runs those in bf16 on x dequantised to bf16).

Inputs are one rank's share of an expert-parallel layer, already routed (expert id -1 marks a
slot that another rank serves).  Small cases compare every output element; the DeepSeek-V3
shaped share (32 local experts of 256, d=7168, f=2048, top-8) is compared on sampled rows and
weight-gradient entries that the oracle computes one by one."""
from collections import OrderedDict

import numpy as np
import pytest
import torch

import oracle
from workloads import make_config, make_prerouted_fp8
from moe_testlib import GpuLayer, TOL_FP8, check_full_parity, oracle_full, rel_err, summarize_errs, to_np

pytestmark = pytest.mark.gpu

CASES = {
    # name: (T_global, E_global, E_local, d, f, k, seed)
    "fp8_small": (256, 16, 4, 256, 256, 4, 21),
    "fp8_multi_tile": (1024, 8, 3, 512, 512, 2, 22),
    "fp8_wide_k": (300, 32, 8, 256, 768, 8, 23),
    "fp8_sparse": (24, 64, 6, 256, 256, 2, 31),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_layer_parity(name):
    Tg, Eg, E, d, f, k, seed = CASES[name]
    inp = make_prerouted_fp8(Tg, Eg, E, d, f, k, seed, name=name)
    counts = np.bincount(inp.topk_ids[inp.topk_ids >= 0], minlength=E)
    print(f"[case] {name} T={inp.T} d={d} f={f} E={E} k={k} counts={counts.tolist()}", flush=True)
    gl = GpuLayer(inp).run()
    errs = check_full_parity(gl, oracle_full(inp), tol=TOL_FP8)
    print(f"[case] {name}: " + ", ".join(f"{k}={v:.2e}" for k, v in summarize_errs(errs).items()), flush=True)


def test_fp8_no_local_tokens():
    # seed 4 routes none of the 24 tokens to this rank's experts: an empty layer
    inp = make_prerouted_fp8(24, 64, 6, 256, 256, 2, 4)
    assert inp.T == 0
    print("[case] fp8 T=0", flush=True)
    gl = GpuLayer(inp)
    gl.b["dW1"].fill_(3.0)
    gl.b["dW2"].fill_(3.0)
    gl.run()
    assert torch.all(gl.b["offsets"] == 0)
    assert torch.all(gl.b["dW1"] == 0) and torch.all(gl.b["dW2"] == 0)


class _DequantExperts:
    """W[e] of blockwise-fp8 expert weights, dequantised exactly to fp64 on first use (a few
    experts are kept), so the sampled checks never hold every expert in fp64 at once."""

    def __init__(self, codes, scales, keep=3):
        self.codes, self.scales, self.keep = codes, scales, keep
        self.shape = codes.shape
        self.cache = OrderedDict()

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = oracle.dequant_blocks_128x128(self.codes[e], self.scales[e])
            if len(self.cache) > self.keep:
                self.cache.popitem(last=False)
        self.cache.move_to_end(e)
        return self.cache[e]


@pytest.mark.slow
def test_fp8_fullsize_dsv3_share():
    inp = make_config("dsv3_fp8")
    ids, w = inp.topk_ids, inp.topk_w.astype(np.float64)
    pl = oracle.plan(ids, inp.E)
    print(f"[case] full-size dsv3_fp8: T={inp.T} d={inp.d} f={inp.f} E={inp.E} k={inp.k} local pairs "
          f"{int(pl.counts.sum())}", flush=True)
    gl = GpuLayer(inp).run()
    r = gl.routing_np()
    assert np.array_equal(r["counts"], pl.counts) and np.array_equal(r["offsets"], pl.offsets)
    assert np.array_equal(r["perm"], pl.perm) and np.array_equal(r["inv_perm"], pl.inv_perm)

    x = oracle.dequant_rows_1x128(inp.x, inp.x_scale)
    dy = oracle.bf16_to_f64(inp.dy)
    W1 = _DequantExperts(inp.W1, inp.W1_scale)
    W2 = _DequantExperts(inp.W2, inp.W2_scale)
    b = gl.b
    g = np.random.default_rng(5)
    # sampled tokens, grouped by their first local expert so the expert cache is reused
    toks = np.unique(np.concatenate([[0, inp.T - 1], g.choice(inp.T, 10, replace=False)]))
    toks = toks[np.argsort([ids[t][ids[t] >= 0][0] for t in toks], kind="stable")]
    y_o = np.stack([oracle.token_forward(x[t], W1, W2, ids[t], w[t]) for t in toks])
    bw = [oracle.token_backward(x[t], W1, W2, ids[t], w[t], dy[t]) for t in toks]
    errs = {"y": rel_err(to_np(b["y"])[toks], y_o),
            "dx": rel_err(to_np(b["dx"])[toks], np.stack([a for a, _ in bw])),
            "d_topk_w": rel_err(to_np(b["d_topk_w"])[toks], np.stack([c for _, c in bw]))}
    # the largest and the smallest expert's weight gradients in full (their whole slices set the
    # error scale)
    for e in (int(np.argmax(pl.counts)), int(np.argmin(pl.counts))):
        r1, r2 = oracle.expert_weight_grads(x, W1, W2, ids, w, dy, e)
        errs[f"dW1[{e}]"] = rel_err(to_np(b["dW1"][e]), r1)
        errs[f"dW2[{e}]"] = rel_err(to_np(b["dW2"][e]), r2)
    # y is linear in the routing weights: sum(dy * y) = sum(w * d_topk_w)
    lhs = float((gl.dy.double() * b["y"].double()).sum())
    mid = float((b["topk_w"].double() * b["d_topk_w"].double()).sum())
    errs["sum(w*dw)"] = abs(mid - lhs) / float(gl.dy.double().abs().mul(b["y"].double().abs()).sum())
    print("[case] dsv3_fp8: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL_FP8}
    assert not bad, bad
