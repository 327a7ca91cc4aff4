"""Full-size GPU parity on the benchmark workloads (Qwen3-30B-A3B, skewed-routing and
Mixtral-8x7B shapes), in the same launch configuration bench.py times.

Routing and the plan are compared bit for bit with the oracle on the full inputs.  Float outputs
are compared on sampled rows and entries that the oracle computes one by one (per-token forward
and backward, single weight-gradient entries), on whole weight-gradient slices of selected
experts (computed from those experts' rows only), plus identities that hold at any size: empty
experts get exactly zero weight gradients, and sum(dy*y) = sum(w*d_topk_w) = sum(W2*dW2)."""
import numpy as np
import pytest
import torch

import oracle
from workloads import make_config
from moe_testlib import GpuLayer, TOL_BF16, TOL_TOPK_W, check_routing_bitexact, rel_err, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _sample_tokens(T, n, seed):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], g.choice(T, n, replace=False)]))


@pytest.mark.parametrize("name", ["qwen3", "skewed", "mixtral"])
def test_fullsize_parity(name):
    inp = make_config(name)
    print(f"[case] full-size {name}: T={inp.T} d={inp.d} f={inp.f} E={inp.E} k={inp.k}", flush=True)
    gl = GpuLayer(inp).run()
    ids, w = oracle.route(inp.logits, inp.k)
    pl = oracle.plan(ids, inp.E)
    r = check_routing_bitexact(gl, ids, pl)
    assert np.abs(r["w"] - w).max() <= TOL_TOPK_W
    print(f"[case] {name}: routing/plan bit-exact; counts min {pl.counts.min()} max {pl.counts.max()}", flush=True)

    x32 = (inp.x.astype(np.uint32) << 16).view(np.float32)
    dy32 = (inp.dy.astype(np.uint32) << 16).view(np.float32)
    W1 = (inp.W1.astype(np.uint32) << 16).view(np.float32)
    W2 = (inp.W2.astype(np.uint32) << 16).view(np.float32)
    wr = w  # fp64 routing weights of the oracle

    b = gl.b
    toks = _sample_tokens(inp.T, 12 if name == "mixtral" else 48, 1)
    y_g, dx_g = to_np(b["y"])[toks], to_np(b["dx"])[toks]
    dtw_g, dl_g = to_np(b["d_topk_w"])[toks], to_np(b["d_logits"])[toks]
    y_o = np.stack([oracle.token_forward(x32[t].astype(np.float64), W1, W2, ids[t], wr[t]) for t in toks])
    bw = [oracle.token_backward(x32[t].astype(np.float64), W1, W2, ids[t], wr[t], dy32[t].astype(np.float64))
          for t in toks]
    dx_o = np.stack([a for a, _ in bw])
    dtw_o = np.stack([c for _, c in bw])
    dl_o = oracle.d_logits_from_dw(wr[toks], dtw_o, ids[toks], inp.E)
    errs = {"y": rel_err(y_g, y_o), "dx": rel_err(dx_g, dx_o), "d_topk_w": rel_err(dtw_g, dtw_o),
            "d_logits": rel_err(dl_g, dl_o)}

    dW1_g, dW2_g = b["dW1"], b["dW2"]
    g = np.random.default_rng(2)
    experts = np.unique(np.concatenate([[int(np.argmax(pl.counts))], np.flatnonzero(pl.counts)[:: max(1, inp.E // 6)]]))
    for e in experts:
        ri, cj = g.integers(0, inp.d, 48), g.integers(0, 2 * inp.f, 48)
        ref = oracle.weight_grad_entries(x32, W1, W2, ids, wr, dy32, e, ri, cj, "dW1")
        got = dW1_g[e][torch.from_numpy(ri).cuda(), torch.from_numpy(cj).cuda()].float().cpu().numpy()
        errs[f"dW1[{e}]"] = rel_err(got, ref)
        ri, cj = g.integers(0, inp.f, 48), g.integers(0, inp.d, 48)
        ref = oracle.weight_grad_entries(x32, W1, W2, ids, wr, dy32, e, ri, cj, "dW2")
        got = dW2_g[e][torch.from_numpy(ri).cuda(), torch.from_numpy(cj).cuda()].float().cpu().numpy()
        errs[f"dW2[{e}]"] = rel_err(got, ref)
    for e in np.flatnonzero(pl.counts == 0):
        assert not torch.any(dW1_g[e] != 0) and not torch.any(dW2_g[e] != 0), f"empty expert {e}"
    # whole weight-gradient slices, element by element, of the smallest routed expert and (where
    # its rows are few enough for the fp64 oracle: the Qwen3 shape) of the largest
    whole = [int(np.flatnonzero(pl.counts)[np.argmin(pl.counts[pl.counts > 0])])]
    if name == "qwen3":
        whole.append(int(np.argmax(pl.counts)))
    if name != "mixtral":
        for e in whole:
            r1, r2 = oracle.expert_weight_grads(x32, W1, W2, ids, wr, dy32, e)
            errs[f"dW1[{e}] whole"] = rel_err(to_np(dW1_g[e]), r1)
            errs[f"dW2[{e}] whole"] = rel_err(to_np(dW2_g[e]), r2)

    # sum(dy*y) = sum(w*dw) = sum(W2*dW2): y is linear in the routing weights and in W2
    lhs = float((gl.dy.double() * b["y"].double()).sum())
    mid = float((b["topk_w"].double() * b["d_topk_w"].double()).sum())
    rhs = float((gl.W2.double() * dW2_g.double()).sum())
    scale = float(gl.dy.double().abs().mul(b["y"].double().abs()).sum())
    errs["sum(w*dw)"] = abs(mid - lhs) / scale
    errs["sum(W2*dW2)"] = abs(rhs - lhs) / scale
    print(f"[case] {name}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL_BF16}
    assert not bad, bad


def test_fullsize_skewed_bitwise_determinism():
    """Two runs of the skewed full-size layer give bitwise-identical outputs.  Its heaviest experts
    hold far more rows than one weight-gradient chunk (2048), so their dW1/dW2 come from fp32
    split-K partials summed in chunk order by the reduce kernel."""
    inp = make_config("skewed")
    counts = np.bincount(oracle.route(inp.logits, inp.k)[0].ravel(), minlength=inp.E)
    assert counts.max() > 2 * 2048, "the split-K path must be engaged"
    print(f"[case] full-size skewed determinism: max rows per expert {counts.max()}", flush=True)
    gl = GpuLayer(inp).run()
    keep = ("topk_ids", "topk_w", "counts", "offsets", "perm", "inv_perm", "y", "saved", "dx", "dW1", "dW2",
            "d_topk_w", "d_logits")
    first = {name: gl.b[name].clone() for name in keep}
    gl.run()
    for name in keep:
        a, b = first[name], gl.b[name]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{name} differs between two runs"
