"""GPU checks of the MXFP8 path: the quantisers bit for bit against the oracle's MX quantiser
(same blocks, same exponent rule, same rounding), and the layer against the fp64 oracle run on
the MX-quantised inputs (x and dy in row blocks along d; W1, W2 in blocks along each GEMM's K)."""
import numpy as np
import pytest
import torch

import grouped_gemm_expert_router_amd as moe
import oracle
from workloads import make_inputs
from moe_testlib import GpuLayer, TOL_FP8, bf16_dev, rel_err, to_np, check_routing_bitexact

pytestmark = pytest.mark.gpu


def _values(codes):
    # +0 and -0 are the same value; compare decoded values where codes may differ only in that
    return oracle.e4m3_to_f64(codes)


@pytest.mark.parametrize("shape,axis", [((3, 64, 96), 1), ((2, 96, 64), 0), ((1, 40, 2048), 1), ((4, 256, 80), 0)])
def test_mx_quantize_bitexact(shape, axis):
    g = np.random.default_rng(sum(shape) + axis)
    v = (g.normal(0, 1, shape) * np.exp2(g.integers(-8, 8, shape[:1] + (1, 1)))).astype(np.float32)
    v.reshape(-1)[:40] = 0.0                                  # an all-zero block at the start
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)       # truncation to bf16 is fine: it is the input
    src = bf16_dev(bits)
    codes = torch.empty(shape, dtype=torch.uint8, device="cuda")
    eshape = (shape[0], shape[1], shape[2] // 32) if axis == 1 else (shape[0], shape[1] // 32, shape[2])
    exps = torch.empty(eshape, dtype=torch.uint8, device="cuda")
    print(f"[case] mx quantize {shape} block_axis={axis}", flush=True)
    moe.moe_mxfp8_quantize(src, shape[0], shape[1], shape[2], axis, codes, exps)
    torch.cuda.synchronize()
    rc, re = oracle.mx_quantize(oracle.bf16_to_f64(bits), axis=2 if axis == 1 else 1)
    np.testing.assert_array_equal(exps.cpu().numpy(), re)
    np.testing.assert_array_equal(_values(codes.cpu().numpy()), _values(rc))


@pytest.mark.parametrize("shape", [(2, 64, 512), (2, 64, 1536), (1, 96, 256), (3, 32, 768)])
def test_mx_weight_quantizer_bitexact(shape):
    """The layer's weight quantiser (both orientations from one read) against the oracle's MX
    quantiser along each axis; the row-block exponents come as words by 128-column step."""
    g = np.random.default_rng(sum(shape) + 7)
    v = (g.normal(0, 1, shape) * np.exp2(g.integers(-8, 8, shape[:1] + (1, 1)))).astype(np.float32)
    v[:, :32, :8] = 0.0                                       # all-zero blocks in both orientations
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    src = bf16_dev(bits)
    B, R, C = shape
    cc = torch.empty(shape, dtype=torch.uint8, device="cuda")
    ce = torch.empty((B, R // 32, C), dtype=torch.uint8, device="cuda")
    rcodes = torch.empty(shape, dtype=torch.uint8, device="cuda")
    rw = torch.empty((B, C // 128, R, 4), dtype=torch.uint8, device="cuda")
    print(f"[case] mx weight quantiser {shape}", flush=True)
    moe.moe_mxfp8_quantize_weights(src, B, R, C, cc, ce, rcodes, rw)
    torch.cuda.synchronize()
    x = oracle.bf16_to_f64(bits)
    oc, oe = oracle.mx_quantize(x, axis=1)                   # blocks of 32 rows of a column
    np.testing.assert_array_equal(ce.cpu().numpy(), oe)
    np.testing.assert_array_equal(_values(cc.cpu().numpy()), _values(oc))
    orc, ore = oracle.mx_quantize(x, axis=2)                 # blocks of 32 values of a row
    words = rw.cpu().numpy()                                 # [B, C/128, R, 4]: byte j = block 4t + j
    np.testing.assert_array_equal(words.transpose(0, 2, 1, 3).reshape(B, R, C // 32), ore)
    np.testing.assert_array_equal(_values(rcodes.cpu().numpy()), _values(orc))


def _mx_oracle(inp):
    """fp64 layer on the MX-quantised operands, with the same quantisation points as the GPU
    path except the intermediates (As, dH), which the oracle keeps exact."""
    x = oracle.bf16_to_f64(inp.x)
    W1 = oracle.bf16_to_f64(inp.W1)
    W2 = oracle.bf16_to_f64(inp.W2)
    dy = oracle.bf16_to_f64(inp.dy)
    q = lambda v, ax: oracle.mx_dequantize(*oracle.mx_quantize(v, ax), ax)
    xq, W1f, W2f = q(x, 1), q(W1, 1), q(W2, 1)          # forward: K = d, f
    dyq, W1b, W2b = q(dy, 1), q(W1, 2), q(W2, 2)         # data gradients: K = d, 2f
    ids, w = oracle.route(inp.logits, inp.k)
    y = oracle.forward(xq, W1f, W2f, ids, w)
    # H from the forward's operands; dA from dy and W2 in blocks along d; dX with W1 in blocks
    # along 2f; the weight gradients take x and dy in blocks along the token axis, inside each
    # expert (the layer also quantises As and dH there; the oracle keeps them exact)
    bw = oracle.backward(xq, W1f, W2f, ids, w, dy, W1_dx=W1b, W2_da=W2b, dy_da=dyq, x_dw=x,
                         q_dw=oracle.mx_roundtrip_rows)
    return dict(ids=ids, w=w, plan=bw["plan"], y=y, dx=bw["dx"], d_topk_w=bw["d_topk_w"], d_logits=bw["d_logits"],
                dW1=bw["dW1"], dW2=bw["dW2"])


CASES = {"mx_small": (160, 256, 256, 8, 2, 41), "mx_wide": (300, 512, 768, 6, 3, 42)}


@pytest.mark.parametrize("name", list(CASES))
def test_mx_layer_parity(name):
    T, d, f, E, k, seed = CASES[name]
    inp = make_inputs(T, d, f, E, k, seed=seed)
    print(f"[case] {name} T={T} d={d} f={f} E={E} k={k}", flush=True)
    _check_mx_layer(name, inp)


@pytest.mark.parametrize("T,k", [(2600, 2), (5000, 1)])
def test_mx_heavy_and_empty_experts(T, k):
    """One expert over the 2048-row weight-gradient chunk (its padded segment split in two or
    three fp32 partials summed in chunk order) and two experts with no rows (zero gradients)."""
    E = 8
    bias = np.zeros(E, np.float32)
    bias[1], bias[5], bias[6] = 10.0, -30.0, -30.0
    inp = make_inputs(T, 256, 256, E, k, seed=44, logits_bias=bias)
    print(f"[case] mx heavy/empty experts T={T} k={k}", flush=True)
    gl = _check_mx_layer(f"heavy{T}", inp)
    counts = gl.routing_np()["counts"]
    assert counts[1] > 2048 and counts[5] == 0 and counts[6] == 0
    for e in (5, 6):
        assert torch.all(gl.b["dW1"][e] == 0) and torch.all(gl.b["dW2"][e] == 0)


def _check_mx_layer(name, inp):
    E = inp.E
    gl = GpuLayer(inp, dtype=moe.MOE_MXFP8).run()
    ref = _mx_oracle(inp)
    check_routing_bitexact(gl, ref["ids"], ref["plan"])
    b = gl.b
    errs = {"y": rel_err(to_np(b["y"]), ref["y"]), "dx": rel_err(to_np(b["dx"]), ref["dx"]),
            "d_topk_w": rel_err(to_np(b["d_topk_w"]), ref["d_topk_w"]),
            "d_logits": rel_err(to_np(b["d_logits"]), ref["d_logits"])}
    dW1, dW2 = to_np(b["dW1"]), to_np(b["dW2"])
    for e in range(E):
        if ref["plan"].counts[e]:
            errs[f"dW1[{e}]"] = rel_err(dW1[e], ref["dW1"][e])
            errs[f"dW2[{e}]"] = rel_err(dW2[e], ref["dW2"][e])
    print(f"[case] {name}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items() if not k.startswith("dW")) +
          f", max dW {max(v for k, v in errs.items() if k.startswith('dW')):.2e}", flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL_FP8}
    assert not bad, bad
    return gl


class _MxExperts:
    """W[e] MX-quantised along `axis` of the expert matrix and dequantised to fp64 on first use
    (a few experts kept), so the full-size check never holds every expert in fp64."""

    def __init__(self, Wbits, axis, keep=4):
        from collections import OrderedDict
        self.W, self.axis, self.keep = Wbits, axis, keep
        self.shape = Wbits.shape
        self.cache = OrderedDict()

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            v = oracle.bf16_to_f64(self.W[e])
            self.cache[e] = oracle.mx_dequantize(*oracle.mx_quantize(v, self.axis), self.axis)
            if len(self.cache) > self.keep:
                self.cache.popitem(last=False)
        self.cache.move_to_end(e)
        return self.cache[e]


@pytest.mark.slow
def test_mx_fullsize_qwen3():
    from workloads import make_config
    inp = make_config("qwen3")
    print(f"[case] full-size qwen3 as MXFP8: T={inp.T} d={inp.d} f={inp.f} E={inp.E} k={inp.k}", flush=True)
    gl = GpuLayer(inp, dtype=moe.MOE_MXFP8).run()
    ids, w = oracle.route(inp.logits, inp.k)
    check_routing_bitexact(gl, ids, oracle.plan(ids, inp.E))
    g = np.random.default_rng(7)
    toks = np.unique(np.concatenate([[0, inp.T - 1], g.choice(inp.T, 8, replace=False)]))
    q = lambda v: oracle.mx_dequantize(*oracle.mx_quantize(v, 0), 0)
    W1f, W2f = _MxExperts(inp.W1, 0), _MxExperts(inp.W2, 0)      # blocks along d / f (forward K)
    W1b, W2b = _MxExperts(inp.W1, 1), _MxExperts(inp.W2, 1)      # blocks along 2f / d (data-gradient K)
    b = gl.b
    y_o, dx_o, dw_o = [], [], []
    for t in toks:
        xq = q(oracle.bf16_to_f64(inp.x[t]))
        dyq = q(oracle.bf16_to_f64(inp.dy[t]))
        y_o.append(oracle.token_forward(xq, W1f, W2f, ids[t], w[t]))
        dxt, dwt = oracle.token_backward(xq, W1f, W2f, ids[t], w[t], dyq, W1_dx=W1b, W2_da=W2b, dy_da=dyq)
        dx_o.append(dxt)
        dw_o.append(dwt)
    errs = {"y": rel_err(to_np(b["y"])[toks], np.stack(y_o)), "dx": rel_err(to_np(b["dx"])[toks], np.stack(dx_o)),
            "d_topk_w": rel_err(to_np(b["d_topk_w"])[toks], np.stack(dw_o))}
    # y is linear in the routing weights: sum(dy * y) ~ sum(w * d_topk_w) up to the quantisation of dy
    lhs = float((gl.dy.double() * b["y"].double()).sum())
    mid = float((b["topk_w"].double() * b["d_topk_w"].double()).sum())
    errs["sum(w*dw)"] = abs(mid - lhs) / float(gl.dy.double().abs().mul(b["y"].double().abs()).sum())
    # two experts' weight gradients in full, with token-axis operand blocks
    x = oracle.bf16_to_f64(inp.x)
    xq_all = oracle.mx_dequantize(*oracle.mx_quantize(x, 1), 1)
    dy = oracle.bf16_to_f64(inp.dy)
    dyq_all = oracle.mx_dequantize(*oracle.mx_quantize(dy, 1), 1)
    dW1, dW2 = b["dW1"], b["dW2"]
    for e in (0, inp.E - 1):
        r1, r2 = oracle.expert_weight_grads(xq_all, W1f, W2f, ids, w, dy, e, W2_da=W2b, dy_da=dyq_all, x_dw=x,
                                            q_dw=oracle.mx_roundtrip_rows)
        errs[f"dW1[{e}]"] = rel_err(to_np(dW1[e]), r1)
        errs[f"dW2[{e}]"] = rel_err(to_np(dW2[e]), r2)
    print("[case] qwen3 MXFP8: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL_FP8}
    assert not bad, bad


def test_mx_bitwise_determinism():
    inp = make_inputs(200, 256, 512, 8, 4, seed=43)
    print("[case] mx determinism", flush=True)
    gl = GpuLayer(inp, dtype=moe.MOE_MXFP8).run()
    first = {k: v.clone() for k, v in gl.b.items() if k not in ("ws_route", "ws_fwd", "ws_bwd")}
    gl.run()
    for k, v in first.items():
        a = v.view(torch.uint8) if v.dtype != torch.uint8 else v
        b = gl.b[k].view(torch.uint8) if gl.b[k].dtype != torch.uint8 else gl.b[k]
        assert torch.equal(a, b), k


def test_mx_zero_tokens():
    # no token: every expert's weight gradient is exactly zero and nothing else is touched
    inp = make_inputs(0, 256, 256, 4, 2, seed=45)
    print("[case] mx T=0", flush=True)
    gl = GpuLayer(inp, dtype=moe.MOE_MXFP8)
    gl.b["dW1"].fill_(3.0)
    gl.b["dW2"].fill_(3.0)
    gl.run()
    assert torch.all(gl.b["offsets"] == 0)
    assert torch.all(gl.b["dW1"] == 0) and torch.all(gl.b["dW2"] == 0)
