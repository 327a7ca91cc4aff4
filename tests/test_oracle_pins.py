"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test checks the oracle against a library routine, a closed form, a hand-derived fixture,
finite differences or an identity the mathematics fixes, chosen so that a plausible slip in the
oracle (a dropped term, a wrong sign or index, a transposed operand, a lost pair) fails one of
them.  Nothing here re-types the oracle's own formula.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import make_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")
_ENV = {"log": math.log, "exp": math.exp, "s": lambda z: 1.0 / (1.0 + math.exp(-z))}


def _ev(text):
    return [float(eval(t, {"__builtins__": {}}, _ENV)) for t in text.split(",")]


def silu(z):
    return z / (1.0 + np.exp(-z))


def dense_mlp(x, W1e, W2e):
    """Textbook SwiGLU MLP: (silu(x Wg) * (x Wu)) Wd with W1e = [Wg | Wu]."""
    f = W2e.shape[0]
    return (silu(x @ W1e[:, :f]) * (x @ W1e[:, f:])) @ W2e


def rand_layer(T, d, f, E, k, seed, gap=None):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, d))
    W1 = g.standard_normal((E, d, 2 * f)) / np.sqrt(d)
    W2 = g.standard_normal((E, f, d)) / np.sqrt(f)
    L = g.standard_normal((T, E))
    dy = g.standard_normal((T, d))
    return x, W1, W2, L, dy


# ----------------------------------------------------------------------------- routing
def test_route_golden_closed_forms():
    n = 0
    for line in open(os.path.join(GOLD, "topk_softmax.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        k, L, ids, w = [s.strip() for s in line.split("|")]
        ids_o, w_o = oracle.route(np.array([_ev(L)]), int(k))
        assert ids_o[0].tolist() == [int(v) for v in ids.split(",")]
        np.testing.assert_allclose(w_o[0], _ev(w), rtol=0, atol=1e-15)
        n += 1
    assert n >= 5


@pytest.mark.parametrize("seed", range(4))
def test_route_matches_stable_argsort_and_python_sort(seed):
    g = np.random.default_rng(seed)
    T, E = 200, 16
    # tie-heavy: small integer logits, plus signed zeros which compare equal
    L = g.integers(-3, 4, size=(T, E)).astype(np.float32)
    L[g.random((T, E)) < 0.1] = -0.0
    for k in (1, 2, 5, 16):
        ids, w = oracle.route(L, k)
        ref = np.argsort(-L.astype(np.float64), axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref)
        for t in range(0, T, 17):
            py = sorted(range(E), key=lambda e: (-float(L[t, e]), e))[:k]
            assert ids[t].tolist() == py
        assert np.allclose(w.sum(1), 1.0, atol=1e-14)
        assert np.all(np.diff(w, axis=1) <= 1e-15)


def test_route_softmax_equals_renormalised_full_softmax():
    g = np.random.default_rng(7)
    L = g.standard_normal((50, 12)) * 3
    ids, w = oracle.route(L, 4)
    full = np.exp(L - L.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, ids, 1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)


def test_route_brute_force_subsets_tiny():
    g = np.random.default_rng(3)
    E, k = 6, 3
    for _ in range(40):
        L = g.integers(-2, 3, size=(1, E)).astype(np.float64)
        ids, _ = oracle.route(L, k)
        # brute force over every ordered k-tuple: the chosen tuple is the lexicographically
        # smallest sequence of keys (-L[e], e)
        best = min(itertools.permutations(range(E), k), key=lambda tup: [(-L[0, e], e) for e in tup])
        assert tuple(ids[0]) == best


# -------------------------------------------------------------------------------- plan
@pytest.mark.parametrize("seed", range(3))
def test_plan_matches_stable_argsort(seed):
    g = np.random.default_rng(seed)
    T, k, E = 300, 4, 9
    ids = g.integers(-1, E, size=(T, k)).astype(np.int32)
    pl = oracle.plan(ids, E)
    flat = ids.ravel()
    valid = np.flatnonzero(flat >= 0)
    ref = valid[np.argsort(flat[valid], kind="stable")]
    assert np.array_equal(pl.perm, ref)
    assert np.array_equal(pl.counts, np.bincount(flat[valid], minlength=E))
    assert pl.offsets[0] == 0 and pl.offsets[-1] == valid.size
    assert np.array_equal(np.diff(pl.offsets), pl.counts)
    assert np.all(np.diff(flat[pl.perm]) >= 0)
    assert np.array_equal(pl.inv_perm[pl.perm], np.arange(valid.size))
    assert np.all(pl.inv_perm[flat < 0] == -1)


# ----------------------------------------------------------------------------- forward
def test_golden_two_expert_layer():
    vals = {}
    for line in open(os.path.join(GOLD, "moe_2expert.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        key, rhs = line.split("=", 1)
        vals[key.strip()] = np.array(_ev(rhs))
    x = vals["x"].reshape(1, 2)
    W1 = np.stack([vals["W1_0"].reshape(2, 2), vals["W1_1"].reshape(2, 2)])
    W2 = np.stack([vals["W2_0"].reshape(1, 2), vals["W2_1"].reshape(1, 2)])
    ids, w = oracle.route(vals["logits"].reshape(1, 2), 2)
    assert ids[0].tolist() == vals["ids"].astype(int).tolist()
    np.testing.assert_allclose(w[0], vals["w"], atol=1e-15)
    y = oracle.forward(x, W1, W2, ids, w)
    np.testing.assert_allclose(y[0], vals["y"], atol=1e-14)
    b = oracle.backward(x, W1, W2, ids, w, vals["dy"].reshape(1, 2))
    np.testing.assert_allclose(b["d_topk_w"][0], vals["d_topk_w"], atol=1e-14)
    np.testing.assert_allclose(b["d_logits"][0], vals["d_logits"], atol=1e-14)
    np.testing.assert_allclose(b["dx"][0], vals["dx"], atol=1e-14)
    np.testing.assert_allclose(b["dW2"][0].ravel(), vals["dW2_0"], atol=1e-14)
    np.testing.assert_allclose(b["dW2"][1].ravel(), vals["dW2_1"], atol=1e-14)
    np.testing.assert_allclose(b["dW1"][0].ravel(), vals["dW1_0"], atol=1e-14)
    np.testing.assert_allclose(b["dW1"][1].ravel(), vals["dW1_1"], atol=1e-14)


def test_all_tokens_to_one_expert_is_dense_mlp():
    x, W1, W2, L, _ = rand_layer(40, 8, 6, 5, 1, 11)
    L[:, 3] += 100.0                                   # every token's top-1 is expert 3
    ids, w = oracle.route(L, 1)
    assert np.all(ids == 3) and np.allclose(w, 1.0)
    y = oracle.forward(x, W1, W2, ids, w)
    np.testing.assert_allclose(y, dense_mlp(x, W1[3], W2[3]), rtol=1e-12, atol=1e-12)


def test_top1_is_per_token_expert_mlp():
    x, W1, W2, L, _ = rand_layer(60, 8, 6, 5, 1, 12)
    ids, w = oracle.route(L, 1)
    y = oracle.forward(x, W1, W2, ids, w)
    for t in range(60):
        np.testing.assert_allclose(y[t], dense_mlp(x[t:t + 1], W1[ids[t, 0]], W2[ids[t, 0]])[0], atol=1e-12)


@pytest.mark.parametrize("k", [1, 2, 4])
def test_identical_experts_equal_one_mlp(k):
    x, W1, W2, L, _ = rand_layer(30, 8, 6, 4, k, 13)
    W1[:] = W1[0]
    W2[:] = W2[0]
    ids, w = oracle.route(L, k)
    y = oracle.forward(x, W1, W2, ids, w)
    np.testing.assert_allclose(y, dense_mlp(x, W1[0], W2[0]), rtol=1e-12, atol=1e-12)


def test_k_equals_E_is_dense_mixture():
    x, W1, W2, L, _ = rand_layer(25, 8, 6, 4, 4, 14)
    ids, w = oracle.route(L, 4)
    y = oracle.forward(x, W1, W2, ids, w)
    p = np.exp(L - L.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ref = sum(p[:, e:e + 1] * dense_mlp(x, W1[e], W2[e]) for e in range(4))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_forward_per_token_loop_equals_grouped():
    x, W1, W2, L, _ = rand_layer(50, 8, 6, 7, 3, 15)
    ids, w = oracle.route(L, 3)
    ids[5, 1] = -1                                      # a slot routed elsewhere
    y = oracle.forward(x, W1, W2, ids, w)
    for t in range(50):
        ref = sum(w[t, j] * dense_mlp(x[t:t + 1], W1[ids[t, j]], W2[ids[t, j]])[0]
                  for j in range(3) if ids[t, j] >= 0)
        np.testing.assert_allclose(y[t], ref, atol=1e-12)


# ---------------------------------------------------------------------------- backward
def _loss(x, W1, W2, ids, w, dy):
    return float(np.sum(dy * oracle.forward(x, W1, W2, ids, w)))


def _fd_check(fun, theta, grad, coords, rtol=1e-6):
    scale = max(1.0, np.abs(grad).max())
    for c in coords:
        h = 1e-6 * max(1.0, abs(theta.flat[c]))
        old = theta.flat[c]
        theta.flat[c] = old + h
        lp = fun()
        theta.flat[c] = old - h
        lm = fun()
        theta.flat[c] = old
        fd = (lp - lm) / (2 * h)
        assert abs(fd - grad.flat[c]) <= rtol * scale, (c, fd, grad.flat[c])


def test_backward_matches_central_differences():
    T, d, f, E, k = 7, 6, 4, 5, 2
    x, W1, W2, L, dy = rand_layer(T, d, f, E, k, 21)
    ids, w = oracle.route(L, k)
    b = oracle.backward(x, W1, W2, ids, w, dy)
    g = np.random.default_rng(0)
    fun = lambda: _loss(x, W1, W2, ids, w, dy)
    _fd_check(fun, x, b["dx"], g.choice(x.size, 30, replace=False))
    _fd_check(fun, W1, b["dW1"], g.choice(W1.size, 50, replace=False))
    _fd_check(fun, W2, b["dW2"], g.choice(W2.size, 50, replace=False))
    _fd_check(fun, w, b["d_topk_w"], range(w.size))


def test_logit_gradient_matches_central_differences():
    T, d, f, E, k = 6, 5, 3, 6, 3
    x, W1, W2, L, dy = rand_layer(T, d, f, E, k, 22)
    srt = np.sort(L, axis=1)[:, ::-1]
    assert np.all(srt[:, k - 1] - srt[:, k] > 1e-3)     # top-k set stays fixed under h
    ids, w = oracle.route(L, k)
    b = oracle.backward(x, W1, W2, ids, w, dy)

    def fun():
        i2, w2 = oracle.route(L, k)
        assert np.array_equal(i2, ids)
        return _loss(x, W1, W2, i2, w2, dy)

    _fd_check(fun, L, b["d_logits"], range(L.size))


def _routed_layer_loss(x, Wg, W1, W2, dy, k, ids_fixed):
    """L = sum(dy * y) of the layer routed by its own router: logits = x Wg, top-k, softmax."""
    ids, w = oracle.route(oracle.router_logits(x, Wg), k)
    assert np.array_equal(ids, ids_fixed)               # the top-k set stays fixed under h
    return _loss(x, W1, W2, ids, w, dy)


def test_router_gradients_match_central_differences():
    """Central differences of the whole routed layer (router scores -> top-k softmax -> experts)
    with respect to the gate weight and the input: dWg = router_backward's dWg; dx = the expert
    path's dx plus router_backward's dx_router (x reaches the loss through both)."""
    T, d, f, E, k = 7, 6, 4, 6, 2
    x, W1, W2, _, dy = rand_layer(T, d, f, E, k, 25)
    g = np.random.default_rng(3)
    Wg = g.standard_normal((d, E)) / np.sqrt(d)
    L = oracle.router_logits(x, Wg)
    srt = np.sort(L, axis=1)[:, ::-1]
    assert np.all(srt[:, k - 1] - srt[:, k] > 1e-3)
    ids, w = oracle.route(L, k)
    b = oracle.backward(x, W1, W2, ids, w, dy)
    dx_r, dWg = oracle.router_backward(x, Wg, b["d_logits"])
    fun = lambda: _routed_layer_loss(x, Wg, W1, W2, dy, k, ids)
    _fd_check(fun, Wg, dWg, range(Wg.size))
    _fd_check(fun, x, b["dx"] + dx_r, range(x.size))
    # and the expert path alone is not the whole input gradient (the router term is not zero)
    assert np.abs(dx_r).max() > 1e-3 * np.abs(b["dx"]).max()


def test_router_logits_against_per_entry_sums_and_linearity():
    g = np.random.default_rng(4)
    x, Wg = g.standard_normal((9, 5)), g.standard_normal((5, 7))
    L = oracle.router_logits(x, Wg)
    for t, e in [(0, 0), (8, 6), (3, 2), (5, 4)]:
        assert abs(L[t, e] - math.fsum(x[t, i] * Wg[i, e] for i in range(5))) <= 1e-12
    dl = g.standard_normal((9, 7))
    dx_r, dWg = oracle.router_backward(x, Wg, dl)
    assert dx_r.shape == x.shape and dWg.shape == Wg.shape
    # logits are bilinear in (x, Wg): <dWg, Wg> = <dx_r, x> = <d_logits, logits>
    np.testing.assert_allclose(np.sum(dWg * Wg), np.sum(dl * L), rtol=1e-12)
    np.testing.assert_allclose(np.sum(dx_r * x), np.sum(dl * L), rtol=1e-12)


def test_dlogits_rows_sum_to_zero_and_inner_product_identities():
    T, d, f, E, k = 40, 8, 6, 6, 2
    x, W1, W2, L, dy = rand_layer(T, d, f, E, k, 23)
    ids, w = oracle.route(L, k)
    y = oracle.forward(x, W1, W2, ids, w)
    b = oracle.backward(x, W1, W2, ids, w, dy)
    np.testing.assert_allclose(b["d_logits"].sum(1), 0.0, atol=1e-13)
    lhs = np.sum(dy * y)
    np.testing.assert_allclose(np.sum(w * b["d_topk_w"]), lhs, rtol=1e-12)      # y linear in w
    np.testing.assert_allclose(np.sum(W2 * b["dW2"]), lhs, rtol=1e-12)          # y linear in W2
    # off the selected set the logit gradient is exactly zero
    mask = np.ones((T, E), bool)
    mask[np.arange(T)[:, None], ids] = False
    assert np.all(b["d_logits"][mask] == 0.0)


def test_empty_experts_have_exactly_zero_weight_gradients():
    T, d, f, E, k = 30, 6, 4, 8, 2
    x, W1, W2, L, dy = rand_layer(T, d, f, E, k, 24)
    L[:, [2, 5]] -= 100.0
    ids, w = oracle.route(L, k)
    b = oracle.backward(x, W1, W2, ids, w, dy)
    for e in (2, 5):
        assert np.all(b["dW1"][e] == 0.0) and np.all(b["dW2"][e] == 0.0)
    assert np.any(b["dW1"][0] != 0.0)


def test_token_permutation_equivariance():
    T, d, f, E, k = 33, 8, 6, 5, 2
    x, W1, W2, L, dy = rand_layer(T, d, f, E, k, 25)
    ids, w = oracle.route(L, k)
    y = oracle.forward(x, W1, W2, ids, w)
    b = oracle.backward(x, W1, W2, ids, w, dy)
    pi = np.random.default_rng(1).permutation(T)
    ids2, w2 = oracle.route(L[pi], k)
    y2 = oracle.forward(x[pi], W1, W2, ids2, w2)
    b2 = oracle.backward(x[pi], W1, W2, ids2, w2, dy[pi])
    np.testing.assert_allclose(y2, y[pi], atol=1e-12)
    np.testing.assert_allclose(b2["dx"], b["dx"][pi], atol=1e-12)
    np.testing.assert_allclose(b2["d_logits"], b["d_logits"][pi], atol=1e-12)
    np.testing.assert_allclose(b2["dW1"], b["dW1"], atol=1e-12)
    np.testing.assert_allclose(b2["dW2"], b["dW2"], atol=1e-12)


def test_per_entry_forms_agree_with_grouped_oracle():
    T, d, f, E, k = 37, 8, 6, 5, 2
    x, W1, W2, L, dy = rand_layer(T, d, f, E, k, 26)
    ids, w = oracle.route(L, k)
    ids[3, 0] = -1
    y = oracle.forward(x, W1, W2, ids, w)
    b = oracle.backward(x, W1, W2, ids, w, dy)
    for t in (0, 3, 17, 36):
        np.testing.assert_allclose(oracle.token_forward(x[t], W1, W2, ids[t], w[t]), y[t], atol=1e-12)
        dxt, dwt = oracle.token_backward(x[t], W1, W2, ids[t], w[t], dy[t])
        np.testing.assert_allclose(dxt, b["dx"][t], atol=1e-12)
        np.testing.assert_allclose(dwt, b["d_topk_w"][t], atol=1e-12)
    g = np.random.default_rng(2)
    for e in range(E):
        ri, cj = g.integers(0, d, 9), g.integers(0, 2 * f, 9)
        np.testing.assert_allclose(oracle.weight_grad_entries(x, W1, W2, ids, w, dy, e, ri, cj, "dW1"),
                                   b["dW1"][e][ri, cj], atol=1e-12)
        ri, cj = g.integers(0, f, 9), g.integers(0, d, 9)
        np.testing.assert_allclose(oracle.weight_grad_entries(x, W1, W2, ids, w, dy, e, ri, cj, "dW2"),
                                   b["dW2"][e][ri, cj], atol=1e-12)
    ids_r, w_r = oracle.route(L, k)
    b_r = oracle.backward(x, W1, W2, ids_r, w_r, dy)
    np.testing.assert_allclose(oracle.d_logits_from_dw(w_r, b_r["d_topk_w"], ids_r, E), b_r["d_logits"], atol=1e-14)


# ----------------------------------------------------------------------------- formats
def test_bf16_decoder_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.bf16_to_f64(bits)[finite], ref[finite])


def test_e4m3_decoder_special_values_and_torch():
    dec = oracle.e4m3_to_f64(np.array([0x00, 0x80, 0x01, 0x08, 0x38, 0xB8, 0x7E, 0xFE, 0x7F, 0xFF, 0x07], np.uint8))
    exp = [0.0, -0.0, 2.0 ** -9, 2.0 ** -6, 1.0, -1.0, 448.0, -448.0, np.nan, np.nan, 7 * 2.0 ** -9]
    np.testing.assert_array_equal(dec, exp)
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.e4m3_to_f64(codes), ref)


def test_block_dequantisers():
    codes = np.full((2, 256), 0x38, np.uint8)                   # all 1.0
    s = np.array([[2.0, 3.0], [0.5, 1.0]], np.float32)
    v = oracle.dequant_rows_1x128(codes, s)
    assert np.all(v[0, :128] == 2.0) and np.all(v[0, 128:] == 3.0) and np.all(v[1, :128] == 0.5)
    wc = np.full((1, 256, 128), 0x40, np.uint8)                 # all 2.0
    ws = np.array([[[4.0], [0.25]]], np.float32)
    W = oracle.dequant_blocks_128x128(wc, ws)
    assert np.all(W[0, :128] == 8.0) and np.all(W[0, 128:] == 0.5)


def test_oracle_on_generated_bf16_layer_runs_finite():
    inp = make_inputs(64, 128, 256, 8, 2, seed=0)
    x = oracle.bf16_to_f64(inp.x)
    W1 = oracle.bf16_to_f64(inp.W1)
    W2 = oracle.bf16_to_f64(inp.W2)
    ids, w = oracle.route(inp.logits, inp.k)
    y = oracle.forward(x, W1, W2, ids, w)
    assert np.all(np.isfinite(y)) and np.abs(y).max() > 0.1
