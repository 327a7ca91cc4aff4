"""Pins of the oracle's MXFP8 pieces (OCP microscaling: 32-value blocks, e4m3 elements, E8M0
shared exponents) against the format definition, a library conversion and brute force."""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle


def test_e8m0_decode():
    e = np.array([0, 1, 126, 127, 128, 254, 255], np.uint8)
    got = oracle.e8m0_to_f64(e)
    np.testing.assert_array_equal(got[:-1], [2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0, 2.0 ** 127])
    assert np.isnan(got[-1])


def test_e4m3_encode_matches_torch_conversion():
    # torch's float8_e4m3fn cast rounds to nearest even; compare inside the finite range
    g = np.random.default_rng(0)
    v = np.concatenate([g.normal(0, 1, 20000), g.normal(0, 100, 20000), g.normal(0, 1e-2, 20000),
                        g.uniform(-448, 448, 20000)])
    tab = oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (tab[1:] + tab[:-1]) / 2                      # exact ties between neighbours
    v = np.concatenate([v, mids, -mids, tab, -tab])
    v = v[np.abs(v) <= 448]
    ours = oracle.e4m3_encode_rne(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # ties and table values are exact in fp32 (e4m3 has 3 mantissa bits), so the fp32 cast
    # feeding torch loses nothing
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_encode_roundtrips_every_code_and_saturates():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode_rne(oracle.e4m3_to_f64(codes)), codes)
    assert oracle.e4m3_encode_rne(np.array([1e6]))[0] == 0x7E       # +448
    assert oracle.e4m3_encode_rne(np.array([-500.0]))[0] == 0xFE     # -448


def test_block_exponent_is_smallest_non_clipping_power():
    g = np.random.default_rng(1)
    amax = np.concatenate([np.exp(g.uniform(-20, 20, 2000)), 448.0 * np.exp2(np.arange(-10, 10)),
                           np.nextafter(448.0 * np.exp2(np.arange(-10, 10)), np.inf)])
    s = oracle.mx_block_exponent(amax)
    for a, si in zip(amax, s):
        fa = Fraction(float(a))
        assert fa <= 448 * Fraction(2) ** int(si)            # fits
        assert not fa <= 448 * Fraction(2) ** (int(si) - 1)  # and one power less would not
    assert oracle.mx_block_exponent(np.array([0.0]))[0] == 0


def _brute_force_quantize(v):
    """Per 32-block: s from the definition (math.log2 checked exactly), then each element the
    e4m3 code minimising |v - value(code) 2^s|, ties to the even code."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle.e4m3_to_f64(finite)
    codes = np.zeros(v.shape, np.uint8)
    scales = np.zeros(v.shape[:-1] + (v.shape[-1] // 32,), np.uint8)
    for idx in np.ndindex(v.shape[:-1]):
        for b in range(v.shape[-1] // 32):
            blk = v[idx][32 * b:32 * b + 32]
            a = np.abs(blk).max()
            if a == 0:
                s = 0
            else:
                s = math.ceil(math.log2(a / 448))
                while Fraction(float(a)) > 448 * Fraction(2) ** s:
                    s += 1
                while Fraction(float(a)) <= 448 * Fraction(2) ** (s - 1):
                    s -= 1
            scales[idx + (b,)] = s + 127
            for t, x in enumerate(blk):
                err = np.abs(vals * 2.0 ** s - x)
                best = np.flatnonzero(err == err.min())
                if len(best) > 1:                     # tie: the even code (sign agrees with x)
                    best = [c for c in best if finite[c] % 2 == 0 and (np.signbit(x) == (finite[c] >= 0x80))]
                codes[idx + (32 * b + t,)] = finite[best[0]]
    return codes, scales


def test_mx_quantize_matches_brute_force():
    g = np.random.default_rng(2)
    v = g.normal(0, 1, (3, 64)) * np.exp2(g.integers(-6, 6, (3, 1)))
    v[1, 32:] = 0.0                                     # an all-zero block
    v[2, :32] *= 1e-30                                  # tiny values: scale exponent far below 0
    codes, scales = oracle.mx_quantize(v, axis=1)
    bc, bs = _brute_force_quantize(v)
    np.testing.assert_array_equal(scales, bs)
    # +0 / -0 may differ for elements that round to zero; compare values then
    np.testing.assert_array_equal(oracle.e4m3_to_f64(codes), oracle.e4m3_to_f64(bc))


def test_mx_quantize_axis0_equals_transposed_axis1():
    g = np.random.default_rng(3)
    v = g.normal(0, 1, (64, 48))
    c0, s0 = oracle.mx_quantize(v, axis=0)
    c1, s1 = oracle.mx_quantize(v.T, axis=1)
    np.testing.assert_array_equal(c0, c1.T)
    np.testing.assert_array_equal(s0, s1.T)


def test_mx_roundtrip_of_representable_values_and_error_bound():
    g = np.random.default_rng(4)
    codes = g.integers(0, 0x7F, (4, 96)).astype(np.uint8) | (g.integers(0, 2, (4, 96)) * 0x80).astype(np.uint8)
    codes[:, ::32] = 0x7E                               # every block holds +-448 once: exponent = s
    s = g.integers(-20, 20, (4, 3)).astype(np.int64)
    v = oracle.mx_dequantize(codes, (s + 127).astype(np.uint8), axis=1)
    c2, s2 = oracle.mx_quantize(v, axis=1)
    np.testing.assert_array_equal(s2.astype(np.int64) - 127, s)
    np.testing.assert_array_equal(oracle.e4m3_to_f64(c2), oracle.e4m3_to_f64(codes))
    # arbitrary data: relative error of a normal-range element is at most 2^-4 (3 mantissa bits)
    w = g.normal(0, 1, (8, 256))
    cw, sw = oracle.mx_quantize(w, axis=1)
    back = oracle.mx_dequantize(cw, sw, axis=1)
    big = np.abs(w) >= np.repeat(oracle.e8m0_to_f64(sw), 32, axis=1) * 2.0 ** -6
    assert np.all(np.abs(back - w)[big] <= np.abs(w)[big] * 2.0 ** -4)


def test_backward_with_separate_operand_copies():
    """The optional operand copies reduce to the plain backward when they are the same arrays,
    and each one only enters its own product."""
    g = np.random.default_rng(5)
    T, d, f, E, k = 12, 8, 6, 3, 2
    x, dy = g.normal(size=(T, d)), g.normal(size=(T, d))
    W1, W2 = g.normal(size=(E, d, 2 * f)) / 3, g.normal(size=(E, f, d)) / 3
    L = g.normal(size=(T, E))
    ids, w = oracle.route(L, k)
    base = oracle.backward(x, W1, W2, ids, w, dy)
    same = oracle.backward(x, W1, W2, ids, w, dy, W1_dx=W1, W2_da=W2, dy_da=dy, x_dw=x)
    for key in ("dx", "dW1", "dW2", "d_topk_w", "d_logits"):
        np.testing.assert_array_equal(base[key], same[key])
    # W1_dx enters dx only (linearly): doubling it doubles dx and leaves the rest unchanged
    dbl = oracle.backward(x, W1, W2, ids, w, dy, W1_dx=2 * W1)
    np.testing.assert_allclose(dbl["dx"], 2 * base["dx"], rtol=1e-12, atol=1e-12)
    for key in ("dW1", "dW2", "d_topk_w"):
        np.testing.assert_array_equal(dbl[key], base[key])
    # x_dw enters dW1 only
    dbx = oracle.backward(x, W1, W2, ids, w, dy, x_dw=3 * x)
    np.testing.assert_allclose(dbx["dW1"], 3 * base["dW1"], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(dbx["dx"], base["dx"])
    # dy_da scales da and the routing-weight gradient, not dW2
    dby = oracle.backward(x, W1, W2, ids, w, dy, dy_da=2 * dy)
    np.testing.assert_allclose(dby["d_topk_w"], 2 * base["d_topk_w"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dby["dx"], 2 * base["dx"], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(dby["dW2"], base["dW2"])


def test_token_backward_with_copies_matches_full_backward():
    g = np.random.default_rng(6)
    T, d, f, E, k = 10, 8, 6, 3, 2
    x, dy = g.normal(size=(T, d)), g.normal(size=(T, d))
    W1, W2 = g.normal(size=(E, d, 2 * f)) / 3, g.normal(size=(E, f, d)) / 3
    W1b, W2b, dyb = W1 + g.normal(size=W1.shape) * 0.01, W2 + g.normal(size=W2.shape) * 0.01, dy * 1.1
    ids, w = oracle.route(g.normal(size=(T, E)), k)
    full = oracle.backward(x, W1, W2, ids, w, dy, W1_dx=W1b, W2_da=W2b, dy_da=dyb)
    for t in range(T):
        dxt, dwt = oracle.token_backward(x[t], W1, W2, ids[t], w[t], dy[t], W1_dx=W1b, W2_da=W2b, dy_da=dyb[t])
        np.testing.assert_allclose(dxt, full["dx"][t], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dwt, full["d_topk_w"][t], rtol=1e-12, atol=1e-12)


def _brute_roundtrip_rows(v):
    """Row-block MX round trip by brute force: zero rows complete the last block of 32, each
    column's block is quantised by _brute_force_quantize, then decoded by hand."""
    n = v.shape[0]
    vp = np.concatenate([v, np.zeros(((-n) % 32, v.shape[1]))])
    codes, scales = _brute_force_quantize(vp.T.copy())           # blocks along the (padded) rows
    val = oracle.e4m3_to_f64(codes) * np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=1)
    return val.T[:n]


def test_mx_roundtrip_rows_matches_brute_force():
    g = np.random.default_rng(7)
    v = g.normal(0, 1, (70, 5)) * np.exp2(g.integers(-5, 5, (1, 5)))  # two full blocks and one of 6 rows
    v[32:64, 2] = 0.0                                                 # an all-zero block
    np.testing.assert_array_equal(oracle.mx_roundtrip_rows(v), _brute_roundtrip_rows(v))
    # the zero padding never decides anything: more zero rows give the same real rows
    more = np.concatenate([v, np.zeros((30, 5))])
    np.testing.assert_array_equal(oracle.mx_roundtrip_rows(more)[:70], oracle.mx_roundtrip_rows(v))


def _tiny_layer(seed, T=90, d=8, f=6, E=3, k=1):
    g = np.random.default_rng(seed)
    x, dy = g.normal(size=(T, d)), g.normal(size=(T, d))
    W1, W2 = g.normal(size=(E, d, 2 * f)) / 3, g.normal(size=(E, f, d)) / 3
    L = g.normal(size=(T, E)) + np.array([1.5, 0.0, -0.5])[:E]    # expert 0 gets more than 32 rows
    ids, w = oracle.route(L, k)
    return x, dy, W1, W2, ids, w


def test_backward_q_dw_identity_and_scaling():
    x, dy, W1, W2, ids, w = _tiny_layer(8, k=2)
    base = oracle.backward(x, W1, W2, ids, w, dy)
    same = oracle.backward(x, W1, W2, ids, w, dy, q_dw=lambda v: v)
    for key in ("dW1", "dW2"):                       # As^T dy = a^T (w dy): only the grouping moves
        np.testing.assert_allclose(same[key], base[key], rtol=1e-12, atol=1e-12)
    dbl = oracle.backward(x, W1, W2, ids, w, dy, q_dw=lambda v: 2.0 * v)
    for key in ("dW1", "dW2"):                       # one operand of each product (x, dy) passes through q
        np.testing.assert_allclose(dbl[key], 2.0 * base[key], rtol=1e-12, atol=1e-12)
    for key in ("dx", "d_topk_w", "d_logits"):
        np.testing.assert_array_equal(dbl[key], base[key])


def test_backward_q_dw_one_expert_by_hand():
    """dW2[e] = As^T q(dy) and dW1[e] = q(x)^T dH with row-block MX inputs, rebuilt from per-row
    loops and the brute-force quantiser, in the expert's token order."""
    x, dy, W1, W2, ids, w = _tiny_layer(9)
    f = W2.shape[1]
    out = oracle.backward(x, W1, W2, ids, w, dy, q_dw=oracle.mx_roundtrip_rows)
    for e in range(W1.shape[0]):
        rows = [t for t in range(x.shape[0]) if ids[t, 0] == e]          # k = 1: slot 0, token order
        assert rows, e
        As, dH = [], []
        for t in rows:
            h = x[t] @ W1[e]
            gt, ut = h[:f], h[f:]
            sg = 1.0 / (1.0 + np.exp(-gt))
            As.append(w[t, 0] * gt * sg * ut)
            da = w[t, 0] * (W2[e] @ dy[t])
            dH.append(np.concatenate([da * ut * sg * (1.0 + gt * (1.0 - sg)), da * gt * sg]))
        As, dH = np.array(As), np.array(dH)
        q = _brute_roundtrip_rows
        np.testing.assert_allclose(out["dW2"][e], As.T @ q(dy[rows]), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(out["dW1"][e], q(x[rows]).T @ dH, rtol=1e-12, atol=1e-12)
    assert max(sum(ids[:, 0] == e) for e in range(3)) > 32          # a block boundary was crossed


def test_expert_weight_grads_matches_backward():
    x, dy, W1, W2, ids, w = _tiny_layer(10, k=2)
    for q in (None, oracle.mx_roundtrip_rows):
        full = oracle.backward(x, W1, W2, ids, w, dy, q_dw=q)
        for e in range(W1.shape[0]):
            dW1, dW2 = oracle.expert_weight_grads(x, W1, W2, ids, w, dy, e, q_dw=q)
            np.testing.assert_allclose(dW1, full["dW1"][e], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(dW2, full["dW2"][e], rtol=1e-12, atol=1e-12)



def test_weight_grad_entries_with_q_dw_match_backward():
    x, dy, W1, W2, ids, w = _tiny_layer(12, k=2)
    full = oracle.backward(x, W1, W2, ids, w, dy, q_dw=oracle.mx_roundtrip_rows)
    g = np.random.default_rng(13)
    for e in range(W1.shape[0]):
        ri, cj = g.integers(0, x.shape[1], 12), g.integers(0, 2 * W2.shape[1], 12)
        got = oracle.weight_grad_entries(x, W1, W2, ids, w, dy, e, ri, cj, "dW1", q_dw=oracle.mx_roundtrip_rows)
        np.testing.assert_allclose(got, full["dW1"][e][ri, cj], rtol=1e-12, atol=1e-12)
        ri, cj = g.integers(0, W2.shape[1], 12), g.integers(0, x.shape[1], 12)
        got = oracle.weight_grad_entries(x, W1, W2, ids, w, dy, e, ri, cj, "dW2", q_dw=oracle.mx_roundtrip_rows)
        np.testing.assert_allclose(got, full["dW2"][e][ri, cj], rtol=1e-12, atol=1e-12)
