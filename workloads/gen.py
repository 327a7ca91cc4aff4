"""Seeded synthetic workloads for the dropless MoE layer.

Shapes follow the four page sources' workloads (a Qwen3-30B-A3B-shaped layer with 128
experts and top-8 over a 16 384-token sequence, a Mixtral-8x7B-shaped layer with 8 experts
and top-2, a DeepSeek-V3-shaped expert-parallel share in blockwise fp8, plus a tiny sanity
layer).  No model weights exist here: every tensor is drawn from a seeded normal
distribution (std 1/sqrt(fan_in) for weights) and rounded to the storage format.

Random streams are split into fixed 16 Mi-element chunks, each with its own
``numpy.random.default_rng((seed, tensor_id, chunk))`` generator, so the values do not depend
on the number of worker threads that fill them.

Formats handed out:
  * bf16 tensors as ``uint16`` bit patterns (round to nearest even from fp32);
  * fp8 tensors as ``uint8`` OCP e4m3fn codes (round to nearest even, saturating at 448)
    with fp32 scales: activations per 1x128 block along the row, weights per 128x128 block;
  * router logits as fp32, computed once here (x @ Wg in fp32) so every consumer reads the
    identical array.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_CHUNK = 1 << 24

# Workload table.  T, d, f, E, k as in the layer's notation (tokens, model dim, expert FFN dim,
# experts, top-k).  "fwd_only" marks the sanity case that is checked in forward only.
CONFIGS = {
    "tiny": dict(T=64, d=128, f=256, E=8, k=2, seed=0, fwd_only=True),
    "mixtral": dict(T=8192, d=4096, f=14336, E=8, k=2, seed=1),
    "qwen3": dict(T=16384, d=2048, f=768, E=128, k=8, seed=2),
    "skewed": dict(T=16384, d=2048, f=768, E=128, k=8, seed=3, skew=3.0),
    # One GPU's expert share of an 8-way expert-parallel DeepSeek-V3-shaped layer: 8 ranks x
    # 4096 tokens each route top-8 over 256 experts; this GPU owns experts 0..31 and receives
    # each token with at least one local slot exactly once.
    "dsv3_fp8": dict(T_global=8 * 4096, E_global=256, E=32, d=7168, f=2048, k=8, seed=4, fp8=True),
}


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_chunks(n: int, fn) -> None:
    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            fn(c)
        return
    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(fn, range(nchunks)))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _normal_bf16(shape, seed: int, tid: int, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.default_rng((seed, tid, c))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[lo:hi] = bf16_bits_from_f32(v)

    _fill_chunks(n, fill)
    return out.reshape(shape)


def _normal_f32(shape, seed: int, tid: int, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.default_rng((seed, tid, c))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[lo:hi] = v

    _fill_chunks(n, fill)
    return out.reshape(shape)


def _bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------------------------
# OCP 8-bit float e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no infinities,
# S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448 and the smallest
# subnormal is 2^-9.
# ---------------------------------------------------------------------------------------------
def e4m3_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> e4m3fn codes, round to nearest even, saturating to +-448 (inputs finite)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    mag = np.abs(a)
    sign = np.signbit(a).astype(np.uint8) << np.uint8(7)
    code = np.zeros(a.shape, dtype=np.int32)
    # subnormal range |v| < 2^-6: code = RNE(|v| / 2^-9), which is 0..8 (8 is the smallest normal)
    sub = mag < np.float32(2.0 ** -6)
    code[sub] = np.rint(mag[sub] * np.float32(512.0)).astype(np.int32)
    # normal range: round the fp32 significand to 3 bits (RNE) and rebias the exponent
    nrm = ~sub
    u = mag[nrm].view(np.uint32)
    u = (u + np.uint32(0x7FFFF) + ((u >> np.uint32(20)) & np.uint32(1))) & np.uint32(0xFFF00000)
    e = (u >> np.uint32(23)).astype(np.int32) - 127
    m = ((u >> np.uint32(20)) & np.uint32(7)).astype(np.int32)
    c = ((e + 7) << 3) | m
    code[nrm] = np.minimum(c, 126)  # saturate: 0x7E is 448
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_rows_1x128(v: np.ndarray):
    """Activations [R, C] -> (e4m3 codes [R, C], fp32 scales [R, C/128]); scale = amax/448 (1 if 0)."""
    R, C = v.shape
    assert C % 128 == 0
    blk = v.reshape(R, C // 128, 128)
    amax = np.abs(blk).max(axis=2)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = e4m3_bits_from_f32(blk / s[:, :, None]).reshape(R, C)
    return q, s


def quantize_blocks_128x128(w: np.ndarray):
    """Weights [K, N] -> (e4m3 codes [K, N], fp32 scales [K/128, N/128]) per 128x128 block."""
    K, N = w.shape
    assert K % 128 == 0 and N % 128 == 0
    blk = w.reshape(K // 128, 128, N // 128, 128)
    amax = np.abs(blk).max(axis=(1, 3))
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = e4m3_bits_from_f32(blk / s[:, None, :, None]).reshape(K, N)
    return q, s


@dataclass
class MoEInputs:
    """One layer's inputs.  bf16 tensors are uint16 bit patterns, fp8 tensors uint8 e4m3 codes."""
    name: str
    T: int
    d: int
    f: int
    E: int
    k: int
    dtype: str                      # "bf16" or "fp8"
    x: np.ndarray                   # [T, d]
    W1: np.ndarray                  # [E, d, 2f]   columns [0,f) gate, [f,2f) up
    W2: np.ndarray                  # [E, f, d]
    dy: Optional[np.ndarray]        # [T, d] bf16 upstream gradient
    logits: Optional[np.ndarray] = None     # [T, E] fp32 router logits (routed configs)
    Wg: Optional[np.ndarray] = None         # [d, E] bf16 gate weight: the same draw that made the
                                            # logits, rounded to bf16 (input of the router front end)
    topk_ids: Optional[np.ndarray] = None   # [T, k] int32, -1 = slot owned by another rank
    topk_w: Optional[np.ndarray] = None     # [T, k] fp32 routing weights (pre-routed configs)
    x_scale: Optional[np.ndarray] = None    # fp8: [T, d/128]
    W1_scale: Optional[np.ndarray] = None   # fp8: [E, d/128, 2f/128]
    W2_scale: Optional[np.ndarray] = None   # fp8: [E, f/128, d/128]
    meta: dict = field(default_factory=dict)


def make_inputs(T: int, d: int, f: int, E: int, k: int, seed: int = 0, *, skew: float = 0.0,
                with_dy: bool = True, name: str = "custom", logits_bias: Optional[np.ndarray] = None,
                identical_experts: bool = False) -> MoEInputs:
    """bf16 layer with router logits = x @ Wg (+ bias).  Distribution recipe:
    x ~ N(0,1); W1 ~ N(0, 1/d); W2 ~ N(0, 1/f); Wg ~ N(0, 1/d) in fp32; dy ~ N(0,1).
    The fp32 logits are computed here from the fp32 Wg; Wg is also handed out rounded to bf16
    for the router front end, which computes its own logits from it.
    skew > 0 adds b_e = skew * ln(1/rank_e) for a seeded random ranking 1..E of the experts."""
    x = _normal_bf16((T, d), seed, 1, 1.0)
    if identical_experts:
        w1 = _normal_bf16((1, d, 2 * f), seed, 2, float(1.0 / np.sqrt(d)))
        w2 = _normal_bf16((1, f, d), seed, 3, float(1.0 / np.sqrt(f)))
        W1 = np.ascontiguousarray(np.broadcast_to(w1, (E, d, 2 * f)))
        W2 = np.ascontiguousarray(np.broadcast_to(w2, (E, f, d)))
    else:
        W1 = _normal_bf16((E, d, 2 * f), seed, 2, float(1.0 / np.sqrt(d)))
        W2 = _normal_bf16((E, f, d), seed, 3, float(1.0 / np.sqrt(f)))
    Wg = _normal_f32((d, E), seed, 4, float(1.0 / np.sqrt(d)))
    logits = (_bf16_bits_to_f32(x) @ Wg).astype(np.float32)
    meta = {}
    if skew:
        rank = np.random.default_rng((seed, 5)).permutation(E) + 1
        b = (np.float32(skew) * np.log(1.0 / rank)).astype(np.float32)
        logits = (logits + b[None, :]).astype(np.float32)
        meta["expert_rank"] = rank
    if logits_bias is not None:
        logits = (logits + logits_bias.astype(np.float32)).astype(np.float32)
    dy = _normal_bf16((T, d), seed, 6, 1.0) if with_dy else None
    return MoEInputs(name=name, T=T, d=d, f=f, E=E, k=k, dtype="bf16", x=x, W1=W1, W2=W2, dy=dy,
                     logits=np.ascontiguousarray(logits), Wg=bf16_bits_from_f32(Wg), meta=meta)


def make_prerouted_fp8(T_global: int, E_global: int, E: int, d: int, f: int, k: int, seed: int,
                       name: str = "dsv3_fp8") -> MoEInputs:
    """One rank's share of an expert-parallel layer, already routed, in blockwise fp8.

    Each of T_global tokens draws i.i.d. N(0,1) router logits over the E_global experts and
    keeps the k largest (descending; a tie has probability zero), with routing weights the
    softmax over those k logits, so each token's k weights sum to 1.  This rank owns experts
    [0, E); it receives every token with at least one local slot once, and non-local slots
    carry expert id -1.  Activations and weights are drawn in fp32 and quantised to e4m3 (x per
    1x128 block along d, W per 128x128 block); dy is bf16."""
    g = np.random.default_rng((seed, 10))
    logits = g.standard_normal((T_global, E_global), dtype=np.float32)
    choice = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
    top = np.take_along_axis(logits, choice, axis=1).astype(np.float64)
    z = np.exp(top - top[:, :1])
    wts = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    local = choice < E
    recv = np.flatnonzero(local.any(axis=1))
    ids = np.where(local[recv], choice[recv], -1).astype(np.int32)
    w = wts[recv].astype(np.float32)
    T = len(recv)
    xf = _normal_f32((T, d), seed, 1, 1.0)
    xq, xs = quantize_rows_1x128(xf)
    del xf
    W1q = np.empty((E, d, 2 * f), np.uint8)
    W1s = np.empty((E, d // 128, 2 * f // 128), np.float32)
    W2q = np.empty((E, f, d), np.uint8)
    W2s = np.empty((E, f // 128, d // 128), np.float32)
    for e in range(E):
        W1q[e], W1s[e] = quantize_blocks_128x128(_normal_f32((d, 2 * f), seed, 100 + e, float(1.0 / np.sqrt(d))))
        W2q[e], W2s[e] = quantize_blocks_128x128(_normal_f32((f, d), seed, 1000 + e, float(1.0 / np.sqrt(f))))
    dy = _normal_bf16((T, d), seed, 6, 1.0)
    return MoEInputs(name=name, T=T, d=d, f=f, E=E, k=k, dtype="fp8", x=xq, W1=W1q, W2=W2q, dy=dy,
                     topk_ids=ids, topk_w=w, x_scale=xs, W1_scale=W1s, W2_scale=W2s,
                     meta={"T_global": T_global, "E_global": E_global, "recv_tokens": recv})


def make_config(name: str, **overrides) -> MoEInputs:
    """Inputs for a named workload from CONFIGS (keyword overrides replace table fields)."""
    c = dict(CONFIGS[name])
    c.update(overrides)
    if c.get("fp8"):
        return make_prerouted_fp8(c["T_global"], c["E_global"], c["E"], c["d"], c["f"], c["k"], c["seed"],
                                  name=name)
    return make_inputs(c["T"], c["d"], c["f"], c["E"], c["k"], c["seed"], skew=c.get("skew", 0.0),
                       with_dy=not c.get("fwd_only", False), name=name)
