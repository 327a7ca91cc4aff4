"""Storage-format decoders for the oracle (test infrastructure only).

Decoding is exact: every bf16 and every finite e4m3 value is representable in fp64, and so is
the product of an e4m3 value with an fp32 block scale.
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64.  A bf16 value is the upper half of an fp32 word."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn codes (uint8) -> fp64, from the format's definition.

    Bit 7 is the sign, bits 6..3 the exponent field E (bias 7), bits 2..0 the mantissa M.
    E == 0 encodes the subnormal M/8 * 2^-6; otherwise (1 + M/8) * 2^(E-7).  The single
    pattern E == 15, M == 7 is NaN (there are no infinities)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    mag = np.where(E == 0, (M / 8.0) * 2.0 ** -6, (1.0 + M / 8.0) * np.exp2(E - 7.0))
    mag = np.where((E == 15) & (M == 7), np.nan, mag)
    return s * mag


def dequant_rows_1x128(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """[R, C] e4m3 with one fp32 scale per row per 128 columns -> fp64 [R, C]."""
    R, C = codes.shape
    v = e4m3_to_f64(codes).reshape(R, C // 128, 128)
    return (v * np.asarray(scale, np.float64)[:, :, None]).reshape(R, C)


def dequant_blocks_128x128(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """[..., K, N] e4m3 with one fp32 scale per 128x128 block -> fp64."""
    *lead, K, N = codes.shape
    v = e4m3_to_f64(codes).reshape(*lead, K // 128, 128, N // 128, 128)
    s = np.asarray(scale, np.float64).reshape(*lead, K // 128, 1, N // 128, 1)
    return (v * s).reshape(*lead, K, N)


# ----------------------------------------------------------------------------- MXFP8
# Microscaling (the OCP MX format named on the JAX and TE pages: one shared scale per block of
# 32 consecutive values): elements are e4m3 codes, the shared scale is an E8M0 exponent byte E
# meaning 2^(E - 127) (E = 255 is NaN).

def e8m0_to_f64(e: np.ndarray) -> np.ndarray:
    """E8M0 bytes -> fp64 powers of two 2^(E - 127); 255 decodes to NaN."""
    e = np.asarray(e, dtype=np.uint8).astype(np.int64)
    return np.where(e == 255, np.nan, np.exp2(e - 127.0))


_E4M3_POS = None


def _e4m3_positive_table():
    """The 127 non-negative finite e4m3 values in code order 0x00..0x7E (increasing)."""
    global _E4M3_POS
    if _E4M3_POS is None:
        _E4M3_POS = e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    return _E4M3_POS


def e4m3_encode_rne(v: np.ndarray) -> np.ndarray:
    """fp64 -> e4m3 codes: the nearest finite e4m3 value, ties to the even code (even mantissa),
    magnitudes above 448 saturate to 448, and the sign is kept (-0 for negative values that round
    to zero).  Built from the value table of the format, not from bit manipulation."""
    v = np.asarray(v, dtype=np.float64)
    tab = _e4m3_positive_table()
    a = np.minimum(np.abs(v), tab[-1])
    hi = np.clip(np.searchsorted(tab, a, side="left"), 0, len(tab) - 1)  # first table value >= a
    lo = np.maximum(hi - 1, 0)
    d_hi = tab[hi] - a
    d_lo = a - tab[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def mx_block_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared exponent s of an MX block with absolute maximum amax: the smallest integer with
    amax <= 448 * 2^s (so no element of the block is clipped), limited to [-127, 127]; a block of
    zeros gets s = 0.  Exact: frexp gives floor(log2 amax) and the comparison is exact."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))      # amax = m 2^ex, m in [0.5, 1)
    s = (ex - 1) - 8                                     # 2^(s+8) <= amax < 2^(s+9)
    s = np.where(amax > 448.0 * np.exp2(s.astype(np.float64)), s + 1, s)
    s = np.where(amax > 0, s, 0)
    return np.clip(s, -127, 127).astype(np.int64)


def mx_quantize(v: np.ndarray, axis: int):
    """Blocks of 32 consecutive values along `axis` -> (e4m3 codes shaped like v, E8M0 bytes
    with that axis divided by 32).  Each element is v / 2^s rounded by e4m3_encode_rne."""
    v = np.asarray(v, dtype=np.float64)
    vm = np.moveaxis(v, axis, -1)
    n = vm.shape[-1]
    assert n % 32 == 0, "MX blocks need a multiple of 32 values along the axis"
    blk = vm.reshape(*vm.shape[:-1], n // 32, 32)
    s = mx_block_exponent(np.abs(blk).max(axis=-1))
    codes = e4m3_encode_rne(blk / np.exp2(s.astype(np.float64))[..., None])
    codes = np.moveaxis(codes.reshape(vm.shape), -1, axis)
    scales = np.moveaxis((s + 127).astype(np.uint8), -1, axis)
    return codes, scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, axis: int) -> np.ndarray:
    """Inverse of mx_quantize's encoding: code value times its block's 2^(E - 127), in fp64."""
    c = np.moveaxis(e4m3_to_f64(codes), axis, -1)
    sc = np.moveaxis(e8m0_to_f64(scales), axis, -1)
    out = c.reshape(*c.shape[:-1], c.shape[-1] // 32, 32) * sc[..., None]
    return np.moveaxis(out.reshape(c.shape), -1, axis)


def mx_roundtrip_rows(v: np.ndarray) -> np.ndarray:
    """MX round trip of a matrix in blocks of 32 consecutive rows (axis 0), in fp64.  A last
    partial block is completed with zero rows, which leave its largest magnitude -- and so its
    exponent -- unchanged; the padding is dropped from the result."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[0]
    vp = np.concatenate([v, np.zeros(((-n) % 32,) + v.shape[1:])], axis=0)
    return mx_dequantize(*mx_quantize(vp, 0), 0)[:n]

