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
