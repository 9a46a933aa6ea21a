"""CPU oracle of FP8 expert weights for the Mixtral sparse-MoE layer.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the library never
imports, links or calls it, and it shares no code with the HIP path.

Source: the pages name FP8 weights as the next serving step for Mixtral but fix
no format (paper-graph-ui page, section 3.4, the "TensorRT-LLM integration"
paragraph, and section 6.1, "Mitigation status").  Readings taken here (each
also listed in the design notes):
  * format: OCP 8-bit floating point E4M3 ("fn" variant): 1 sign bit, 4
    exponent bits with bias 7, 3 mantissa bits, subnormals for exponent 0, no
    infinities, S.1111.111 is NaN; largest finite magnitude 448;
  * one fp32 scale per output row of each expert matrix (row f of w1[e] and
    w3[e], row j of w2[e]): scale = amax(|row|) / 448 in fp32, or 1 for an
    all-zero row; code = RNE_e4m3(w / scale), the division in fp32, the
    rounding to nearest with ties to an even mantissa, saturating at 448;
  * the layer with FP8 weights is the plain layer evaluated on the dequantized
    weights decode(code) * scale (fp32 product).

Pins (tests/test_oracle_pins.py): every one of the 256 codes against torch's
float8_e4m3fn, hand values (1, 448, the smallest subnormal, -0, NaN), encoding
against torch's rounding cast inside the finite range, exact midpoints
(ties to even), saturation, and the round-trip error bound of half a quantum.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import moe_layer

F32 = np.float32
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3 code in float64 (NaN for S.1111.111).

    Exponent field E, mantissa field M: E > 0 gives 2^(E-7) * (1 + M/8),
    E = 0 gives the subnormal 2^-6 * (M/8)."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    mag = np.where(E > 0, np.ldexp(1.0 + M / 8.0, E - 7), np.ldexp(M / 8.0, -6))
    mag = np.where((E == 15) & (M == 7), np.nan, mag)
    return sign * mag


def e4m3_encode_rne(v: np.ndarray) -> np.ndarray:
    """E4M3 code of each float32 value, rounded to nearest with ties to an
    even mantissa, magnitudes past 448 saturated to 448.

    For |v| >= 2^-6 the quantum is 2^(e-3) where 2^e <= |v| < 2^(e+1); below
    that it is the subnormal quantum 2^-9.  |v| / quantum is rounded half to
    even and the result re-encoded from its exponent and mantissa."""
    v = np.asarray(v, F32).astype(np.float64)  # exact
    a = np.abs(v)
    neg = np.signbit(v)
    _, e = np.frexp(a)                # a = f * 2^e, 0.5 <= f < 1
    e = e - 1                         # 2^e <= a < 2^(e+1)
    normal = a >= 2.0 ** -6
    qexp = np.where(normal, e - 3, -9)
    n = np.round(np.ldexp(a, -qexp))  # numpy rounds half to even
    r = np.ldexp(n, qexp)             # rounded magnitude
    r = np.minimum(r, E4M3_MAX)
    # encode the rounded magnitude
    _, e2 = np.frexp(r)
    e2 = e2 - 1
    is_norm = r >= 2.0 ** -6
    E = np.where(is_norm, e2 + 7, 0)
    M = np.where(is_norm, np.ldexp(r, -e2) * 8 - 8, np.ldexp(r, 9))
    code = (E.astype(np.int64) << 3) | M.astype(np.int64)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def quantize_rows_fp8(w: np.ndarray):
    """Per-row FP8 quantization of a [..., rows, cols] matrix.

    Returns (codes uint8 of w's shape, scale float32 [..., rows])."""
    w = np.asarray(w, F32)
    amax = np.abs(w).max(axis=-1)
    scale = np.where(amax > 0, amax / F32(E4M3_MAX), F32(1.0)).astype(F32)
    v = (w / scale[..., None]).astype(F32)  # one fp32 division per element
    return e4m3_encode_rne(v), scale


def dequantize_rows_fp8(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """decode(code) * scale, rounded to float32 (decode is exact in fp32)."""
    return (e4m3_decode(codes).astype(F32) * np.asarray(scale, F32)[..., None]).astype(F32)


def moe_layer_fp8(x, wg, q1, s1, q3, s3, q2, s2, K: int = 2) -> dict:
    """The layer with FP8 expert weights: the dense oracle layer on the
    dequantized w1, w3, w2 (router weights stay fp32)."""
    return moe_layer(x, wg, dequantize_rows_fp8(q1, s1), dequantize_rows_fp8(q3, s3),
                     dequantize_rows_fp8(q2, s2), K=K)
