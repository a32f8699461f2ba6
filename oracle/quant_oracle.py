"""CPU oracle: a KV pool stored as 8-bit floats (TEST INFRASTRUCTURE ONLY).

The pages name a one-byte KV cache without defining it: [KVF] section
"Use-o" serves Llama-3.1-70B with an fp8 KV-cache dtype, [WHY] "El precio"
counts 1 byte per element for an 8-bit cache, and [WHY] "Lo que esta página
NO cubre" lists cache quantisation as a later topic.  Reading taken here (the
plainest one that the rest supports):

* the element format is FP8 E4M3 in its OCP form ("E4M3FN"): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; subnormals below 2^-6; no
  infinities; S.1111.111 is NaN; the largest finite magnitude is 448;
* one scale per tensor (K and V each): the stored code is the float32 value
  x / scale (division rounded as float32 division is) rounded to the nearest
  E4M3 value, ties to an even mantissa, saturating at +-448; the attended value
  is decode(code) * scale;
* attention itself is unchanged: it runs on the dequantised pools (the cache
  keeps content only, so keys are quantised before any rotation).

Everything is float64 numpy apart from the one float32 division that decides
the code (both sides take that decision in float32).

The pages also count one byte per element for an int8 cache ([WHY] "El
precio", s = 1) without a format.  Reading taken for it: symmetric signed
8-bit integers with one scale per tensor; the code is the float32 quotient
x / scale rounded to the nearest integer, ties to even, clamped to
[-127, 127] (-128 is never written, so the range is symmetric; infinities
clamp, NaN is stored as 0); the attended value is code * scale.
"""

import numpy as np

from .lazy_oracle import append as _append
from .lazy_oracle import decode as _decode
from .lazy_oracle import prefill as _prefill

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_decode(codes):
    """Value of each E4M3 code (uint8 array) as float64: (-1)^s * (1 + m/8) *
    2^(e - 7) for e > 0, (-1)^s * (m/8) * 2^-6 for e == 0, NaN for e == 15 and
    m == 7."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_quantize(x):
    """Nearest E4M3 code of each value of x (float64 holding float32 values),
    ties to an even mantissa, magnitudes above 448 saturating to 448, NaN to
    the code 0x7F.  Returns uint8."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    a = np.where(np.isfinite(a), a, E4M3_MAX + 1.0)  # inf saturates; NaN is coded below
    sign = np.signbit(x).astype(np.int64) << 7
    # exponent of the binade holding a, floored at the subnormal binade
    # (zero takes a stand-in inside the subnormal binade, where it rounds to 0)
    _, ex = np.frexp(np.where(a > 0, a, 2.0 ** -10))  # a = f * 2^ex with f in [0.5, 1)
    e_unb = np.maximum(ex - 1, -6)             # a in [2^e_unb, 2^(e_unb+1)) or subnormal
    step = np.ldexp(1.0, e_unb - 3)            # spacing of the 3-bit mantissa grid there
    k = np.rint(a / step).astype(np.int64)     # multiples of step; rint = ties to even
    # k in 0..16; k == 16 is the next binade's first value, whose code is the
    # same arithmetic: code = (e_unb + 7) * 8 + k - 8 for normals, k for subnormals
    code = np.where(e_unb > -6, (e_unb + 7) * 8 + (k - 8), k)
    code = np.where(a > E4M3_MAX, 0x7E, np.minimum(code, 0x7E))
    code = code | sign
    code = np.where(np.isnan(x), E4M3_NAN, code)
    return code.astype(np.uint8)


def quantize_kv(x, scale):
    """Codes of new K or V rows: the float32 quotient x / scale, quantised."""
    q = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return e4m3_quantize(q.astype(np.float64))


def dequantize(codes, scale):
    """Attended values of stored codes: decode(code) * scale (float64)."""
    return e4m3_decode(codes) * float(np.float32(scale))


def append_fp8(k_codes, v_codes, k_new, v_new, slot_mapping, k_scale, v_scale):
    """Append on an 8-bit pool: quantise the new rows, then the plain append
    ([WHY] "El remedio"; [KVF] "Construa" Passo 1).  Returns new code pools."""
    return _append(k_codes, v_codes, quantize_kv(k_new, k_scale), quantize_kv(v_new, v_scale), slot_mapping)


def decode_fp8(q, q_pos, k_codes, v_codes, block_table, seq_lens, scale, theta, k_scale, v_scale,
               block_fill=None):
    """Deferred-RoPE decode over the dequantised pools."""
    return _decode(q, q_pos, dequantize(k_codes, k_scale), dequantize(v_codes, v_scale), block_table,
                   seq_lens, scale, theta, block_fill=block_fill)


def prefill_fp8(q, cu_q_lens, q_pos_start, k_codes, v_codes, block_table, kv_lens, scale, theta, k_scale,
                v_scale, block_fill=None):
    """Deferred-RoPE prefill over the dequantised pools."""
    return _prefill(q, cu_q_lens, q_pos_start, dequantize(k_codes, k_scale), dequantize(v_codes, v_scale),
                    block_table, kv_lens, scale, theta, block_fill=block_fill)


# ------------------------------------------------------------------ int8 pool
INT8_MAX = 127


def int8_quantize(x):
    """Nearest integer of each value of x (float64 holding float32 values),
    ties to even, clamped to [-127, 127]; NaN to 0.  Returns int8."""
    x = np.asarray(x, dtype=np.float64)
    r = np.rint(np.clip(np.where(np.isnan(x), 0.0, x), -INT8_MAX, INT8_MAX))
    return r.astype(np.int8)


def int8_decode(codes):
    """Value of each int8 code as float64."""
    return np.asarray(codes).view(np.int8).astype(np.float64)


def quantize_kv_int8(x, scale):
    """int8 codes of new K or V rows: the float32 quotient x / scale, quantised."""
    q = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return int8_quantize(q.astype(np.float64))


def dequantize_int8(codes, scale):
    """Attended values of stored int8 codes: code * scale (float64)."""
    return int8_decode(codes) * float(np.float32(scale))


def append_int8(k_codes, v_codes, k_new, v_new, slot_mapping, k_scale, v_scale):
    """Append on an int8 pool: quantise the new rows, then the plain append."""
    return _append(k_codes, v_codes, quantize_kv_int8(k_new, k_scale), quantize_kv_int8(v_new, v_scale),
                   slot_mapping)


def decode_int8(q, q_pos, k_codes, v_codes, block_table, seq_lens, scale, theta, k_scale, v_scale,
                block_fill=None):
    """Deferred-RoPE decode over the dequantised int8 pools."""
    return _decode(q, q_pos, dequantize_int8(k_codes, k_scale), dequantize_int8(v_codes, v_scale), block_table,
                   seq_lens, scale, theta, block_fill=block_fill)


def prefill_int8(q, cu_q_lens, q_pos_start, k_codes, v_codes, block_table, kv_lens, scale, theta, k_scale,
                 v_scale, block_fill=None):
    """Deferred-RoPE prefill over the dequantised int8 pools."""
    return _prefill(q, cu_q_lens, q_pos_start, dequantize_int8(k_codes, k_scale),
                    dequantize_int8(v_codes, v_scale), block_table, kv_lens, scale, theta, block_fill=block_fill)
