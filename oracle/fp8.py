"""FP8 (E4M3) KV cache for decode, in fp64: the code's value from its bit layout, the
quantizer that stores K/V in it, and attention over such a cache.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
use this module.

Sources: the vLLM other-backends page ("[vLLM] 기타 Attention Backends ..."), "Triton
Attention" section, says an FP8 KV cache is supported there; the RBLN "Attention 모드" page
says naive attention has no FP8 KV cache and that one sparse mode has it. Neither gives the
format or the scaling, so this module states its readings (also in the design notes):
  * format: OCP 8-bit E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent field 0 encodes subnormals m * 2^-9; exponent 15 with mantissa 7 is NaN;
    there is no infinity; the largest finite magnitude is 448;
  * one scale per tensor for K and one for V (fp32, > 0): a stored code c stands for
    value(c) * k_scale (or v_scale);
  * storing x: the code nearest to x / scale, ties to the even code (even mantissa), with
    magnitudes beyond 448 saturated to 448 (NaN stays a NaN code). The quotient x / scale is
    formed in fp32 (IEEE, correctly rounded), the precision the storing kernel uses, so that
    both sides take the rounding decision on the same value;
  * attention over the cache is the plain definition applied to the dequantised K and V.
"""
from __future__ import annotations

import numpy as np

from .naive_attention import attention

E4M3_MAX = 448.0


def e4m3_value(codes) -> np.ndarray:
    """float64 value of each uint8 E4M3 code, from the bit layout."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * m * 2.0 ** -9
    v = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


_ALL = e4m3_value(np.arange(256))
_POS = np.array(sorted(set(float(x) for x in _ALL[:128] if np.isfinite(x))))   # 0 .. 448


def e4m3_quantize(x, scale: float) -> np.ndarray:
    """uint8 codes of x / scale (quotient in fp32): nearest representable value, ties to the
    even mantissa, magnitudes beyond 448 saturated, NaN to a NaN code (0x7F with the sign)."""
    with np.errstate(over="ignore", invalid="ignore"):
        y = (np.asarray(x, dtype=np.float32) / np.float32(scale)).astype(np.float64)
    mag = np.minimum(np.abs(np.nan_to_num(y, nan=0.0)), E4M3_MAX)
    i = np.searchsorted(_POS, mag)                 # _POS[i-1] < mag <= _POS[i]
    i = np.clip(i, 1, len(_POS) - 1)
    lo, hi = _POS[i - 1], _POS[i]
    pick_hi = (mag - lo > hi - mag)
    tie = (mag - lo == hi - mag)
    lo_code = np.searchsorted(_ALL[:127], lo)       # codes 0..126 are increasing
    hi_code = np.searchsorted(_ALL[:127], hi)
    even_hi = (hi_code & 1) == 0
    code = np.where(pick_hi | (tie & even_hi), hi_code, lo_code)
    code = np.where(mag == lo, lo_code, code)
    code = np.where(mag == hi, hi_code, code)
    code = code | np.where(np.signbit(y), 0x80, 0)
    code = np.where(np.isnan(y), 0x7F | np.where(np.signbit(y), 0x80, 0), code)
    return code.astype(np.uint8)


def attention_fp8_kv(q, kv_codes, k_scale: float, v_scale: float, block_table,
                     query_start_loc, seq_lens, scale: float, causal: bool, window: int = 0,
                     rows=None):
    """Attention over an E4M3 cache [2, num_blocks, block_size, num_kv_heads, head_size]
    (uint8 codes): K and V are dequantised (value(code) * scale) and the plain definition
    applied."""
    codes = np.asarray(kv_codes, dtype=np.uint8)
    kv = np.empty(codes.shape, dtype=np.float64)
    kv[0] = e4m3_value(codes[0]) * float(k_scale)
    kv[1] = e4m3_value(codes[1]) * float(v_scale)
    return attention(q, kv, block_table, query_start_loc, seq_lens, scale, causal, window,
                     rows=rows)
