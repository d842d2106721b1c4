"""Number-format decoders for the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything under ``oracle/``.  The GPU library never does.

Each decoder maps stored bit patterns to exact float64 values, written from the
format's bit-field definition (sign, biased exponent, fraction):

* IEEE 754 binary16 ("fp16"): 1 sign, 5 exponent (bias 15), 10 fraction bits.
* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits (the top half of an
  IEEE binary32).
* OCP 8-bit E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 fraction bits; no
  infinities; only S.1111.111 is NaN; largest finite magnitude 448.
* 8-bit E4M3 "fnuz" ("e4m3fnuz"): the same fields with exponent bias 8; no
  infinities and no negative zero: the one code 1.0000.000 (0x80) is NaN and
  every other code is finite, so the largest magnitude is 240 (0x7F, 0xFF).

The pages name these storage types for the KV cache and queries: fp16/bf16
caches throughout the RocKE ``unified_attention`` README (section "Scenarios"),
and the fp8 e4m3 KV cache with per-tensor scales in AITER PR #3962 (section
"Testing") and the README's section "fp8 KV cache"; the same PR's "Testing"
section tests both fp8 dialects, e4m3fn and e4m3fnuz.
"""

import numpy as np


def _decode_binary(bits, exp_bits, frac_bits, bias, ieee_specials, nan_all_ones_frac_only,
                   nan_negative_zero=False):
    """Decode unsigned integer bit patterns of a binary floating format.

    ``ieee_specials``: an all-ones exponent encodes inf (zero fraction) or NaN.
    ``nan_all_ones_frac_only``: (E4M3FN) only all-ones exponent *and* all-ones
    fraction is NaN; other all-ones-exponent codes are ordinary normals.
    ``nan_negative_zero``: (fnuz formats) the sign-only code is NaN.
    """
    b = np.asarray(bits).astype(np.int64)
    sign = np.where((b >> (exp_bits + frac_bits)) & 1, -1.0, 1.0)
    e = (b >> frac_bits) & ((1 << exp_bits) - 1)
    f = (b & ((1 << frac_bits) - 1)).astype(np.float64)
    emax = (1 << exp_bits) - 1
    # normal: (1 + f/2^p) * 2^(e - bias); subnormal (e == 0): (f/2^p) * 2^(1 - bias)
    normal = (1.0 + f / (1 << frac_bits)) * np.exp2((e - bias).astype(np.float64))
    sub = (f / (1 << frac_bits)) * np.exp2(float(1 - bias))
    mag = np.where(e == 0, sub, normal)
    if ieee_specials:
        mag = np.where(e == emax, np.where(f == 0, np.inf, np.nan), mag)
    if nan_all_ones_frac_only:
        mag = np.where((e == emax) & (f == (1 << frac_bits) - 1), np.nan, mag)
    out = sign * mag
    if nan_negative_zero:
        out = np.where(b == (1 << (exp_bits + frac_bits)), np.nan, out)
    return out


def decode_fp16(bits):
    """binary16 bit patterns (uint16) -> float64."""
    return _decode_binary(bits, 5, 10, 15, True, False)


def decode_bf16(bits):
    """bfloat16 bit patterns (uint16) -> float64."""
    return _decode_binary(bits, 8, 7, 127, True, False)


def decode_e4m3fn(bits):
    """OCP E4M3 (fn: finite, single NaN code per sign) bit patterns (uint8) -> float64."""
    return _decode_binary(bits, 4, 3, 7, False, True)


def decode_e4m3fnuz(bits):
    """E4M3 fnuz (bias 8, no inf, no -0, NaN = 0x80) bit patterns (uint8) -> float64."""
    return _decode_binary(bits, 4, 3, 8, False, False, nan_negative_zero=True)


_DECODERS = {"f16": decode_fp16, "bf16": decode_bf16, "e4m3fn": decode_e4m3fn,
             "e4m3fnuz": decode_e4m3fnuz}
_BYTE_FORMATS = ("e4m3fn", "e4m3fnuz")

_TABLE_CACHE = {}


def decode(bits, dtype):
    """Decode stored bits of ``dtype`` (a key of ``_DECODERS``) via a full lookup table.

    The table is built once per format by the decoders above (all 2^16 or 2^8 codes).
    """
    if dtype not in _TABLE_CACHE:
        n = 256 if dtype in _BYTE_FORMATS else 65536
        codes = np.arange(n, dtype=np.int64)
        _TABLE_CACHE[dtype] = _DECODERS[dtype](codes)
    table = _TABLE_CACHE[dtype]
    b = np.asarray(bits)
    if dtype in _BYTE_FORMATS:
        idx = b.view(np.uint8) if b.dtype.itemsize == 1 else b.astype(np.uint8)
    else:
        idx = b.view(np.uint16) if b.dtype.itemsize == 2 else b.astype(np.uint16)
    return table[idx]
