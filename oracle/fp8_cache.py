"""Plain reference for KV blocks stored as 8-bit floats with a scale per row (test infrastructure).

Only tests/, the smoke check and the CPU-baseline leg of bench.py use this module.

What the pages fix and what is read into them:
  * [BlockManager essay] §3 sizes a quantised cache at fewer bytes per element than fp16,
    and §6.3 stores some blocks as int8. Neither page names a format or a scale
    granularity. The reading taken here: elements are 8-bit floats in the OCP E4M3 format
    (the "FN" variant: sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
    NaN = S.1111.111, largest finite magnitude 448), as defined in the Open Compute Project
    8-bit floating point specification; every (token, kv head) row of a block carries its
    own float32 scale s, so a row is worth code_value * s.
  * Appending a row (the quantised form of [BlockManager essay] §4.4's write into a slot):
    a = max |x| over the row, in float32; s = a / 448 in float32; each element becomes the
    E4M3 code nearest to x / s (float32 quotient, clamped to [-448, 448]), ties to the code
    with an even mantissa. A row of zeros has s = 0 and all codes 0. Every float step here
    is float32 so that the integer decision is taken in the same precision as the library's.
  * Decode over such a cache is the plain decode of paged_attention over the dequantised
    rows code_value * s, in float64.

Pins for every function here live in tests/oracle_pins.py.
"""

from __future__ import annotations

import numpy as np

from .paged_attention import OracleInputError, copy_blocks, paged_decode, paged_decode_window

E4M3_MAX = 448.0
E4M3_NAN_CODE = 0x7F


def e4m3_value(codes) -> np.ndarray:
    """float64 value of each E4M3 code (array of uint8), from the format's definition.

    Exponent field 0 is subnormal: m/8 * 2^(1-7). Otherwise (1 + m/8) * 2^(e-7). The
    all-ones exponent and mantissa (0x7F, 0xFF) is NaN; there is no infinity.
    """
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def _finite_magnitudes() -> np.ndarray:
    """Values of codes 0x00..0x7E: the non-negative finite magnitudes, ascending with the code."""
    return e4m3_value(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even code); |x| must be <= 448.

    The sign bit copies the sign bit of x (so -0.0 gives 0x80). Works by looking the
    magnitude up between the two neighbouring finite magnitudes.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise OracleInputError("e4m3_encode takes finite values within [-448, 448]")
    mags = _finite_magnitudes()
    a = np.abs(x)
    hi = np.searchsorted(mags, a, side="left")  # first magnitude >= a
    hi = np.minimum(hi, len(mags) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == mags[hi], hi, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Codes (uint8, same shape) and float32 scales (shape without the last axis) of rows x."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(s == 0, np.float32(1), s)
    quot = (x / safe[..., None]).astype(np.float32)
    quot = np.clip(quot, -np.float32(E4M3_MAX), np.float32(E4M3_MAX))
    codes = e4m3_encode(quot)
    codes = np.where((s == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes, s


def dequantize(codes, scales) -> np.ndarray:
    """float64 rows code_value * scale (exact: a 4-bit significand times a float32)."""
    return e4m3_value(codes) * np.asarray(scales, np.float64)[..., None]


def reshape_and_cache_fp8(k_codes, v_codes, k_scale, v_scale, key, value, slot_mapping):
    """Quantise and append tokens; returns updated copies of the code and scale pools.

    Token i's rows key[i][h], value[i][h] are quantised one (token, kv head) row at a time
    and land in block slot // block_size at offset slot % block_size, scale included. A
    negative slot is padding and skipped; a slot beyond the pool raises.
    """
    kc, vc = k_codes.copy(), v_codes.copy()
    ks, vs = k_scale.copy(), v_scale.copy()
    num_blocks, _, block_size, _ = k_codes.shape
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), block_size)
        if blk >= num_blocks:
            raise OracleInputError(f"slot {slot} outside a pool of {num_blocks} x {block_size}")
        ck, sk = quantize_rows(key[i])
        cv, sv = quantize_rows(value[i])
        kc[blk, :, off, :] = ck
        vc[blk, :, off, :] = cv
        ks[blk, :, off] = sk
        vs[blk, :, off] = sv
    return kc, vc, ks, vs


def copy_blocks_fp8(k_codes, v_codes, k_scale, v_scale, pairs):
    """Copy-on-write of quantised blocks: codes and their scales move together."""
    kc, vc = copy_blocks(k_codes, v_codes, pairs)
    ks, vs = copy_blocks(k_scale, v_scale, pairs)
    return kc, vc, ks, vs


def paged_decode_fp8(q, k_codes, v_codes, k_scale, v_scale, block_table, context_lens, scale,
                     window: int = 0) -> np.ndarray:
    """Decode over a quantised cache: dequantise every row, then the float64 decode."""
    kf = dequantize(k_codes, k_scale)
    vf = dequantize(v_codes, v_scale)
    if window > 0:
        return paged_decode_window(q, kf, vf, block_table, context_lens, scale, window)
    return paged_decode(q, kf, vf, block_table, context_lens, scale)
