"""Number formats used by the layer: bf16 rounding, MXFP8 (E4M3FN), MXFP4
(E2M1) elements and E8M0 block scales.  TEST INFRASTRUCTURE ONLY (see the
package docstring).

Where the formats come from:

* bf16 is the layer's storage type (Hy3 295B MoE on Atlas A3 page, section 1:
  BF16 deployment).
* MXFP8 activations: the Qwen3-MoE low-latency page, prefill section "MoE EP
  optimisation -> compute decomposition (AllGather scheme, W4A8)" quantises
  hidden_states dynamically to MXFP8 data plus a scale tensor, and its fused
  operator section names round_mode 'rint' and dst_type float8_e4m3fn.
* MXFP4 weights: the same page's overview (W4A8 mixed precision on Atlas 950).

The pages give the element type and the rounding mode but not the block
size or the scale-exponent rule.  Reading taken (plainest one consistent with
"MX"): blocks of 32 along the reduction dimension, one E8M0 scale per block,
shared exponent = floor(log2(amax)) - emax_elem (emax_elem = 8 for E4M3,
2 for E2M1) clamped to [-127, 127]; elements are the block values divided by
the scale, rounded to nearest-even, saturated to the largest finite element
(448 for E4M3, 6 for E2M1).  A value that rounds to zero keeps its sign bit.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64

# ---------------------------------------------------------------- bf16 -----

def bf16_round(a) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), returned as
    fp64.  bf16 = 1 sign, 8 exponent (bias 127), 7 stored mantissa bits."""
    a = np.asarray(a, dtype=F64)
    out = np.empty_like(a)
    tiny = np.abs(a) < 2.0 ** -126           # bf16 subnormal range: grid 2^-133
    big = ~tiny
    # normal range: keep 8 significant bits of the fp64 significand.
    bits = a[big].view(np.uint64)
    drop = np.uint64(45)                     # 52 - 7 mantissa bits dropped
    lsb = (bits >> drop) & np.uint64(1)
    bits = bits + (np.uint64((1 << 44) - 1) + lsb)
    bits = bits & ~np.uint64((1 << 45) - 1)
    out[big] = bits.view(F64)
    q = 2.0 ** -133
    out[tiny] = np.round(a[tiny] / q) * q    # np.round is half-to-even
    maxbf = (2.0 - 2.0 ** -7) * 2.0 ** 127
    out[np.abs(out) > maxbf] = np.copysign(np.inf, a[np.abs(out) > maxbf])
    return out


# ------------------------------------------------------------ decoders -----

def e4m3_decode(codes) -> np.ndarray:
    """E4M3FN byte -> value.  Sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0.  Exponent 0 is subnormal (m/8 * 2^-6); the two codes
    with all exponent and mantissa bits set are NaN; there is no infinity."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def e2m1_decode(nibbles) -> np.ndarray:
    """E2M1 4-bit code -> value.  Sign bit 3, exponent bits 2..1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (m * 0.5).  Grid: 0, 0.5, 1, 1.5,
    2, 3, 4, 6 and negatives."""
    c = np.asarray(nibbles, dtype=np.int64) & 15
    s = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * 2.0 ** (e - 1.0))
    return s * mag


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 scale byte -> 2^(code-127); code 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def unpack_fp4(packed, cols: int) -> np.ndarray:
    """[rows, cols/2] bytes -> [rows, cols] nibbles; the low nibble holds the
    even column."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (cols,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def mxfp4_dequant(packed, scales, cols: int) -> np.ndarray:
    """MXFP4 weight [rows, cols] = E2M1 element x E8M0 scale of its 32-block."""
    vals = e2m1_decode(unpack_fp4(packed, cols))
    sc = e8m0_decode(scales)
    return vals * np.repeat(sc, 32, axis=-1)


# ----------------------------------------------------------- quantiser -----

def e4m3_encode_rne(v) -> np.ndarray:
    """Round fp64 values (already divided by their block scale) to E4M3FN,
    nearest-even, saturating at +-448.  Returns codes (uint8)."""
    v = np.asarray(v, dtype=F64)
    a = np.abs(v)
    sign = np.signbit(v).astype(np.int64)
    # quantum of the binade holding a; below 2^-6 the subnormal grid 2^-9
    _, ex = np.frexp(np.where(a > 0, a, 1.0))  # a = f * 2^ex, f in [0.5, 1)
    E = np.maximum(ex - 1, -6)
    quantum = np.exp2(E - 3.0)
    r = np.round(a / quantum) * quantum          # half-to-even; a/quantum exact
    r = np.minimum(r, 448.0)
    # encode r
    _, ex2 = np.frexp(np.where(r > 0, r, 1.0))
    Er = ex2 - 1
    normal = (r >= 2.0 ** -6)
    e_field = np.where(normal, Er + 7, 0)
    m_field = np.where(normal, np.round((r / np.exp2(Er) - 1.0) * 8.0), np.round(r / 2.0 ** -9))
    code = (sign << 7) | (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    return code.astype(np.uint8)


def mx_block_exponent(amax, emax_elem: int) -> np.ndarray:
    """Shared exponent of a block: floor(log2(amax)) - emax_elem, clamped to
    [-127, 127]; an all-zero block gets -127."""
    amax = np.asarray(amax, dtype=F64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.where(amax > 0, (ex - 1) - emax_elem, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def mxfp8_quantize(x, exponents=None) -> tuple:
    """Dynamic MXFP8 quantisation along the last axis (blocks of 32).

    Returns (codes uint8 [..., K], scales uint8 [..., K/32]) where
    scale code = shared exponent + 127 and code = E4M3_RNE_sat(x / 2^exp).
    ``exponents`` ([..., K/32] ints), when given, replaces the shared
    exponents the rule would take from the block maxima: the elements are
    then rounded at those exponents (used where another computation decided
    a block's exponent from its own, rounded values of the same block).
    """
    x = np.asarray(x, dtype=F64)
    K = x.shape[-1]
    assert K % 32 == 0
    blocks = x.reshape(x.shape[:-1] + (K // 32, 32))
    if exponents is None:
        amax = np.abs(blocks).max(axis=-1)
        e = mx_block_exponent(amax, 8)
    else:
        e = np.asarray(exponents, dtype=np.int64)
        assert e.shape == blocks.shape[:-1] and np.all((e >= -127) & (e <= 127))
    q = blocks / np.exp2(e.astype(F64))[..., None]
    codes = e4m3_encode_rne(q).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def mxfp8_dequant(codes, scales) -> np.ndarray:
    vals = e4m3_decode(codes)
    return vals * np.repeat(e8m0_decode(scales), 32, axis=-1)
