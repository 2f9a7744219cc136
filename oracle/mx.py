"""MXFP4 encode/decode, written from the format's definition (oracle; test-only).

The pages fix the storage format of the expert weights as MXFP4 with a block
size of 32 ("MiMo-V2.5-Pro-FP4-DFlash" model card, §2 "FP4 Quantization";
nxbn.cn article, "量化策略的智能选择": store_dtype mxfp4, mxfp4_block_size 32).
MXFP4 is the OCP MX v1.0 format: each element is an FP4 E2M1 number and each
block of 32 consecutive elements shares one E8M0 power-of-two scale.

Readings where the pages are silent:
  * blocks run along the last (reduction, K) axis of each row;
  * byte j of a packed row holds element 2j in bits 3..0 and element 2j+1 in
    bits 7..4;
  * quantisation (pack) is the OCP v1.0 conversion: shared exponent
    floor(log2(amax)) - 2, then each scaled element rounded to the nearest
    E2M1 value with ties to the even code, saturating at 6;
  * an all-zero block gets scale byte 0; a block holding NaN or Inf gets
    scale byte 0xFF (NaN) and all-zero codes;
  * the sign bit of a code is the sign bit of the input element, so -0.0
    and negative values that round to zero give code 0x8.
"""

import numpy as np

BLOCK = 32

# E2M1 magnitudes for codes 0..7 (OCP MX v1.0, FP4 E2M1: 1 sign, 2 exponent,
# 1 mantissa bit, exponent bias 1, no Inf/NaN).
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_value(code):
    """Value of one 4-bit E2M1 code: bit 3 is the sign, bits 2..0 index the
    magnitude list.  Code 0x8 is -0.0."""
    code = int(code)
    if not 0 <= code <= 15:
        raise ValueError("E2M1 code out of range")
    mag = E2M1_MAGNITUDES[code & 7]
    return -mag if code & 8 else mag


def e8m0_value(e):
    """Value of one E8M0 scale byte: 2**(e-127) for e in 0..254, NaN for 255."""
    e = int(e)
    if not 0 <= e <= 255:
        raise ValueError("E8M0 byte out of range")
    if e == 255:
        return float("nan")
    return float(np.ldexp(1.0, e - 127))


def e2m1_table():
    """float64[16]: value of every code."""
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_table():
    """float64[256]: value of every scale byte."""
    return np.array([e8m0_value(e) for e in range(256)], dtype=np.float64)


# ---------------------------------------------------------------------------
# nibble packing (reading: low nibble = even element)

def split_nibbles(codes):
    """uint8[..., K/2] -> uint8[..., K] element codes (element 2j = low nibble)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 0x0F
    out[..., 1::2] = codes >> 4
    return out


def join_nibbles(elem_codes):
    """uint8[..., K] element codes (each 0..15) -> uint8[..., K/2] bytes."""
    elem_codes = np.asarray(elem_codes, dtype=np.uint8)
    if elem_codes.shape[-1] % 2:
        raise ValueError("odd element count")
    return (elem_codes[..., 0::2] | (elem_codes[..., 1::2] << 4)).astype(np.uint8)


# ---------------------------------------------------------------------------
# unpack

def unpack(codes, scales):
    """Exact dequantisation: codes uint8[rows, K/2], scales uint8[rows, K/32]
    -> float64[rows, K], value = E2M1(code) * 2**(e-127).

    The product has at most two significant bits, so it is exact in float64;
    a NaN scale byte (255) makes the whole block NaN."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    rows = codes.shape[:-1]
    K = codes.shape[-1] * 2
    if K % BLOCK or scales.shape != rows + (K // BLOCK,):
        raise ValueError("codes/scales shapes do not describe 32-element blocks")
    vals = e2m1_table()[split_nibbles(codes)]
    s = e8m0_table()[scales]
    blocks = vals.reshape(rows + (K // BLOCK, BLOCK)) * s[..., None]
    return blocks.reshape(rows + (K,))


# ---------------------------------------------------------------------------
# rounding of float64 values to the storage types

def to_f32(v):
    """float64 -> float32 with round-to-nearest-even (IEEE conversion;
    magnitudes beyond fp32's range become Inf)."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float32)


def to_bf16_bits(v):
    """float64 -> bfloat16 bit patterns (uint16), one rounding, RNE.

    bfloat16 has 8 significant bits and fp32's exponent range: normal
    numbers from 2**-126, subnormals with quantum 2**-133, overflow to Inf.
    The value is rounded directly from float64 (no detour through fp32,
    which would round twice)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint16)
    sign = np.signbit(v).astype(np.uint16) << 15
    a = np.abs(v)
    nan = np.isnan(v)
    fin = np.isfinite(v) & (a > 0)
    # exponent of each finite nonzero value: a = f * 2**ex, f in [0.5, 1)
    _, ex = np.frexp(np.where(fin, a, 1.0))
    # quantum = 2**(floor(log2 a) - 7) for normals, 2**-133 below 2**-126
    qexp = np.maximum(ex - 1 - 7, -133)
    n = np.rint(np.ldexp(np.where(fin, a, 0.0), (-qexp).astype(np.int32)))  # exact: n < 2**9; rint is RNE
    r = np.ldexp(n, qexp.astype(np.int32))                                  # rounded magnitude
    # encode r as bf16 bits via float32 (r is exactly representable in bf16,
    # hence in fp32 unless it overflowed to >= 2**128)
    over = fin & (r >= 2.0 ** 128)
    r32 = np.where(fin & ~over, r, 0.0).astype(np.float32)
    bits = (r32.view(np.uint32) >> 16).astype(np.uint16)
    out = np.where(fin & ~over, bits, out)
    out = np.where(over | (np.isinf(v)), np.uint16(0x7F80), out)
    out = (out | sign).astype(np.uint16)
    out = np.where(nan, np.uint16(0x7FC0), out)
    return out.astype(np.uint16)


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns -> exact float64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def unpack_to(codes, scales, dtype):
    """unpack() rounded to the output dtype: 'f32' -> float32 array,
    'bf16' -> uint16 bit patterns."""
    v = unpack(codes, scales)
    if dtype == "f32":
        return to_f32(v)
    if dtype == "bf16":
        return to_bf16_bits(v)
    raise ValueError("dtype must be 'f32' or 'bf16'")


# ---------------------------------------------------------------------------
# pack: the OCP MX v1.0 conversion, block by block

def _nearest_e2m1_code(a):
    """Magnitude code (0..7) of the E2M1 value nearest to a >= 0, ties to
    the even code; anything above 6 is nearest to 6 (saturation)."""
    mags = np.array(E2M1_MAGNITUDES, dtype=np.float64)
    d = np.abs(a[..., None] - mags)            # distance to each magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                            # one or two candidates
    n_cand = cand.sum(axis=-1)
    first = cand.argmax(axis=-1)                # lowest candidate code
    # on a tie between codes c and c+1 take the even one
    tie_pick = np.where(first % 2 == 0, first, first + 1)
    return np.where(n_cand > 1, tie_pick, first).astype(np.uint8)


def pack(v):
    """Quantise float values [rows, K] (K % 32 == 0) to MXFP4.

    Returns (codes uint8[rows, K/2], scales uint8[rows, K/32]).  The input is
    promoted exactly to float64 (fp32 and bf16 inputs are exact there)."""
    v = np.asarray(v, dtype=np.float64)
    if v.ndim != 2 or v.shape[1] % BLOCK:
        raise ValueError("pack expects [rows, K] with K % 32 == 0")
    rows, K = v.shape
    nb = K // BLOCK
    b = v.reshape(rows, nb, BLOCK)
    bad = ~np.isfinite(b).all(axis=-1)          # NaN or Inf anywhere in the block
    bs = np.where(bad[..., None], 0.0, b)
    amax = np.abs(bs).max(axis=-1)
    # floor(log2(amax)) taken exactly from the binary exponent
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.clip(ex - 1 - 2 + 127, 0, 254)       # "-2": E2M1's largest exponent (6 = 1.5*2**2)
    e = np.where(amax > 0, e, 0)
    q = np.ldexp(bs, (127 - e).astype(np.int32)[..., None])      # exact scaling by 2**(127-e)
    mag = _nearest_e2m1_code(np.abs(q))
    sign = np.signbit(bs).astype(np.uint8) << 3
    elem = (mag | sign).astype(np.uint8)
    elem = np.where(bad[..., None], np.uint8(0), elem)
    scales = np.where(bad, 255, e).astype(np.uint8)
    return join_nibbles(elem.reshape(rows, K)), scales
