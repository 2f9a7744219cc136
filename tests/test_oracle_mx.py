"""Pins of the oracle's MXFP4 codec against the format's own definition.

Nothing here re-calls the oracle to check itself: values come from the OCP MX
bit-field definition, golden fixtures, exact rational brute force and
round-trip invariants."""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import mx

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def e2m1_from_bits(c):
    """E2M1 from its bit fields: sign | 2-bit exponent (bias 1) | 1-bit mantissa."""
    s, E, M = (c >> 3) & 1, (c >> 1) & 3, c & 1
    if E == 0:                       # subnormal: 2**(1-bias) * (M/2)
        v = 0.5 * M
    else:
        v = 2.0 ** (E - 1) * (1 + M / 2)
    return -v if s else v


def test_block_size_is_the_pages(golden):
    consts = {r[0]: int(r[1]) for r in golden("page_constants.txt")}
    assert mx.BLOCK == consts["mx_block"] == 32


def test_e2m1_against_bitfields_and_golden(golden):
    rows = golden("e2m1_ocp.txt")
    assert len(rows) == 16
    for bits, val in rows:
        c = int(bits, 2)
        v = mx.e2m1_value(c)
        assert v == float(val) == e2m1_from_bits(c)
        assert math.copysign(1.0, v) == math.copysign(1.0, float(val))
    assert math.copysign(1.0, mx.e2m1_value(8)) == -1.0      # code 0x8 is -0.0


def test_e8m0_golden_and_doubling(golden):
    for b, val in golden("e8m0_ocp.txt"):
        v = mx.e8m0_value(int(b))
        if val == "nan":
            assert math.isnan(v)
        else:
            assert v == float(val)
    t = mx.e8m0_table()
    assert np.all(t[1:255] == 2.0 * t[0:254])                 # each step doubles
    assert np.all(t[:255] > 0)


def test_nibble_order_golden(golden):
    for ce, co, byte, ve, vo in golden("nibble_order.txt"):
        ce, co, byte = int(ce, 16), int(co, 16), int(byte, 16)
        packed = mx.join_nibbles(np.array([[ce, co]], np.uint8))
        assert packed[0, 0] == byte
        codes = np.zeros((1, 16), np.uint8)
        codes[0, 0] = byte
        vals = mx.unpack(codes, np.array([[127]], np.uint8))
        assert vals[0, 0] == float(ve) and vals[0, 1] == float(vo)
        assert math.copysign(1, vals[0, 0]) == math.copysign(1, float(ve))
        assert np.all(vals[0, 2:] == 0)


def test_unpack_exhaustive_all_code_scale_pairs():
    # row e holds every code twice (32 elements) with scale byte e
    elem = np.tile(np.arange(16, dtype=np.uint8), 2)
    codes = np.tile(mx.join_nibbles(elem[None, :]), (256, 1))
    scales = np.arange(256, dtype=np.uint8)[:, None]
    vals = mx.unpack(codes, scales)
    for e in range(256):
        for i in range(32):
            want = math.ldexp(e2m1_from_bits(int(elem[i])), e - 127) if e < 255 else math.nan
            got = vals[e, i]
            if e == 255:
                assert math.isnan(got)
            else:
                assert got == want and math.copysign(1, got) == math.copysign(1, want)


def _all_finite_bf16():
    """All finite non-negative bf16 values (sorted), their bit patterns."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return vals, bits


def bf16_brute(x):
    """Exact RNE of a float64 onto bf16 by search over every bf16 value."""
    vals, bits = _all_finite_bf16()
    a = abs(x)
    sgn = 0x8000 if math.copysign(1, x) < 0 else 0
    if math.isnan(x):
        return None
    if math.isinf(x):
        return 0x7F80 | sgn
    i = int(np.searchsorted(vals, a))
    if i < len(vals) and vals[i] == a:
        return int(bits[i]) | sgn
    lo = i - 1
    if i == len(vals):   # above max finite: compare with the next step 2**128
        hi_val, hi_bits = Fraction(2) ** 128, 0x7F80
    else:
        hi_val, hi_bits = Fraction(vals[i]), int(bits[i])
    dlo = Fraction(a) - Fraction(vals[lo])
    dhi = hi_val - Fraction(a)
    if dlo < dhi or (dlo == dhi and bits[lo] % 2 == 0):
        return int(bits[lo]) | sgn
    return hi_bits | sgn


def test_bf16_rounding_against_brute_force():
    rng = np.random.default_rng(7)
    xs = list(rng.standard_normal(400) * np.exp2(rng.integers(-140, 130, 400)))
    # exact midpoints and neighbours, subnormal edge, overflow edge
    xs += [1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -40, -(1 + 2 ** -8),
           2 ** -133, 2 ** -134, 3 * 2 ** -135, 2 ** -135, 2 ** -126 * (1 - 2 ** -9),
           (2 - 2 ** -8) * 2 ** 127, (2 - 2 ** -7) * 2 ** 127, (2 - 2 ** -8 - 2 ** -30) * 2 ** 127,
           0.0, -0.0, math.inf, -math.inf]
    got = mx.to_bf16_bits(np.array(xs))
    for x, g in zip(xs, got):
        assert int(g) == bf16_brute(x), (x, hex(int(g)), hex(bf16_brute(x)))
    assert mx.to_bf16_bits(np.array([math.nan]))[0] & 0x7FFF > 0x7F80


def test_bf16_decode_roundtrip():
    bits = np.arange(0, 1 << 16, dtype=np.uint16)
    vals = mx.bf16_bits_to_f64(bits)
    fin = np.isfinite(vals)
    back = mx.to_bf16_bits(vals[fin])
    assert np.array_equal(back, bits[fin])


# ---------------------------------------------------------------------------
# pack


def pack_brute(block):
    """OCP MX v1.0 conversion of one 32-block by exact rational search."""
    vals = [float(v) for v in block]
    if any(math.isnan(v) or math.isinf(v) for v in vals):
        return [0] * 32, 255
    amax = max(abs(Fraction(v)) for v in vals)
    if amax == 0:
        e = 0
    else:
        s = 0                         # find s with 2**s <= amax < 2**(s+1)
        while Fraction(2) ** s > amax:
            s -= 1
        while Fraction(2) ** (s + 1) <= amax:
            s += 1
        e = min(max(s - 2 + 127, 0), 254)
    mags = [Fraction(m) for m in mx.E2M1_MAGNITUDES]
    codes = []
    for v in vals:
        q = abs(Fraction(v)) / Fraction(2) ** (e - 127)
        d = [abs(q - m) for m in mags]
        best = min(d)
        cands = [c for c in range(8) if d[c] == best]
        c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        if math.copysign(1, v) < 0:
            c |= 8
        codes.append(c)
    return codes, e


def test_pack_ties_golden(golden):
    for q, code, mag in golden("pack_ties.txt"):
        block = np.zeros((1, 32))
        block[0, 0] = 6.0            # fixes the shared exponent at 2**0 (scale byte 127)
        block[0, 1] = float(q)
        block[0, 2] = -float(q)
        codes, scales = mx.pack(block)
        elem = mx.split_nibbles(codes)[0]
        assert scales[0, 0] == 127
        assert elem[1] == int(code), q
        assert elem[2] == int(code) | 8, q
        assert mx.E2M1_MAGNITUDES[int(code)] == float(mag)


@pytest.mark.parametrize("seed", range(4))
def test_pack_matches_rational_brute_force(seed):
    rng = np.random.default_rng(seed)
    rows = []
    for i in range(24):
        kind = i % 6
        if kind == 0:     # normal data over a wide range of magnitudes
            b = rng.standard_normal(32) * 2.0 ** rng.integers(-30, 30)
        elif kind == 1:   # exact midpoints of the scaled grid
            b = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], 32) * \
                rng.choice([-1, 1], 32) * 2.0 ** rng.integers(-5, 5)
        elif kind == 2:   # fp32 subnormals and tiny values (scale clamps at 0)
            b = rng.standard_normal(32) * 2.0 ** -140
        elif kind == 3:   # huge values (scale near the top)
            b = rng.standard_normal(32) * 2.0 ** 125
        elif kind == 4:   # signed zeros and one nonzero
            b = np.where(rng.random(32) < 0.5, -0.0, 0.0)
            b[rng.integers(32)] = rng.standard_normal()
        else:             # bf16-representable values
            b = np.round(rng.standard_normal(32) * 64) / 16
        rows.append(np.asarray(b, dtype=np.float32).astype(np.float64))
    v = np.stack(rows)
    codes, scales = mx.pack(v)
    elem = mx.split_nibbles(codes)
    for r in range(v.shape[0]):
        bc, be = pack_brute(v[r])
        assert scales[r, 0] == be, r
        assert list(elem[r]) == bc, r


def test_pack_special_blocks():
    v = np.zeros((4, 32))
    v[1, 3] = np.nan
    v[2, 5] = -np.inf
    v[3, :] = -0.0
    v[3, 7] = 1.0
    v[3, 8] = -1e-30                     # rounds to zero, keeps its sign bit
    codes, scales = mx.pack(v)
    elem = mx.split_nibbles(codes)
    assert scales[0, 0] == 0 and np.all(elem[0] == 0)
    assert scales[1, 0] == 255 and np.all(elem[1] == 0)
    assert scales[2, 0] == 255 and np.all(elem[2] == 0)
    assert elem[3, 0] == 8 and elem[3, 8] == 8 and elem[3, 7] != 0


def test_pack_scale_brackets_block_max():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((64, 96)) * 2.0 ** rng.integers(-20, 20, (64, 1))).astype(np.float32)
    codes, scales = mx.pack(v)
    amax = np.abs(v.astype(np.float64).reshape(64, 3, 32)).max(-1)
    ratio = amax / np.ldexp(1.0, scales.astype(np.int32) - 127)
    assert np.all((ratio >= 4) & (ratio < 8))


def test_pack_unpack_roundtrip_on_representable_blocks():
    rng = np.random.default_rng(11)
    rows, K = 200, 128
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(1, 250, (rows, K // 32), dtype=np.uint8)
    v = mx.unpack(codes, scales)
    c2, s2 = mx.pack(v)
    assert np.array_equal(mx.unpack(c2, s2), v)         # values always round-trip
    # codes and scale identical when the block's largest magnitude is 4 or 6
    elem = mx.split_nibbles(codes).reshape(rows, K // 32, 32)
    big = (elem & 7).max(-1) >= 6
    e2 = mx.split_nibbles(c2).reshape(rows, K // 32, 32)
    assert big.mean() > 0.9
    assert np.array_equal(e2[big], elem[big])
    assert np.array_equal(s2[big], scales[big])
