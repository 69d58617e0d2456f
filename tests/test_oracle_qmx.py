"""Pins of the oracle's quantized-query (MXFP8) scoring variant.

The conversion is the OCP MX v1.0 rule with E4M3FN elements (the keys are
"standard MXFP4": [FP4] section "Le coût d'une entrée"). Pinned against a
brute-force nearest search over every finite E4M3FN value, the closed form of
the shared exponent, lossless round trips of representable queries (where the
variant must give exactly the exact path's scores), saturation, zero blocks,
and the rounding error bound.
"""
import numpy as np
import pytest

from oracle import cache as OC
from oracle import indexer as OI
from oracle.formats import bf16_bits_to_float
from long_context_fp4_amd import synth

FINITE = np.array([b for b in range(128) if b != 0x7F], np.uint8)        # non-negative finite codes


def e4m3_value(b):
    """E4M3FN magnitude of a code below 0x7F, from the format's definition."""
    e, m = b >> 3, b & 7
    return (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)


GRID = np.array([e4m3_value(int(b)) for b in FINITE])


def brute_code(v):
    """Nearest E4M3FN magnitude to v >= 0 (ties: even code), values beyond 448 clamped."""
    d = np.abs(GRID - min(v, 448.0))
    best = np.flatnonzero(d == d.min())
    even = [i for i in best if FINITE[i] % 2 == 0]
    return int(FINITE[even[0] if even else best[0]])


def to_bf16_bits(x):
    """float values that are exact in bf16 -> bits."""
    f = np.asarray(x, np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_bits_to_float(bits), f), "value not exact in bf16"
    return bits


def test_shared_exponent_closed_form_and_brute_force_codes():
    rng = np.random.default_rng(5)
    x = synth.indexer_query(rng, 16).astype(np.uint16)       # bf16 bits [16, 128]
    xf = bf16_bits_to_float(x).astype(np.float64)
    # widen the dynamic range: each block gets its own power-of-two factor
    f = np.ldexp(1.0, rng.integers(-20, 20, size=(16, 4)))
    x = to_bf16_bits((xf.reshape(16, 4, 32) * f[:, :, None]).reshape(16, 128))
    xf = bf16_bits_to_float(x).astype(np.float64)
    codes, sb = OI.quantize_query_mx(x)
    for h in range(16):
        for blk in range(4):
            v = xf[h, 32 * blk:32 * blk + 32]
            amax = np.abs(v).max()
            X = int(sb[h, blk]) - 127
            assert 2.0 ** (X + 8) <= amax < 2.0 ** (X + 9)
            for c in range(32):
                want = brute_code(abs(v[c]) * 2.0 ** -X) | (0x80 if np.signbit(v[c]) else 0)
                assert codes[h, 32 * blk + c] == want, (h, blk, c, v[c])


def test_representable_queries_round_trip_and_score_exactly():
    """A query whose blocks are E4M3FN values times 2^X with a block maximum in
    [256, 448] * 2^X is quantized without loss, so the variant's scores equal
    the exact path's bit for bit."""
    rng = np.random.default_rng(6)
    Hi = 16
    codes = rng.choice(FINITE, size=(Hi, 128)).astype(np.uint8)
    top = rng.integers(0x78, 0x7F, size=(Hi, 4))             # exponent field 15: 256 .. 448
    for h in range(Hi):
        for blk in range(4):
            codes[h, 32 * blk + rng.integers(0, 32)] = top[h, blk]
    codes |= (rng.integers(0, 2, size=codes.shape) * 0x80).astype(np.uint8)
    X = rng.integers(-20, 0, size=(Hi, 4))
    vals = np.array([[e4m3_value(int(c) & 0x7F) * (-1 if c & 0x80 else 1) for c in row] for row in codes])
    q = to_bf16_bits(vals * np.repeat(np.ldexp(1.0, X), 32, axis=1))
    got_codes, got_sb = OI.quantize_query_mx(q)
    zero = (codes & 0x7F) == 0
    assert np.array_equal(got_codes[~zero], codes[~zero])
    assert np.array_equal(got_sb, (X + 127).astype(np.uint8))
    np.testing.assert_array_equal(OI.dequant_query_mx(got_codes, got_sb),
                                  bf16_bits_to_float(q).astype(np.float64))
    _, ik, iks = OC.cache_write(synth.hidden_host(rng, (40, 512)), synth.hidden_host(rng, (40, 128)),
                                synth.merge_weights(rng, 1, 512), synth.merge_weights(rng, 1, 128), 1)
    w = synth.head_weights(rng, Hi)
    np.testing.assert_array_equal(OI.scores(ik, iks, q, w, OI.SCORE_RELU_W | OI.SCORE_QMX8),
                                  OI.scores(ik, iks, q, w, OI.SCORE_RELU_W))
    np.testing.assert_array_equal(OI.scores(ik, iks, q[:1], None, OI.SCORE_DOT | OI.SCORE_QMX8),
                                  OI.scores(ik, iks, q[:1], None, OI.SCORE_DOT))


def test_saturation_ties_and_zero_blocks():
    q = np.zeros((1, 128), np.float64)
    q[0, 0] = 480.0          # X = 0 (256 <= 480 < 512): 480 saturates to 448
    q[0, 1] = -1.5 * 2 ** -9 # below 2^-6: subnormal spacing 2^-9, 1.5 -> 2 (even) ulps
    q[0, 2] = 2.5 * 2 ** -9  # 2.5 -> 2 ulps (even)
    q[0, 3] = 272.0          # 256 + 16: halfway between 256 and 288 -> 256 (even mantissa)
    q[0, 32:64] = -0.0       # a zero block: X = -127, signs kept
    q[0, 64] = 2.0 ** -130   # a tiny block: X clamps at -127
    codes, sb = OI.quantize_query_mx(to_bf16_bits(q))
    assert sb[0, 0] == 127 and codes[0, 0] == 0x7E
    assert codes[0, 1] == 0x82 and codes[0, 2] == 0x02 and codes[0, 3] == 0x78
    assert sb[0, 1] == 0 and np.all(codes[0, 32:64] == 0x80)
    assert sb[0, 2] == 0 and codes[0, 64] == 0x20     # X clamps at -127: 2^-130 * 2^127 = 2^-3
    assert sb[0, 3] == 0 and np.all(codes[0, 96:] == 0)


def test_rounding_error_bound():
    """Every unsaturated value is within half a unit of its E4M3FN binade."""
    rng = np.random.default_rng(7)
    x = synth.indexer_query(rng, 16).astype(np.uint16)
    xf = bf16_bits_to_float(x).astype(np.float64)
    codes, sb = OI.quantize_query_mx(x)
    qd = OI.dequant_query_mx(codes, sb)
    X = np.repeat(sb.astype(np.int64) - 127, 32, axis=1)
    e = np.floor(np.log2(np.maximum(np.abs(xf), 2.0 ** -140))).astype(np.int64)
    ulp = np.ldexp(1.0, np.maximum(e - X, -6) - 3 + X)
    unsat = np.ldexp(np.abs(xf), -X) <= 448.0
    assert unsat.mean() > 0.9
    assert np.all(np.abs(qd - xf)[unsat] <= ulp[unsat] / 2)
    assert np.all(np.abs(qd[~unsat]) == np.ldexp(448.0, X[~unsat]))
