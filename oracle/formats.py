"""Number formats of the FP4 cache: E2M1 values, E4M3FN scales, E8M0 scales.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

[FP4] section "Le coût d'une entrée": the main-cache latent is stored as E2M1
values with one E4M3 scale per 16 channels, and the indexer key as E2M1 with
one E8M0 scale per 32 channels ("standard MXFP4"). [FP4] section "D'où
viennent ces deux réglages" names the scale dtype ``torch.float8_e4m3fn``,
which fixes the FN variant of E4M3 (no infinities, 0x7F/0xFF are NaN, largest
finite value 448).

The pages name the formats but do not print their value grids; the grids
below are the OCP Microscaling (MX) v1.0 definitions of E2M1, E4M3 and E8M0.
All arithmetic here is done in float64, where every value of these formats
and every power-of-two rescaling used below is exact.
"""
import numpy as np

# E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; no inf/NaN.
# Magnitude codes 0..7 in order of increasing value.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0

E4M3FN_MAX = 448.0
E4M3FN_MIN_NORMAL_EXP = -6   # smallest normal is 2**-6
E4M3FN_MANT_BITS = 3         # subnormal spacing is 2**-9


def e2m1_decode(codes):
    """Value of 4-bit E2M1 codes (bit 3 = sign, bits 0..2 = magnitude code)."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[codes & 7]
    return np.where(codes & 8, -mag, mag)


def e2m1_round_magnitude(q):
    """Round-to-nearest-even of non-negative values onto the E2M1 grid.

    Returns the 3-bit magnitude code. Values above 6 saturate to 6 (E2M1 has
    no infinity). Within each binade the grid is uniform: spacing 0.5 on
    [0, 2) (this includes the single subnormal 0.5), 1 on [2, 4) and 2 on
    [4, 8). Rounding to the nearest multiple of the spacing with ties to the
    even multiple is round-to-nearest-even, because on every binade the even
    multiples are exactly the codes whose mantissa bit is 0.
    """
    q = np.asarray(q, dtype=np.float64)
    if np.any(q < 0) or np.any(~np.isfinite(q)):
        raise ValueError("e2m1_round_magnitude expects finite non-negative input")
    spacing = np.where(q < 2.0, 0.5, np.where(q < 4.0, 1.0, 2.0))
    r = np.rint(q / spacing) * spacing          # np.rint rounds half to even
    r = np.minimum(r, E2M1_MAX)
    # value -> magnitude code
    code = np.searchsorted(E2M1_MAGNITUDES, r)
    assert np.all(E2M1_MAGNITUDES[code] == r)
    return code.astype(np.uint8)


def e4m3fn_decode(b):
    """Value of E4M3FN bytes: bias 7, 3 mantissa bits, subnormals, 0x7F/0xFF NaN."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m / 8.0, -6)
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return s * v


def e4m3fn_round(v):
    """Round non-negative finite values to E4M3FN, nearest-even, saturating.

    Reading taken: values whose nearest-even rounding is beyond the largest
    finite value (448) are clamped to 448 rather than mapped to NaN, since the
    scale of a block must stay usable. Returns the byte encoding.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(~np.isfinite(v)):
        raise ValueError("e4m3fn_round expects finite non-negative input")
    _, e2 = np.frexp(v)                 # v = f * 2**e2 with f in [0.5, 1)
    exp = e2 - 1                        # v in [2**exp, 2**(exp+1))
    exp = np.maximum(exp, E4M3FN_MIN_NORMAL_EXP)   # below 2**-6: subnormal spacing
    spacing = np.ldexp(1.0, exp - E4M3FN_MANT_BITS)
    r = np.rint(v / spacing) * spacing
    r = np.minimum(r, E4M3FN_MAX)
    return e4m3fn_encode_exact(r)


def e4m3fn_encode_exact(r):
    """Byte of non-negative values that are exactly representable in E4M3FN."""
    r = np.asarray(r, dtype=np.float64)
    out = np.zeros(r.shape, dtype=np.uint8)
    nz = r > 0
    _, e2 = np.frexp(np.where(nz, r, 1.0))
    exp = e2 - 1
    is_norm = nz & (exp >= E4M3FN_MIN_NORMAL_EXP)
    mant_n = (np.ldexp(np.where(is_norm, r, 1.0), -exp) - 1.0) * 8.0
    byte_n = ((exp + 7) << 3) + mant_n.astype(np.int64)
    mant_s = np.ldexp(r, 9)             # subnormal: r = m * 2**-9
    out = np.where(is_norm, byte_n, np.where(nz, mant_s.astype(np.int64), 0))
    out = out.astype(np.uint8)
    assert np.array_equal(e4m3fn_decode(out), r), "value not exactly representable"
    return out


def e8m0_decode(b):
    """Value 2**(b-127) of E8M0 bytes; 0xFF is NaN."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def mx_shared_exponent(amax):
    """OCP MX shared exponent of a block: floor(log2(amax)) - emax(E2M1).

    emax of E2M1 is 2 (largest value 6 = 1.5 * 2**2). Returned as the E8M0
    byte X + 127, clamped to [0, 254]; a block whose amax is zero gets the
    byte 0. ``amax`` is a float32/float64 array; floor(log2) is read from
    the binary exponent, so it is exact.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, e2 = np.frexp(np.where(amax > 0, amax, 1.0))
    x = (e2 - 1) - 2
    b = np.clip(x + 127, 0, 254)
    return np.where(amax > 0, b, 0).astype(np.uint8)


def bf16_bits_to_float(bits):
    """bfloat16 bit patterns (uint16) to float32 values (exact widening)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)
