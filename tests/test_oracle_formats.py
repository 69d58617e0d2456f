"""Pins of the number formats: closed forms, brute force, and torch's float8 cast."""
import numpy as np
import pytest
import torch

from oracle import formats as F


def e2m1_closed_form(code):
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    return s * (m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2))


def test_e2m1_decode_all_codes():
    got = F.e2m1_decode(np.arange(16))
    want = np.array([e2m1_closed_form(c) for c in range(16)])
    assert np.array_equal(got, want)
    assert np.array_equal(np.abs(got[:8]), [0, 0.5, 1, 1.5, 2, 3, 4, 6])


def brute_force_e2m1(q):
    """Nearest grid point by exhaustive search; ties go to the even code."""
    grid = [abs(e2m1_closed_form(c)) for c in range(8)]
    out = []
    for v in q:
        d = [abs(v - g) for g in grid]
        best = min(d)
        cands = [c for c in range(8) if d[c] == best]
        if len(cands) == 2:
            cands = [c for c in cands if c % 2 == 0]
        out.append(cands[0])
    return np.array(out, dtype=np.uint8)


def sweep_values():
    rng = np.random.default_rng(7)
    fine = np.arange(0, 8 * 1024 + 1) / 1024.0                       # every multiple of 2**-10 in [0, 8]
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0])
    around = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                             np.nextafter(mids.astype(np.float32), np.float32(10)), mids])
    rand = rng.random(20000) * 8
    return np.concatenate([fine, around.astype(np.float64), rand, [6.0, 6.2, 6.375, 7.9, 100.0]])


def test_e2m1_rounding_matches_brute_force():
    q = sweep_values()
    assert np.array_equal(F.e2m1_round_magnitude(q), brute_force_e2m1(q))


def test_e2m1_rounding_matches_threshold_form():
    # independent statement of the same rule: strict thresholds where the tie goes down
    q = sweep_values()
    code = ((q > 0.25).astype(int) + (q >= 0.75) + (q > 1.25) + (q >= 1.75)
            + (q > 2.5) + (q >= 3.5) + (q > 5.0))
    assert np.array_equal(F.e2m1_round_magnitude(q), code)


def test_e4m3fn_decode_matches_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3fn_decode(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.nanmax(got) == 448.0


def test_e4m3fn_round_matches_torch_cast():
    rng = np.random.default_rng(11)
    exps = rng.integers(-14, 9, size=200000)
    v = np.ldexp(1.0 + rng.random(200000), exps).astype(np.float32)
    # all representable values, their midpoints and neighbours
    rep = F.e4m3fn_decode(np.arange(0, 127)).astype(np.float64)
    mids = ((rep[1:] + rep[:-1]) / 2).astype(np.float32)
    extra = np.concatenate([rep.astype(np.float32), mids,
                            np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                            np.float32([0.0, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 447.9, 448.0, 455.9, 463.9])])
    v = np.concatenate([v[v < 464], extra])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3fn_round(v)
    assert np.array_equal(got, ref)


def test_e4m3fn_round_saturates():
    got = F.e4m3fn_round(np.array([464.0, 1000.0, 1e30]))
    assert np.all(got == 0x7E) and F.e4m3fn_decode(0x7E) == 448.0


def test_e8m0_decode_and_shared_exponent():
    b = np.arange(255)
    assert np.array_equal(F.e8m0_decode(b), 2.0 ** (b - 127.0))
    assert np.isnan(F.e8m0_decode(255))
    for k in range(-120, 120, 7):
        for frac in (1.0, 1.3, 1.999):
            amax = np.float32(2.0 ** k * frac)
            byte = int(F.mx_shared_exponent(amax))
            assert byte == k + 125
            r = float(amax) * 2.0 ** -(byte - 127)
            assert 4.0 <= r < 8.0       # the block maximum lands in [4, 8) after rescaling
    assert F.mx_shared_exponent(np.float32(0.0)) == 0
