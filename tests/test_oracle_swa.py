"""Pins of the sliding-window oracle: the page's byte count, the scale rule, quantizer
bounds, ring placement and the lse merge (one softmax over the union of two sets)."""
import numpy as np
import pytest

from oracle import swa as S
from oracle.formats import bf16_bits_to_float, e4m3fn_decode
from long_context_fp4_amd import synth


def test_row_bytes_and_the_pages_window_size():
    """[FP4] 'La contrepartie : la fenêtre glissante': 40 x 128 x (512 + 512/16) bytes = 2.66 MiB."""
    rows = S.quantize_window_rows(synth.hidden_host(np.random.default_rng(0), (3, 512)))
    assert rows.shape == (3, 544) and S.ROW_BYTES == 512 + 512 // 16
    total = 40 * S.WINDOW * rows.shape[1]
    assert total == 2_785_280 and round(total / 2 ** 20, 2) == 2.66


@pytest.mark.parametrize("amax", [1.0, 3.0, 448.0, 449.0, 0.001, 1e4, 2.0 ** -20])
def test_scale_is_the_smallest_power_of_two_that_fits(amax):
    X = int(S.block_exponent(np.array([amax]))[0])
    assert amax <= 448.0 * 2.0 ** X
    assert amax > 448.0 * 2.0 ** (X - 1)


def test_grid_values_round_trip():
    """A block whose values lie on the E4M3 grid times 2^X, with amax = 448 * 2^X, is exact."""
    rng = np.random.default_rng(1)
    grid = e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))          # all finite non-negative E4M3 values
    rows = []
    for X in (-3, 0, 2):
        v = rng.choice(grid, (32, 16)) * np.where(rng.random((32, 16)) < 0.5, -1, 1)
        v[:, 0] = 448.0
        rows.append(v * 2.0 ** X)
    x = np.concatenate(rows).reshape(-1, 512)
    bits = synth.bf16_bits(x.astype(np.float32))
    assert np.array_equal(bf16_bits_to_float(bits), x.astype(np.float32))   # exact in bf16
    d = S.dequant_window_rows(S.quantize_window_rows(bits))
    assert np.array_equal(d, x)


def test_quantizer_error_bound():
    """Relative error <= 2^-4 in E4M3's normal range; absolute <= 2^-10 * 2^X below it."""
    rng = np.random.default_rng(2)
    # rows of very different magnitudes, so blocks use many scale exponents
    x = synth.bf16_bits((rng.standard_normal((64, 512)) * np.exp(rng.uniform(-6, 6, (64, 1)))).astype(np.float32))
    xf = bf16_bits_to_float(x).astype(np.float64)
    rows = S.quantize_window_rows(x)
    d = S.dequant_window_rows(rows)
    X = rows[:, 512:].astype(np.int64) - 127
    s = np.repeat(2.0 ** X, 16, axis=1)
    normal = np.abs(xf) >= 2.0 ** -6 * s
    err = np.abs(d - xf)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(xf[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * s[~normal])


def test_ring_keeps_the_last_128_tokens():
    rng = np.random.default_rng(3)
    x = synth.hidden_host(rng, (200, 512))
    ring = S.window_write(x, pos0=5)
    rows = S.quantize_window_rows(x)
    for t in range(200 - 128, 200):
        assert np.array_equal(ring[(5 + t) % 128], rows[t])
    # a ring written in two parts equals one write
    ring2 = S.window_write(x[130:], pos0=135, ring=S.window_write(x[:130], pos0=5))
    assert np.array_equal(ring, ring2)


def test_merge_is_one_softmax_over_the_union():
    """Closed form: merging the (o, lse) of two disjoint sets equals attention over both."""
    rng = np.random.default_rng(4)
    rows = S.quantize_window_rows(synth.hidden_host(rng, (40, 512)))
    q = synth.latent_query(rng, 8)
    o_a, l_a = S.window_attention(rows[:25], q)
    o_b, l_b = S.window_attention(rows[25:], q)
    o, l = S.merge_branches(o_a, l_a, o_b, l_b)
    qf = bf16_bits_to_float(q).astype(np.float64)
    c = S.dequant_window_rows(rows)
    logits = qf @ c.T
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    want_o = (p @ c) / p.sum(axis=1, keepdims=True)
    want_l = logits.max(axis=1) + np.log(p.sum(axis=1))
    np.testing.assert_allclose(o, want_o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, want_l, rtol=1e-12)


def test_merge_with_an_empty_branch():
    rng = np.random.default_rng(5)
    rows = S.quantize_window_rows(synth.hidden_host(rng, (7, 512)))
    q = synth.latent_query(rng, 4)
    o, l = S.window_attention(rows, q)
    o0, l0 = S.window_attention(rows[:0], q)
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))
    for a, b in (((o, l), (o0, l0)), ((o0, l0), (o, l))):
        om, lm = S.merge_branches(a[0], a[1], b[0], b[1])
        np.testing.assert_array_equal(om, o)
        np.testing.assert_array_equal(lm, l)
    om, lm = S.merge_branches(o0, l0, o0, l0)
    assert np.all(om == 0) and np.all(np.isneginf(lm))


def test_one_token_window():
    rng = np.random.default_rng(6)
    rows = S.quantize_window_rows(synth.hidden_host(rng, (1, 512)))
    q = synth.latent_query(rng, 3)
    o, l = S.window_attention(rows, q, tau=0.5)
    c = S.dequant_window_rows(rows)[0]
    assert np.array_equal(o, np.tile(c, (3, 1)))
    np.testing.assert_allclose(l, 0.5 * bf16_bits_to_float(q).astype(np.float64) @ c, rtol=1e-15)
