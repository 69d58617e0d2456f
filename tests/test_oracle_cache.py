"""Pins of the cache write: hand-worked examples, closed forms of the merge, quantizer bounds."""
import json
import os

import numpy as np
import pytest

from oracle import cache as C
from oracle import formats as F
from long_context_fp4_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quant_examples.json")))


def bf16(vals):
    return synth.bf16_bits(np.asarray(vals, dtype=np.float32))


def test_hand_worked_latent_blocks():
    blocks = GOLD["latent_blocks"]
    # one 512-channel row: the examples, then repeats of the first example
    xs = [b["x"] for b in blocks] + [blocks[0]["x"]] * (32 - len(blocks))
    x = bf16(np.concatenate(xs))[None, :]
    kv, _, _ = C.cache_write(x, bf16(np.zeros((1, 128))), np.ones((1, 512), np.float32),
                             np.ones((1, 128), np.float32), 1)
    assert kv.shape == (1, 288)
    for bi, b in enumerate(blocks):
        assert kv[0, 8 * bi: 8 * bi + 8].tobytes().hex().upper() == b["codes_hex"], b["why"]
        assert "%02X" % kv[0, 256 + bi] == b["scale_hex"], b["why"]


def test_hand_worked_indexer_blocks():
    blocks = GOLD["indexer_blocks"]
    x = bf16(np.concatenate([b["x"] for b in blocks]))[None, :]
    _, ik, iks = C.cache_write(bf16(np.zeros((1, 512))), x, np.ones((1, 512), np.float32),
                               np.ones((1, 128), np.float32), 1)
    assert ik.shape == (1, 64) and iks.shape == (1, 4)
    for bi, b in enumerate(blocks):
        assert ik[0, 16 * bi: 16 * bi + 16].tobytes().hex().upper() == b["codes_hex"], b["why"]
        assert "%02X" % iks[0, bi] == b["scale_hex"], b["why"]


def test_merge_ratio_one_is_identity():
    rng = np.random.default_rng(1)
    x = synth.hidden_host(rng, (64, 512))
    e = C.merge(x, np.ones((1, 512), np.float32), 1)
    assert np.array_equal(e, F.bf16_bits_to_float(x))


def test_merge_one_hot_weights_select_a_position():
    rng = np.random.default_rng(2)
    x = synth.hidden_host(rng, (64, 128))
    for j in range(4):
        w = np.zeros((4, 128), np.float32)
        w[j] = 1.0
        e = C.merge(x, w, 4)
        assert np.array_equal(e, F.bf16_bits_to_float(x)[j::4])


def test_merge_equal_weights_give_the_correctly_rounded_mean():
    rng = np.random.default_rng(3)
    x = synth.hidden_host(rng, (1000, 512))
    e = C.merge(x, np.full((2, 512), 0.5, np.float32), 2)
    xf = F.bf16_bits_to_float(x).astype(np.float64)
    mean = (xf[0::2] + xf[1::2]) / 2          # halving is exact; one rounding to float32
    assert np.array_equal(e, mean.astype(np.float32))


def test_merge_weighted_sum_error_bound_and_trailing_group():
    rng = np.random.default_rng(4)
    w = synth.merge_weights(rng, 3, 128)
    x = synth.hidden_host(rng, (301, 128))
    e = C.merge(x, w, 3)
    assert e.shape == (100, 128)              # floor(301 / 3) entries, the partial group is dropped
    xf = F.bf16_bits_to_float(x).astype(np.float64)[:300].reshape(100, 3, 128)
    exact = np.einsum("ejc,jc->ec", xf, w.astype(np.float64))
    bound = 4 * np.finfo(np.float32).eps * np.einsum("ejc,jc->ec", np.abs(xf), w.astype(np.float64))
    assert np.all(np.abs(e - exact) <= bound)


def _grid_aligned_latent(rng, n):
    """Rows whose blocks hold exact multiples of an E4M3 scale, block maximum 6*scale."""
    s_bytes = rng.integers(0x10, 0x70, size=(n, 32)).astype(np.uint8)
    s = F.e4m3fn_decode(s_bytes)
    codes = rng.integers(0, 16, size=(n, 32, 16)).astype(np.uint8)
    codes[:, :, 0] = 7                           # one element at +6 * scale: amax / 6 == scale
    codes[:, :, 1:] &= np.uint8(0xF) ^ np.uint8(0x7)   # keep sign, clear magnitude...
    codes[:, :, 1:] |= rng.integers(0, 8, size=(n, 32, 15)).astype(np.uint8)
    x = F.e2m1_decode(codes) * s[:, :, None]
    return x.reshape(n, 512).astype(np.float32), codes, s_bytes


def test_grid_aligned_latent_round_trips():
    rng = np.random.default_rng(5)
    x, codes, s_bytes = _grid_aligned_latent(rng, 64)
    # negative zeros come from e2m1_decode(0x8) * s = -0.0, matching code 0x8
    kv = C.quantize_latent(x)
    assert np.array_equal(kv[:, 256:], s_bytes)
    assert np.array_equal(C.unpack_nibbles(kv[:, :256]).reshape(64, 32, 16), codes)
    assert np.array_equal(C.dequant_latent(kv), x.astype(np.float64))


def test_grid_aligned_indexer_round_trips():
    rng = np.random.default_rng(6)
    n = 64
    X = rng.integers(-20, 20, size=(n, 4))
    codes = rng.integers(0, 16, size=(n, 4, 32)).astype(np.uint8)
    codes[:, :, 0] = 6                              # +4 * 2**X: floor(log2 amax) - 2 == X
    codes[:, :, 1:] &= np.uint8(0x8)
    codes[:, :, 1:] |= rng.integers(0, 7, size=(n, 4, 31)).astype(np.uint8)   # magnitude <= 4
    x = (F.e2m1_decode(codes) * np.ldexp(1.0, X)[:, :, None]).reshape(n, 128).astype(np.float32)
    ik, iks = C.quantize_indexer(x)
    assert np.array_equal(iks.astype(np.int64) - 127, X)
    assert np.array_equal(C.unpack_nibbles(ik).reshape(n, 4, 32), codes)
    assert np.array_equal(C.dequant_indexer(ik, iks), x.astype(np.float64))


def test_latent_quantizer_error_bounds():
    rng = np.random.default_rng(8)
    x = F.bf16_bits_to_float(synth.hidden_host(rng, (2000, 512), outliers=np.array([3, 77]))).copy()
    kv = C.quantize_latent(x)
    deq = C.dequant_latent(kv).reshape(2000, 32, 16)
    xb = x.astype(np.float64).reshape(2000, 32, 16)
    s = F.e4m3fn_decode(kv[:, 256:])[:, :, None]
    q = np.abs(xb) / s
    half_spacing = np.where(q < 2, 0.25, np.where(q < 4, 0.5, 1.0))
    inside = q <= 6
    err = np.abs(xb - deq)
    assert np.all(err[inside] <= (half_spacing * s)[inside] * (1 + 1e-6))
    assert np.all(err[~inside] <= 0.375 * np.broadcast_to(s, q.shape)[~inside])
    # the scale tracks amax/6 within E4M3's relative step
    amax = np.abs(xb).max(axis=2)
    assert np.all(np.abs(s[:, :, 0] - amax / 6) <= amax / 6 * 2.0 ** -4)
    assert np.all(np.sign(deq[deq != 0]) == np.sign(xb[deq != 0]))


def test_indexer_quantizer_error_bounds():
    rng = np.random.default_rng(9)
    x = F.bf16_bits_to_float(synth.hidden_host(rng, (2000, 128), outliers=np.array([5]))).copy()
    ik, iks = C.quantize_indexer(x)
    deq = C.dequant_indexer(ik, iks).reshape(2000, 4, 32)
    xb = x.astype(np.float64).reshape(2000, 4, 32)
    s = F.e8m0_decode(iks)[:, :, None]
    r = np.abs(xb) / s
    assert np.all(r.max(axis=2) >= 4) and np.all(r.max(axis=2) < 8)
    half_spacing = np.where(r < 2, 0.25, np.where(r < 4, 0.5, 1.0))
    inside = r <= 6
    err = np.abs(xb - deq)
    assert np.all(err[inside] <= (half_spacing * s)[inside])
    assert np.all(err[~inside] <= 2 * np.broadcast_to(s, r.shape)[~inside])


def test_row_layout_sizes():
    rng = np.random.default_rng(10)
    p = synth.params(synth.Workload("t", 1, B=1, m=2, T=100, H=2, Hi=1, score_mode=0))
    x_lat = synth.hidden_host(rng, (101, 512))
    x_idx = synth.hidden_host(rng, (101, 128))
    kv, ik, iks = C.cache_write(x_lat, x_idx, p["w_lat"], p["w_idx"], 2)
    assert kv.shape == (50, 288) and ik.shape == (50, 64) and iks.shape == (50, 4)
    assert kv.shape[1] + ik.shape[1] + iks.shape[1] == 356


@pytest.mark.parametrize("m,T", [(1, 5), (2, 9), (3, 10), (4, 4), (4, 3), (16, 40)])
def test_append_one_token_at_a_time_equals_one_write(m, T):
    """Tokens appended one at a time leave the entries of one write of all of
    them (floor(T/m) groups of consecutive tokens, in order) and the last
    T mod m tokens in the stage."""
    rng = np.random.default_rng(100 * m + T)
    x_lat = synth.hidden_host(rng, (T, 512))
    x_idx = synth.hidden_host(rng, (T, 128))
    w_lat = synth.merge_weights(rng, m, 512)
    w_idx = synth.merge_weights(rng, m, 128)
    kv, ik, iks, st_lat, st_idx = C.append_tokens(x_lat, x_idx, w_lat, w_idx, m)
    wkv, wik, wiks = C.cache_write(x_lat, x_idx, w_lat, w_idx, m)
    assert kv.shape == (T // m, 288) and np.array_equal(kv, wkv)
    assert np.array_equal(ik, wik) and np.array_equal(iks, wiks)
    E = T // m
    assert np.array_equal(st_lat, x_lat[E * m:]) and np.array_equal(st_idx, x_idx[E * m:])
