"""GPU parity of the fused merge + quantize + pack kernel against the oracle (bit-exact)."""
import json
import os

import numpy as np
import pytest

from oracle import cache as OC
from long_context_fp4_amd import synth
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def lib_write(x_lat, x_idx, w_lat, w_idx, m):
    import long_context_fp4_amd as L
    kv, ik, iks = L.cache_write(dev(x_lat), dev(x_idx), dev(w_lat), dev(w_idx), m)
    return host(kv), host(ik), host(iks)


def oracle_write(x_lat, x_idx, w_lat, w_idx, m):
    outs = [OC.cache_write(x_lat[b], x_idx[b], w_lat, w_idx, m) for b in range(x_lat.shape[0])]
    return tuple(np.concatenate([o[i] for o in outs]) for i in range(3))


def assert_same(got, want, what):
    for name, g, w in zip(("kv", "ik", "iks"), got, want):
        assert g.shape == w.shape, f"{what}/{name}: shape {g.shape} vs {w.shape}"
        if not np.array_equal(g, w):
            rows = np.nonzero(np.any(g != w, axis=1))[0]
            raise AssertionError(f"{what}/{name}: {rows.size} rows differ, first {rows[:5]}")


def test_tiny_workload_bit_exact():
    w = synth.workload("tiny")
    p = synth.params(w)
    xs = synth.hidden_states_host(w, p)
    x_lat = np.stack([a for a, _ in xs])
    x_idx = np.stack([b for _, b in xs])
    assert_same(lib_write(x_lat, x_idx, p["w_lat"], p["w_idx"], w.m),
                oracle_write(x_lat, x_idx, p["w_lat"], p["w_idx"], w.m), "tiny")


@pytest.mark.parametrize("m,T,B", [(1, 333, 2), (2, 1001, 3), (3, 998, 1), (4, 1024, 2), (5, 77, 2), (16, 64, 1)])
def test_ratios_and_ragged_tails(m, T, B):
    rng = np.random.default_rng(100 + m)
    w_lat = synth.merge_weights(rng, m, 512)
    w_idx = synth.merge_weights(rng, m, 128)
    x_lat = synth.hidden_host(rng, (B, T, 512), outliers=np.array([1, 300]))
    x_idx = synth.hidden_host(rng, (B, T, 128), outliers=np.array([64]))
    assert_same(lib_write(x_lat, x_idx, w_lat, w_idx, m), oracle_write(x_lat, x_idx, w_lat, w_idx, m),
                f"m={m},T={T},B={B}")


@pytest.mark.parametrize("m", [1, 2, 3])
def test_ragged_batch_one_launch(m):
    """Sequences of different lengths (one empty, one shorter than m) padded to the longest,
    written in one call at per-sequence offsets into one buffer with gaps between the
    sequences: each sequence's rows bit-exact, the gap rows untouched."""
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(300 + m)
    lens = np.array([517, 0, m - 1, 2048, 35, 1000], np.int64)
    B, T = len(lens), int(lens.max())
    w_lat = synth.merge_weights(rng, m, 512)
    w_idx = synth.merge_weights(rng, m, 128)
    x_lat = synth.hidden_host(rng, (B, T, 512), outliers=np.array([7]))
    x_idx = synth.hidden_host(rng, (B, T, 128))
    ents = lens // m
    off = np.zeros(B, np.int64)
    cur = 3
    for b in rng.permutation(B):                       # sequences placed out of order, with gaps
        off[b] = cur
        cur += int(ents[b]) + int(rng.integers(0, 5))
    rows = cur + 4
    kv0 = rng.integers(0, 256, (rows, 288), dtype=np.uint8)
    ik0 = rng.integers(0, 256, (rows, 64), dtype=np.uint8)
    iks0 = rng.integers(0, 256, (rows, 4), dtype=np.uint8)
    kv, ik, iks = dev(kv0), dev(ik0), dev(iks0)
    L.cache_write(dev(x_lat), dev(x_idx), dev(w_lat), dev(w_idx), m, kv=kv, ik=ik, iks=iks,
                  n_tokens=dev(lens), out_entry_offset=dev(off))
    torch.cuda.synchronize()
    ekv, eik, eiks = kv0.copy(), ik0.copy(), iks0.copy()
    for b in range(B):
        okv, oik, oiks = OC.cache_write(x_lat[b, :lens[b]], x_idx[b, :lens[b]], w_lat, w_idx, m)
        r = slice(int(off[b]), int(off[b]) + len(okv))
        ekv[r], eik[r], eiks[r] = okv, oik, oiks
    assert_same((host(kv), host(ik), host(iks)), (ekv, eik, eiks), f"ragged m={m}")


def test_hand_worked_blocks():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quant_examples.json")))
    lat = [b["x"] for b in g["latent_blocks"]]
    lat = lat + [lat[0]] * (32 - len(lat))
    x_lat = synth.bf16_bits(np.concatenate(lat))[None, None, :]
    x_idx = synth.bf16_bits(np.concatenate([b["x"] for b in g["indexer_blocks"]]))[None, None, :]
    kv, ik, iks = lib_write(x_lat, x_idx, np.ones((1, 512), np.float32), np.ones((1, 128), np.float32), 1)
    for bi, b in enumerate(g["latent_blocks"]):
        assert kv[0, 8 * bi: 8 * bi + 8].tobytes().hex().upper() == b["codes_hex"], b["why"]
        assert "%02X" % kv[0, 256 + bi] == b["scale_hex"], b["why"]
    for bi, b in enumerate(g["indexer_blocks"]):
        assert ik[0, 16 * bi: 16 * bi + 16].tobytes().hex().upper() == b["codes_hex"], b["why"]
        assert "%02X" % iks[0, bi] == b["scale_hex"], b["why"]


def test_extreme_magnitudes():
    """Blocks scaled by 2^e for e in [-140, 120]: zero, subnormal and saturated scales, float32 subnormals."""
    rng = np.random.default_rng(7)
    B, T, m = 2, 512, 2
    x = rng.standard_normal((B, T, 640), dtype=np.float32)
    e_lat = rng.integers(-140, 121, size=(B, T // m, 32))
    e_idx = rng.integers(-140, 121, size=(B, T // m, 4))
    sc_lat = np.repeat(np.repeat(np.ldexp(1.0, e_lat), 16, axis=2), m, axis=1)
    sc_idx = np.repeat(np.repeat(np.ldexp(1.0, e_idx), 32, axis=2), m, axis=1)
    x_lat = synth.bf16_bits((x[..., :512] * sc_lat).astype(np.float32))
    x_idx = synth.bf16_bits((x[..., 512:] * sc_idx).astype(np.float32))
    x_lat[:, :8] = 0                                   # some all-zero entries
    x_idx[:, 8:16] = 0x8000                            # negative zeros
    w_lat = synth.merge_weights(rng, m, 512)
    w_idx = synth.merge_weights(rng, m, 128)
    assert_same(lib_write(x_lat, x_idx, w_lat, w_idx, m), oracle_write(x_lat, x_idx, w_lat, w_idx, m), "extreme")


def test_write128k_full_size_sampled():
    """The 8 x 131072-token write with outlier channels, in the benchmark's launch configuration.

    All entries of the first and last sequence, plus 4096 random entries of the others, bit-exact.
    """
    import torch
    import long_context_fp4_amd as L
    w = synth.workload("write128k")
    p = synth.params(w)
    xl, xi = [], []
    for b in range(w.B):
        a, c = synth.hidden_states_device(w, p, b)
        xl.append(a)
        xi.append(c)
    x_lat = torch.stack(xl)
    x_idx = torch.stack(xi)
    del xl, xi
    kv, ik, iks = L.cache_write(x_lat, x_idx, dev(p["w_lat"]), dev(p["w_idx"]), w.m)
    torch.cuda.synchronize()
    E = w.T // w.m
    for b in (0, w.B - 1):
        want = OC.cache_write(host(x_lat[b]), host(x_idx[b]), p["w_lat"], p["w_idx"], w.m)
        got = (host(kv[b * E:(b + 1) * E]), host(ik[b * E:(b + 1) * E]), host(iks[b * E:(b + 1) * E]))
        assert_same(got, want, f"write128k seq {b}")
    rng = np.random.default_rng(1)
    for b in range(1, w.B - 1):
        ent = np.sort(rng.choice(E, size=512, replace=False))
        rows = (ent[:, None] * w.m + np.arange(w.m)[None, :]).reshape(-1)
        r = torch.as_tensor(rows, device="cuda")
        xl_h = host(x_lat[b].index_select(0, r))
        xi_h = host(x_idx[b].index_select(0, r))
        want = OC.cache_write(xl_h, xi_h, p["w_lat"], p["w_idx"], w.m)
        e_idx = torch.as_tensor(b * E + ent, device="cuda")
        got = (host(kv.index_select(0, e_idx)), host(ik.index_select(0, e_idx)), host(iks.index_select(0, e_idx)))
        assert_same(got, want, f"write128k seq {b} sample")
