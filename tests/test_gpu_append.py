"""GPU parity of the decode-time append against the oracle (one token per sequence per call)."""
import numpy as np
import pytest

from oracle import cache as OC
from long_context_fp4_amd import synth
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def run_append(m, B, cap, steps, seed, ragged=False):
    """cap: rows reserved per sequence; ragged: each sequence gets its own capacity in
    [0, cap] and the sequences' row ranges are packed back to back with one spare row
    between neighbours (which must stay untouched)."""
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(seed)
    w_lat = synth.merge_weights(rng, m, 512)
    w_idx = synth.merge_weights(rng, m, 128)
    caps = rng.integers(0, cap + 1, B).astype(np.int64) if ragged else np.full(B, cap, np.int64)
    n0 = np.array([rng.integers(0, c + 1) for c in caps], np.int32)
    n0[B // 2] = caps[B // 2]                          # one sequence starts full: its groups are dropped
    c0 = rng.integers(0, m, B).astype(np.int32)
    st_lat0 = synth.hidden_host(rng, (B, max(m - 1, 1), 512))
    st_idx0 = synth.hidden_host(rng, (B, max(m - 1, 1), 128))
    tok_lat = synth.hidden_host(rng, (steps, B, 512))
    tok_idx = synth.hidden_host(rng, (steps, B, 128))
    off = np.concatenate([[0], np.cumsum(caps + 1)[:-1]]).astype(np.int64)   # one spare row after each
    rows_total = int(off[-1] + caps[-1] + 1)
    kv0 = rng.integers(0, 256, (rows_total, 288), dtype=np.uint8)
    ik0 = rng.integers(0, 256, (rows_total, 64), dtype=np.uint8)
    iks0 = rng.integers(0, 256, (rows_total, 4), dtype=np.uint8)

    kv, ik, iks = dev(kv0), dev(ik0), dev(iks0)
    st_lat = dev(st_lat0[:, : m - 1]) if m > 1 else None
    st_idx = dev(st_idx0[:, : m - 1]) if m > 1 else None
    cnt, n = dev(c0), dev(n0)
    dropped = torch.zeros(B, dtype=torch.int32, device="cuda")
    drops = np.zeros(B, np.int64)
    for t in range(steps):
        L.cache_append(dev(tok_lat[t]), dev(tok_idx[t]), dev(w_lat), dev(w_idx), m, st_lat, st_idx, cnt, dev(off),
                       n, dev(caps), kv, ik, iks, dropped=dropped)
        torch.cuda.synchronize()
        drops += host(dropped)
    kv, ik, iks, cnt, n = host(kv), host(ik), host(iks), host(cnt), host(n)

    ekv, eik, eiks = kv0.copy(), ik0.copy(), iks0.copy()
    for b in range(B):
        stream_lat = np.concatenate([st_lat0[b, : c0[b]], tok_lat[:, b]])
        stream_idx = np.concatenate([st_idx0[b, : c0[b]], tok_idx[:, b]])
        okv, oik, oiks, rest_lat, rest_idx = OC.append_tokens(stream_lat, stream_idx, w_lat, w_idx, m)
        room = int(caps[b]) - int(n0[b])
        take = min(len(okv), room)
        rows = slice(off[b] + n0[b], off[b] + n0[b] + take)
        ekv[rows], eik[rows], eiks[rows] = okv[:take], oik[:take], oiks[:take]
        assert n[b] == n0[b] + take, f"seq {b}: n_entries"
        assert drops[b] == len(okv) - take, f"seq {b}: dropped groups"
        assert cnt[b] == len(rest_lat), f"seq {b}: stage count"
        if m > 1 and len(rest_lat):
            assert np.array_equal(host(st_lat)[b, : len(rest_lat)], rest_lat), f"seq {b}: staged latent rows"
            assert np.array_equal(host(st_idx)[b, : len(rest_idx)], rest_idx), f"seq {b}: staged key rows"
    assert np.array_equal(kv, ekv) and np.array_equal(ik, eik) and np.array_equal(iks, eiks)


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_append_one_token_at_a_time(m):
    """Five sequences with different filled entries and staged counts (one full
    from the start), eleven calls: bit-exact entries, counters, stage rows, drops."""
    run_append(m, B=5, cap=4, steps=11, seed=700 + m)


def test_append_many_sequences():
    """More sequences than one workgroup takes (16), ratio 2."""
    run_append(2, B=41, cap=3, steps=7, seed=77)


@pytest.mark.parametrize("m", [1, 2])
def test_append_ragged_capacities(m):
    """Per-sequence capacities (some 0) with the row ranges packed back to back: a
    sequence that fills up drops its groups and never writes into its neighbour's rows."""
    run_append(m, B=23, cap=5, steps=9, seed=900 + m, ragged=True)
