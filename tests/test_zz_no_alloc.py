"""The allocation-free decode layer against the workspace one (same kernels, bit-identical results).

Two pairs of calls: a large batch first (32 sequences of up to 65536 entries,
whose fused plan does not fit the static scratch, so the separate-launch plan
runs), then a smaller ragged batch on the same device (the fused plan, with a
pool, then Reindex and Reuse over it). Every output of the allocation-free entry
point must equal the workspace entry point's bit for bit: the static scratch
keeps what the first call left, and no kernel may read it before writing it.
"""
import numpy as np
import pytest

from long_context_fp4_amd import synth
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def step(msg):
    import sys
    print(f"[no-alloc] {msg}", file=sys.stderr, flush=True)


def make_cache(L, torch, rng, gen, ents, m=1):
    """Library-written cache of sequences with `ents` entries each, packed back to back."""
    ents = np.asarray(ents, np.int64)
    off = np.concatenate([[0], np.cumsum(ents)[:-1]]).astype(np.int64)
    E = int(ents.sum())
    kv = torch.empty((E, 288), dtype=torch.uint8, device="cuda")
    ik = torch.empty((E, 64), dtype=torch.uint8, device="cuda")
    iks = torch.empty((E, 4), dtype=torch.uint8, device="cuda")
    w_lat, w_idx = dev(synth.merge_weights(rng, m, 512)), dev(synth.merge_weights(rng, m, 128))
    T = int(ents.max()) * m
    for b0 in range(0, len(ents), 8):                  # 8 sequences per write call
        sel = list(range(b0, min(b0 + 8, len(ents))))
        xl = synth.hidden_device(gen, (len(sel), T, 512))
        xi = synth.hidden_device(gen, (len(sel), T, 128))
        L.cache_write(xl, xi, w_lat, w_idx, m, kv=kv, ik=ik, iks=iks,
                      n_tokens=dev(ents[sel] * m), out_entry_offset=dev(off[sel]))
        del xl, xi
    torch.cuda.synchronize()
    return kv, ik, iks, dev(off), dev(ents.astype(np.int32))


def queries(rng, B, H=64, Hi=16):
    q = dev(np.stack([synth.latent_query(rng, H) for _ in range(B)]))
    qi = dev(np.stack([synth.indexer_query(rng, Hi) for _ in range(B)]))
    w = dev(np.stack([synth.head_weights(rng, Hi) for _ in range(B)]))
    return q, qi, w


def same(a, b, what):
    a, b = host(a), host(b)
    assert a.shape == b.shape and a.dtype == b.dtype, what
    if a.tobytes() != b.tobytes():
        raise AssertionError(f"{what}: {int(np.count_nonzero(a != b))} of {a.size} elements differ")


def run_pair(L, torch, mode, cache, max_n, q, k=512, pool_k=0, q_idx=None, w=None, pool=None, topk_in=None):
    """The layer through both entry points; returns both result tuples."""
    kv, ik, iks, off, ne = cache
    B, H = q.shape[0], q.shape[1]
    ref = L.decode_layer(mode, kv, ik, iks, off, ne, max_n, q, q_idx=q_idx, w=w, k=k, pool_k=pool_k, pool=pool,
                         topk=None if topk_in is None else topk_in.clone())
    topk = topk_in.clone() if topk_in is not None else torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    pl = pool if mode != L.CSA2_FULL or not pool_k else torch.full((B, pool_k), -7, dtype=torch.int32,
                                                                      device="cuda")
    got = L.decode_layer_noalloc(mode, kv, ik, iks, off, ne, max_n, q, topk, out, lse, q_idx=q_idx, w=w, k=k,
                                 pool_k=pool_k, pool=pl)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_entry_point():
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(2024)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2024)
    # call 1: 32 sequences, ragged up to 65536 entries (fused scratch ~120 MiB > 64 MiB)
    ents1 = np.full(32, 65536, np.int64)
    ents1[::5] = rng.integers(20000, 65536, len(ents1[::5]))
    ents1[3] = 0
    step("cache 1")
    c1 = make_cache(L, torch, rng, gen, ents1)
    max1 = int(ents1.max())
    B1 = len(ents1)
    need = L.lib().csa2_decode_workspace_bytes(B1, max1, 64, 512, 0)
    assert need > L.CSA2_NOALLOC_SCRATCH_BYTES                   # this call takes the separate-launch plan
    q, qi, w = queries(rng, B1)
    step("call 1 (Full, 32 sequences)")
    ref, got = run_pair(L, torch, L.CSA2_FULL, c1, max1, q, q_idx=qi, w=w)
    for nm, a, b in zip(("topk", "out", "lse"), (ref[0], ref[2], ref[3]), (got[0], got[2], got[3])):
        same(b, a, f"call 1 {nm}")
    del c1
    # call 2: smaller, ragged, with a pool (fused plan), then Reindex and Reuse over that pool
    ents2 = np.array([40000, 23000, 70000, 5000], np.int64)
    step("cache 2")
    c2 = make_cache(L, torch, rng, gen, ents2, m=2)
    max2 = int(ents2.max())
    B2 = len(ents2)
    q, qi, w = queries(rng, B2)
    step("call 2 (Full with a pool of 16384)")
    ref, got = run_pair(L, torch, L.CSA2_FULL, c2, max2, q, pool_k=16384, q_idx=qi, w=w)
    for nm, a, b in zip(("topk", "pool", "out", "lse"), ref, got):
        same(b, a, f"call 2 {nm}")
    pool = ref[1]
    q2, qi2, w2 = queries(rng, B2)
    step("call 3 (Reindex)")
    ref, got = run_pair(L, torch, L.CSA2_REINDEX, c2, max2, q2, q_idx=qi2, w=w2, pool=pool)
    for nm, a, b in zip(("topk", "out", "lse"), (ref[0], ref[2], ref[3]), (got[0], got[2], got[3])):
        same(b, a, f"call 3 {nm}")
    step("call 4 (Reuse)")
    ref, got = run_pair(L, torch, L.CSA2_REUSE, c2, max2, q2, topk_in=ref[0])
    for nm, a, b in zip(("out", "lse"), (ref[2], ref[3]), (got[2], got[3])):
        same(b, a, f"call 4 {nm}")
    # a call whose indexer scratch exceeds the array is refused before any launch
    kv, ik, iks, off, ne = c2
    topk = torch.empty((B2, 512), dtype=torch.int32, device="cuda")
    out = torch.empty((B2, 64, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B2, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(L.Csa2Error, match="static scratch"):
        L.decode_layer_noalloc(L.CSA2_FULL, kv, ik, iks, off, ne, 1 << 22, q, topk, out, lse, q_idx=qi, w=w)
