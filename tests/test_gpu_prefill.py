"""GPU parity of multi-query (prefill) sparse attention: every query token with its
own causal top-k over the entries its token has completed, against the oracle."""
import numpy as np
import pytest

from oracle import attention as OA
from oracle import cache as OC
from oracle import indexer as OI
from long_context_fp4_amd import synth
from tests.gpu_util import ATTN_REL_TOL, attn_rel_err, check_topk, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,T_list,k", [(2, [50000, 90000], 512), (1, [9000, 3000, 12000], 64)])
def test_prefill_queries_see_only_completed_entries(m, T_list, k):
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(sum(T_list) + m)
    w_lat = synth.merge_weights(rng, m, 512)
    w_idx = synth.merge_weights(rng, m, 128)
    parts = [OC.cache_write(synth.hidden_host(rng, (T, 512)), synth.hidden_host(rng, (T, 128)), w_lat, w_idx, m)
             for T in T_list]
    E = [p[0].shape[0] for p in parts]
    kv, ik, iks = (np.concatenate([p[i] for p in parts]) for i in range(3))
    off = np.concatenate([[0], np.cumsum(E)[:-1]]).astype(np.int64)
    # (a negative position and one past the sequence's tokens clamp to none and all)
    B, Tq, H = len(T_list), 7, 32
    pos = np.stack([np.array([-1, 0, 2 * k - 1, T // 3, T - 2, T - 1, T + 300], np.int64) for T in T_list])
    q = np.stack([[synth.latent_query(rng, H) for _ in range(Tq)] for _ in range(B)])
    qi = np.stack([[synth.indexer_query(rng, 16) for _ in range(Tq)] for _ in range(B)])
    w = np.stack([[synth.head_weights(rng, 16) for _ in range(Tq)] for _ in range(B)])
    top, out, lse = L.prefill_layer(dev(kv), dev(ik), dev(iks), dev(off), dev(np.asarray(E, np.int32)), max(E), m,
                                    dev(pos), dev(qi), dev(q), w=dev(w), k=k)
    torch.cuda.synchronize()
    top, out, lse = host(top), host(out), host(lse)
    for b in range(B):
        for t in range(Tq):
            nv = max(0, min(E[b], (int(pos[b, t]) + 1) // m))
            rows = slice(off[b], off[b] + nv)
            s = OI.scores(ik[rows], iks[rows], qi[b, t], w[b, t], 1) if nv else np.zeros(0, np.float32)
            want = OI.topk(s, np.arange(nv), k)
            check_topk(top[b, t], want, lambda p: s[p], k, f"seq {b} query {t}")
            ro, rl = OA.sparse_attention(kv[off[b]:off[b] + E[b]], top[b, t], q[b, t])
            err = attn_rel_err(out[b, t], ro)
            assert np.all(err <= ATTN_REL_TOL), f"seq {b} query {t}: max rel err {err.max():.3g}"
            fin = np.isfinite(rl)
            assert np.array_equal(fin, np.isfinite(lse[b, t]))
            assert np.all(np.abs(lse[b, t][fin] - rl[fin]) <= 2e-3), f"seq {b} query {t}: lse"


def test_prefill_multi_query_pass_matches_oracle():
    """The multi-query scoring pass (a long sequence, so the fused plan runs):
    Tq = 11 is not a multiple of the queries a workgroup scores together, the
    queries' visible ranges end in different 1024-entry chunks (one inside the
    first chunk, one exactly at a chunk boundary), and two sequences of
    different lengths share the launch."""
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(777)
    m, k, H = 2, 512, 16
    T_list = [70000, 41000]
    w_lat = synth.merge_weights(rng, m, 512)
    w_idx = synth.merge_weights(rng, m, 128)
    parts = [OC.cache_write(synth.hidden_host(rng, (T, 512)), synth.hidden_host(rng, (T, 128)), w_lat, w_idx, m)
             for T in T_list]
    E = [p[0].shape[0] for p in parts]
    kv, ik, iks = (np.concatenate([p[i] for p in parts]) for i in range(3))
    off = np.concatenate([[0], np.cumsum(E)[:-1]]).astype(np.int64)
    B, Tq = len(T_list), 11
    pos = np.stack([np.array([1500, 2047, 2048 * 3 - 1, 2048 * 5, T // 2, T // 2 + 1, T - 700, T - 40, T - 3,
                              T - 2, T - 1], np.int64) for T in T_list])
    q = np.stack([[synth.latent_query(rng, H) for _ in range(Tq)] for _ in range(B)])
    qi = np.stack([[synth.indexer_query(rng, 16) for _ in range(Tq)] for _ in range(B)])
    w = np.stack([[synth.head_weights(rng, 16) for _ in range(Tq)] for _ in range(B)])
    top, out, lse = L.prefill_layer(dev(kv), dev(ik), dev(iks), dev(off), dev(np.asarray(E, np.int32)), max(E), m,
                                    dev(pos), dev(qi), dev(q), w=dev(w), k=k)
    torch.cuda.synchronize()
    top, out, lse = host(top), host(out), host(lse)
    for b in range(B):
        for t in range(Tq):
            nv = min(E[b], (int(pos[b, t]) + 1) // m)
            rows = slice(off[b], off[b] + nv)
            s = OI.scores(ik[rows], iks[rows], qi[b, t], w[b, t], 1)
            want = OI.topk(s, np.arange(nv), k)
            check_topk(top[b, t], want, lambda p: s[p], k, f"seq {b} query {t}")
            ro, rl = OA.sparse_attention(kv[off[b]:off[b] + E[b]], top[b, t], q[b, t])
            err = attn_rel_err(out[b, t], ro)
            assert np.all(err <= ATTN_REL_TOL), f"seq {b} query {t}: max rel err {err.max():.3g}"
            assert np.all(np.abs(lse[b, t] - rl) <= 2e-3), f"seq {b} query {t}: lse"


def test_prefill_128_queries():
    """128 query tokens of one sequence in one call (32 query groups of the
    multi-query pass), every 37th token position of the sequence's last ~4.7K,
    so consecutive queries see different numbers of entries and the visible
    ranges end inside chunks and at chunk boundaries alike."""
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(128)
    m, k, H, T = 2, 512, 16, 70001
    w_lat = synth.merge_weights(rng, m, 512)
    w_idx = synth.merge_weights(rng, m, 128)
    kv, ik, iks = OC.cache_write(synth.hidden_host(rng, (T, 512)), synth.hidden_host(rng, (T, 128)), w_lat, w_idx, m)
    E = kv.shape[0]
    Tq = 128
    pos = (T - 1 - 37 * np.arange(Tq)[::-1]).astype(np.int64)[None]
    q = np.stack([synth.latent_query(rng, H) for _ in range(Tq)])[None]
    qi = np.stack([synth.indexer_query(rng, 16) for _ in range(Tq)])[None]
    w = np.stack([synth.head_weights(rng, 16) for _ in range(Tq)])[None]
    top, out, lse = L.prefill_layer(dev(kv), dev(ik), dev(iks), dev(np.zeros(1, np.int64)),
                                    dev(np.array([E], np.int32)), E, m, dev(pos), dev(qi), dev(q), w=dev(w), k=k)
    torch.cuda.synchronize()
    top, out, lse = host(top), host(out), host(lse)
    for t in range(Tq):
        nv = min(E, (int(pos[0, t]) + 1) // m)
        s = OI.scores(ik[:nv], iks[:nv], qi[0, t], w[0, t], 1)
        want = OI.topk(s, np.arange(nv), k)
        check_topk(top[0, t], want, lambda p: s[p], k, f"query {t}")
        ro, rl = OA.sparse_attention(kv, top[0, t], q[0, t])
        err = attn_rel_err(out[0, t], ro)
        assert np.all(err <= ATTN_REL_TOL), f"query {t}: max rel err {err.max():.3g}"
        assert np.all(np.abs(lse[0, t] - rl) <= 2e-3), f"query {t}: lse"


@pytest.mark.parametrize("Tq,mode", [(8, "relu_w"), (6, "relu_w"), (5, "dot"), (4, "qmx8")])
def test_prefill_selects_what_decode_selects(Tq, mode):
    """The multi-query pass scores four queries per key tile with one combined
    head-sum reduction and computes the queries' visible entries itself; its
    scores must equal the one-query pass's bit for bit. Each query of the
    prefill is also run as a decode sequence over the entries it sees: the
    selections must be the same positions (near-ties included) and the
    attention outputs the same bits. The first query sees no entry (even Tq)
    or fewer than k, the last sits past the cached entries and sees them all.
    Tq = 6 leaves the second group of four queries half empty; the
    dot-product mode takes the multi-query pass's per-query head sums; the
    quantized-query mode has no multi-query pass (a launch of its own
    computes the views, then the decode path runs)."""
    import torch
    import long_context_fp4_amd as L
    sm = {"relu_w": L.CSA2_SCORE_RELU_W, "dot": L.CSA2_SCORE_DOT,
          "qmx8": L.CSA2_SCORE_RELU_W | L.CSA2_SCORE_QMX8}[mode]
    rng = np.random.default_rng(4000 + Tq)
    m, k, H, T = 2, 512, 16, 90001
    w_lat = synth.merge_weights(rng, m, 512)
    w_idx = synth.merge_weights(rng, m, 128)
    kv, ik, iks = OC.cache_write(synth.hidden_host(rng, (T, 512)), synth.hidden_host(rng, (T, 128)), w_lat, w_idx, m)
    E = kv.shape[0]
    pos = np.sort(rng.choice(np.arange(3000, T), size=Tq, replace=False)).astype(np.int64)
    pos[-1] = T + 500                                  # past the cached entries: all of them visible
    pos[0] = -1 if Tq % 2 == 0 else 700                # no entry visible / fewer than k
    q = np.stack([synth.latent_query(rng, H) for _ in range(Tq)])
    Hi = 1 if mode == "dot" else 16                   # the dot-product score takes one indexer head
    qi = np.stack([synth.indexer_query(rng, Hi) for _ in range(Tq)])
    w = np.stack([synth.head_weights(rng, Hi) for _ in range(Tq)])
    dkv, dik, diks = dev(kv), dev(ik), dev(iks)
    top, out, lse = L.prefill_layer(dkv, dik, diks, dev(np.zeros(1, np.int64)), dev(np.array([E], np.int32)), E, m,
                                    dev(pos[None]), dev(qi[None]), dev(q[None]), w=dev(w[None]), score_mode=sm, k=k)
    vis = np.where(pos < 0, 0, np.minimum(E, (pos + 1) // m)).astype(np.int32)
    dtop, _, dout, dlse = L.decode_layer(L.CSA2_FULL, dkv, dik, diks, dev(np.zeros(Tq, np.int64)), dev(vis), E,
                                         dev(q), q_idx=dev(qi), w=dev(w), score_mode=sm, k=k)
    torch.cuda.synchronize()
    assert np.array_equal(host(top)[0], host(dtop))
    assert np.array_equal(host(out)[0].view(np.uint32), host(dout).view(np.uint32))
    assert np.array_equal(host(lse)[0].view(np.uint32), host(dlse).view(np.uint32))
