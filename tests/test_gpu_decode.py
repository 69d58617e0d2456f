"""GPU parity of whole decode layers (Full / Reindex / Reuse) against the oracle."""
import numpy as np
import pytest

from oracle import attention as OA
from oracle import cache as OC
from oracle import indexer as OI
from long_context_fp4_amd import synth
from tests.gpu_util import ATTN_REL_TOL, attn_rel_err, check_topk, dev, host

pytestmark = pytest.mark.gpu


def oracle_cache(rng, n_list, m):
    w_lat = synth.merge_weights(rng, m, 512)
    w_idx = synth.merge_weights(rng, m, 128)
    parts = [OC.cache_write(synth.hidden_host(rng, (n * m, 512)), synth.hidden_host(rng, (n * m, 128)),
                            w_lat, w_idx, m) for n in n_list]
    kv, ik, iks = (np.concatenate([p[i] for p in parts]) for i in range(3))
    off = np.concatenate([[0], np.cumsum(n_list)[:-1]]).astype(np.int64)
    return kv, ik, iks, off


def check_attention(kv_rows, sel, q, out, lse, what):
    ro, rl = OA.sparse_attention(kv_rows, sel, q)
    err = attn_rel_err(out, ro)
    assert np.all(err <= ATTN_REL_TOL), f"{what}: max rel err {err.max():.3g}"
    assert np.all(np.abs(lse - rl) <= 2e-3), f"{what}: lse"


@pytest.mark.parametrize("n_list,pool_k", [([40000, 23000, 70000], 16384), ([9000, 30000], 4096)])
def test_layer_group_full_reindex_reuse(n_list, pool_k):
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(sum(n_list))
    kv, ik, iks, off = oracle_cache(rng, n_list, 1)
    B, H = len(n_list), 64
    nb = np.asarray(n_list, np.int32)
    ws = L.Workspace()
    d = dict(kv=dev(kv), ik=dev(ik), iks=dev(iks), entry_offset=dev(off), n_entries=dev(nb), max_n=max(n_list),
             workspace=ws)
    qF, qiF, wF = (np.stack([f(rng, h) for _ in range(B)]) for f, h in
                   ((synth.latent_query, H), (synth.indexer_query, 16), (synth.head_weights, 16)))
    qR, qiR, wR = (np.stack([f(rng, h) for _ in range(B)]) for f, h in
                   ((synth.latent_query, H), (synth.indexer_query, 16), (synth.head_weights, 16)))
    qU = np.stack([synth.perturb(rng, qR[b], 0.01) for b in range(B)])
    topF, pool, outF, lseF = L.decode_layer(L.CSA2_FULL, q=dev(qF), q_idx=dev(qiF), w=dev(wF), pool_k=pool_k, **d)
    topR, _, outR, lseR = L.decode_layer(L.CSA2_REINDEX, q=dev(qR), q_idx=dev(qiR), w=dev(wR), pool=pool, **d)
    _, _, outU, lseU = L.decode_layer(L.CSA2_REUSE, q=dev(qU), topk=topR, **d)
    torch.cuda.synchronize()
    topF, pool, topR = host(topF), host(pool), host(topR)
    outF, outR, outU, lseF, lseR, lseU = map(host, (outF, outR, outU, lseF, lseR, lseU))
    for b, n in enumerate(n_list):
        rows = slice(off[b], off[b] + n)
        s = OI.scores(ik[rows], iks[rows], qiF[b], wF[b], 1)
        check_topk(pool[b], OI.topk(s, np.arange(n), pool_k), lambda p: s[p], pool_k, f"pool{b}")
        gp = pool[b][pool[b] >= 0]
        check_topk(topF[b], OI.topk(s[gp], gp, 512), lambda p: s[p], 512, f"full{b}")
        check_attention(kv[rows], topF[b], qF[b], outF[b], lseF[b], f"full attention {b}")
        s2 = np.zeros(n, np.float32)
        s2[gp] = OI.scores(ik[rows][gp], iks[rows][gp], qiR[b], wR[b], 1)
        check_topk(topR[b], OI.topk(s2[gp], gp, 512), lambda p: s2[p], 512, f"reindex{b}")
        check_attention(kv[rows], topR[b], qR[b], outR[b], lseR[b], f"reindex attention {b}")
        check_attention(kv[rows], topR[b], qU[b], outU[b], lseU[b], f"reuse attention {b}")


def test_full_layer_pool_edge_cases():
    """A Full layer with a 4096 pool whose finish is split over several
    workgroups per sequence: sequence 0 has its 700 largest keys in its first
    chunk (too few keys reach the highest pool cutoff: the fallback), sequence
    1 is shorter than the pool, sequence 2 holds one indexer row 30000 times
    (every key in the threshold bin, more than the parts exchange: one
    workgroup finishes it with its scratch rows), sequence 3 is empty and
    sequence 4 takes the split path; then the same workspace with the batch
    reversed."""
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(77)
    n_list = [40000, 3000, 30000, 0, 50000]
    pool_k, H = 4096, 64
    kv, ik, iks, off = oracle_cache(rng, n_list, 1)
    ik, iks = ik.copy(), iks.copy()
    iks[:700] = np.minimum(iks[:700].astype(np.int32) + 6, 254).astype(np.uint8)
    a = int(off[2])
    ik[a:a + 30000] = ik[a]
    iks[a:a + 30000] = iks[a]
    ws = L.Workspace()
    for order in (list(range(5)), list(range(4, -1, -1))):
        nl = [n_list[i] for i in order]
        offs = np.asarray([off[i] for i in order], np.int64)
        B = len(nl)
        qF, qiF, wF = (np.stack([f(rng, h) for _ in range(B)]) for f, h in
                       ((synth.latent_query, H), (synth.indexer_query, 16), (synth.head_weights, 16)))
        topF, pool, outF, lseF = L.decode_layer(L.CSA2_FULL, dev(kv), dev(ik), dev(iks), dev(offs),
                                                dev(np.asarray(nl, np.int32)), max(nl), dev(qF), q_idx=dev(qiF),
                                                w=dev(wF), pool_k=pool_k, workspace=ws)
        torch.cuda.synchronize()
        topF, pool, outF, lseF = host(topF), host(pool), host(outF), host(lseF)
        for b, n in enumerate(nl):
            what = f"seq{order[b]} (n={n})"
            if n == 0:
                assert np.all(pool[b] == -1) and np.all(topF[b] == -1), what
                continue
            rows = slice(offs[b], offs[b] + n)
            s = OI.scores(ik[rows], iks[rows], qiF[b], wF[b], 1)
            check_topk(pool[b], OI.topk(s, np.arange(n), pool_k), lambda p: s[p], pool_k, f"pool {what}")
            gp = pool[b][pool[b] >= 0]
            check_topk(topF[b], OI.topk(s[gp], gp, 512), lambda p: s[p], 512, f"full {what}")
            check_attention(kv[rows], topF[b], qF[b], outF[b], lseF[b], f"attention {what}")


def test_decode128k_full_size():
    """32 sequences x 131072 tokens (65536 ratio-2 entries), one Full layer, as the benchmark runs it.

    Every sequence: the oracle's scores, top-512 and attention over the GPU-written cache
    bytes; sequences 0 and 31 also have those bytes checked bit-exact against the oracle's
    cache write of their hidden states. On the same cache, as the benchmark's legs run them:
    the quantized-query variant of the layer (sequences 0 and 31, within its accumulation
    bound) and the prefill of 32 query tokens at the last 32 positions of sequence 0
    (queries 0, 17 and 31 checked).
    """
    import torch
    import long_context_fp4_amd as L
    w = synth.workload("decode128k")
    p = synth.params(w)
    E = w.T // w.m
    kv = torch.empty((w.B * E, 288), dtype=torch.uint8, device="cuda")
    ik = torch.empty((w.B * E, 64), dtype=torch.uint8, device="cuda")
    iks = torch.empty((w.B * E, 4), dtype=torch.uint8, device="cuda")
    hidden = {}
    for b in range(w.B):
        x_lat, x_idx = synth.hidden_states_device(w, p, b)
        L.cache_write(x_lat[None], x_idx[None], dev(p["w_lat"]), dev(p["w_idx"]), w.m,
                      kv=kv[b * E:(b + 1) * E], ik=ik[b * E:(b + 1) * E], iks=iks[b * E:(b + 1) * E])
        if b in (0, w.B - 1):
            hidden[b] = (host(x_lat), host(x_idx))
    Lr = p["layers"][0]
    off = np.arange(w.B, dtype=np.int64) * E
    nb = np.full(w.B, E, np.int32)
    top, _, out, lse = L.decode_layer(L.CSA2_FULL, kv, ik, iks, dev(off), dev(nb), E, dev(Lr["q"]),
                                      q_idx=dev(Lr["q_idx"]), w=dev(Lr["w"]), k=w.k)
    torch.cuda.synchronize()
    top, out, lse = host(top), host(out), host(lse)
    hkv, hik, hiks = host(kv), host(ik), host(iks)
    for b, (xl, xi) in hidden.items():
        okv, oik, oiks = OC.cache_write(xl, xi, p["w_lat"], p["w_idx"], w.m)
        assert np.array_equal(hkv[b * E:(b + 1) * E], okv)
        assert np.array_equal(hik[b * E:(b + 1) * E], oik)
        assert np.array_equal(hiks[b * E:(b + 1) * E], oiks)
        hidden[b] = (okv, oik, oiks)
    for b in range(w.B):
        rows = slice(b * E, (b + 1) * E)
        s = OI.scores(hik[rows], hiks[rows], Lr["q_idx"][b], Lr["w"][b], 1)
        check_topk(top[b], OI.topk(s, np.arange(E), w.k), lambda q: s[q], w.k, f"seq{b}")
        check_attention(hkv[rows], top[b], Lr["q"][b], out[b], lse[b], f"attention seq{b}")
    del hkv, hik, hiks

    # the quantized-query variant of the same layer
    from tests.test_gpu_qmx import qmx_bound
    qmode = OI.SCORE_RELU_W | OI.SCORE_QMX8
    top, _, out, lse = L.decode_layer(L.CSA2_FULL, kv, ik, iks, dev(off), dev(nb), E, dev(Lr["q"]),
                                      q_idx=dev(Lr["q_idx"]), w=dev(Lr["w"]), score_mode=qmode, k=w.k)
    torch.cuda.synchronize()
    top, out, lse = host(top), host(out), host(lse)
    for b, (okv, oik, oiks) in hidden.items():
        s = OI.scores(oik, oiks, Lr["q_idx"][b], Lr["w"][b], qmode)
        tol = 2 * qmx_bound(oik, oiks, Lr["q_idx"][b], Lr["w"][b], qmode).max()
        check_topk(top[b], OI.topk(s, np.arange(E), w.k), lambda q: s[q], w.k, f"qmx seq{b}", tol=tol)
        check_attention(okv, top[b], Lr["q"][b], out[b], lse[b], f"qmx attention seq{b}")

    # prefill: 32 query tokens at the last 32 positions of sequence 0
    okv, oik, oiks = hidden[0]
    rng = np.random.default_rng(20261213)
    Tq = 32
    pos = np.arange(w.T - Tq, w.T, dtype=np.int64)[None]
    qp = np.stack([synth.latent_query(rng, w.H) for _ in range(Tq)])[None]
    qi = np.stack([synth.indexer_query(rng, w.Hi) for _ in range(Tq)])[None]
    wh = np.stack([synth.head_weights(rng, w.Hi) for _ in range(Tq)])[None]
    ptop, pout, plse = L.prefill_layer(kv, ik, iks, dev(off[:1]), dev(nb[:1]), E, w.m, dev(pos), dev(qi),
                                       dev(qp), w=dev(wh), k=w.k)
    torch.cuda.synchronize()
    ptop, pout, plse = host(ptop), host(pout), host(plse)
    for t in (0, 17, 31):
        nv = min(E, (int(pos[0, t]) + 1) // w.m)
        s = OI.scores(oik[:nv], oiks[:nv], qi[0, t], wh[0, t], 1)
        check_topk(ptop[0, t], OI.topk(s, np.arange(nv), w.k), lambda q: s[q], w.k, f"prefill query {t}")
        check_attention(okv, ptop[0, t], qp[0, t], pout[0, t], plse[0, t], f"prefill attention query {t}")


def run_full(kv, ik, iks, off, n_list, H, k, rng, ws=None):
    import torch
    import long_context_fp4_amd as L
    B = len(n_list)
    q = np.stack([synth.latent_query(rng, H) for _ in range(B)])
    qi = np.stack([synth.indexer_query(rng, 16) for _ in range(B)])
    w = np.stack([synth.head_weights(rng, 16) for _ in range(B)])
    top, _, out, lse = L.decode_layer(L.CSA2_FULL, dev(kv), dev(ik), dev(iks), dev(off),
                                      dev(np.asarray(n_list, np.int32)), max(n_list), dev(q), q_idx=dev(qi),
                                      w=dev(w), k=k, workspace=ws)
    torch.cuda.synchronize()
    return q, qi, w, host(top), host(out), host(lse)


def check_full(kv, ik, iks, off, n_list, k, q, qi, w, top, out, lse, what):
    for b, n in enumerate(n_list):
        rows = slice(off[b], off[b] + n)
        if n == 0:
            assert np.all(top[b] == -1), f"{what} seq{b}: empty sequence selects nothing"
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b])), f"{what} seq{b}: empty attention"
            continue
        s = OI.scores(ik[rows], iks[rows], qi[b], w[b], 1)
        check_topk(top[b], OI.topk(s, np.arange(n), k), lambda p: s[p], k, f"{what} seq{b}")
        check_attention(kv[rows], top[b], q[b], out[b], lse[b], f"{what} attention seq{b}")


@pytest.mark.parametrize("n_list,H,k", [([40000, 300, 17000, 65536, 0], 64, 512),   # two splits
                                        ([20000, 33000, 511], 20, 100)])               # ragged head group
def test_full_direct_top_k_inside_attention(n_list, H, k):
    """Full layers whose direct top-k finish runs inside the attention launch:
    short, empty and long sequences, one and two splits, a ragged head group."""
    rng = np.random.default_rng(len(n_list) * 1000 + H + k)
    kv, ik, iks, off = oracle_cache(rng, n_list, 1)
    q, qi, w, top, out, lse = run_full(kv, ik, iks, off, n_list, H, k, rng)
    check_full(kv, ik, iks, off, n_list, k, q, qi, w, top, out, lse, "fused")


def test_full_direct_fallback_inside_attention():
    """The 700 largest indexer keys of sequence 1 sit in its first chunk (E8M0
    scales raised by 2^6): too few keys reach the highest local cutoff, so each
    attention workgroup of that sequence recomputes its scores and selects from
    all of them; sequence 0 takes the fast path in the same launch."""
    rng = np.random.default_rng(23)
    n_list = [30000, 40000]
    kv, ik, iks, off = oracle_cache(rng, n_list, 1)
    iks = iks.copy()
    a = off[1]
    iks[a:a + 700] = np.minimum(iks[a:a + 700].astype(np.int32) + 6, 254).astype(np.uint8)
    q, qi, w, top, out, lse = run_full(kv, ik, iks, off, n_list, 64, 512, rng)
    check_full(kv, ik, iks, off, n_list, 512, q, qi, w, top, out, lse, "fallback")
    # the same workspace again with a smaller batch: the scratch rows are rewritten
    import long_context_fp4_amd as L
    ws = L.Workspace()
    for nl in (n_list, n_list[1:]):
        offs = off if len(nl) == 2 else off[1:] - off[1]
        sl = slice(off[0] if len(nl) == 2 else off[1], off[-1] + n_list[-1])
        q, qi, w, top, out, lse = run_full(kv[sl], ik[sl], iks[sl], offs, nl, 64, 512, rng, ws)
        check_full(kv[sl], ik[sl], iks[sl], offs, nl, 512, q, qi, w, top, out, lse, f"reuse B={len(nl)}")


@pytest.mark.parametrize("chunks", [[63], [0, 5, 17], [1, 4, 9, 12, 20, 26, 31, 37, 44, 50, 55, 61]])
def test_full_direct_clustered_top_keys(chunks):
    """The top keys of sequence 1 sit in a few chunks (300 rows at the start of
    each listed chunk with E8M0 scales raised by 2^6): those chunks' local
    cutoffs lie far above the others', so too few keys reach the highest one.
    With one or three such chunks the finish rescores only them and takes every
    other chunk's listed keys; with twelve (more than it rescores alone) it
    rescores the whole sequence. Sequence 0 takes the fast path."""
    rng = np.random.default_rng(97 + len(chunks))
    n_list = [30000, 65000]
    kv, ik, iks, off = oracle_cache(rng, n_list, 1)
    iks = iks.copy()
    for c in chunks:
        a = off[1] + 1024 * c
        iks[a:a + 300] = np.minimum(iks[a:a + 300].astype(np.int32) + 6, 254).astype(np.uint8)
    q, qi, w, top, out, lse = run_full(kv, ik, iks, off, n_list, 64, 512, rng)
    check_full(kv, ik, iks, off, n_list, 512, q, qi, w, top, out, lse, f"clustered {len(chunks)}")


def test_full_direct_overflowed_tied_chunk():
    """Sequence 1: copies of its best indexer row with E8M0 scales raised by a
    power of two (scores scale exactly): 800 tied copies (x4) fill chunk 7's
    list past its capacity, and 30 copies (x64) after them are the best keys
    of the sequence; 20 chunks hold 30 copies (x8) each and three chunks 300
    copies (x16). The finish must rescore chunk 7 although its list holds
    only ties, and break the ties by position."""
    rng = np.random.default_rng(131)
    n_list = [20000, 60000]
    kv, ik, iks, off = oracle_cache(rng, n_list, 1)
    ik, iks = ik.copy(), iks.copy()
    qi1 = synth.indexer_query(np.random.default_rng(7), 16)
    w1 = synth.head_weights(np.random.default_rng(8), 16)
    a = off[1]
    s1 = OI.scores(ik[a:a + n_list[1]], iks[a:a + n_list[1]], qi1, w1, 1)
    best = a + int(np.argmax(s1))

    def put(row, cnt, boost):
        ik[row:row + cnt] = ik[best]
        iks[row:row + cnt] = np.minimum(iks[best].astype(np.int32) + boost, 254).astype(np.uint8)

    put(a + 7 * 1024, 800, 2)
    put(a + 7 * 1024 + 900, 30, 6)
    for c in range(20, 40):
        put(a + c * 1024, 30, 3)
    for c in (50, 52, 54):
        put(a + c * 1024, 300, 4)
    import torch
    import long_context_fp4_amd as L
    B = 2
    q = np.stack([synth.latent_query(rng, 64) for _ in range(B)])
    qi = np.stack([synth.indexer_query(rng, 16), qi1])
    w = np.stack([synth.head_weights(rng, 16), w1])
    top, _, out, lse = L.decode_layer(L.CSA2_FULL, dev(kv), dev(ik), dev(iks), dev(off),
                                      dev(np.asarray(n_list, np.int32)), max(n_list), dev(q), q_idx=dev(qi),
                                      w=dev(w), k=512)
    torch.cuda.synchronize()
    top, out, lse = host(top), host(out), host(lse)
    check_full(kv, ik, iks, off, n_list, 512, q, qi, w, top, out, lse, "overflowed tied chunk")
    assert np.all(np.isin(np.arange(7 * 1024 + 900, 7 * 1024 + 930), top[1]))


def test_full_direct_long_lists_inside_attention():
    """Sequence 0 carries 90 and 100 copies of its best indexer row in two
    chunks: their lists exceed 64 candidates, so the attention workgroups copy
    the lists to LDS before selecting; sequence 1 has more than 64 chunks."""
    rng = np.random.default_rng(41)
    n_list = [40000, 70000]
    kv, ik, iks, off = oracle_cache(rng, n_list, 1)
    qi0 = synth.indexer_query(np.random.default_rng(0), 16)
    ik, iks = ik.copy(), iks.copy()
    s0 = OI.scores(ik[:n_list[0]], iks[:n_list[0]], qi0, synth.head_weights(np.random.default_rng(1), 16), 1)
    best = int(np.argmax(s0))
    for a, cnt in ((3072, 90), (20000, 100)):
        ik[a:a + cnt] = ik[best]
        iks[a:a + cnt] = iks[best]
    q, qi, w, top, out, lse = run_full(kv, ik, iks, off, n_list, 64, 512, rng)
    check_full(kv, ik, iks, off, n_list, 512, q, qi, w, top, out, lse, "long lists")
