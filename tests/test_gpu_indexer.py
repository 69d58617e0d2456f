"""GPU parity of indexer scoring and top-k against the oracle."""
import numpy as np
import pytest

from oracle import cache as OC
from oracle import indexer as OI
from long_context_fp4_amd import synth
from tests.gpu_util import TOPK_SCORE_TOL, check_topk, dev, host

pytestmark = pytest.mark.gpu


def make_keys(rng, n_list, m=2):
    """Packed indexer rows of several sequences (oracle-written), concatenated."""
    w = synth.merge_weights(rng, m, 128)
    iks_all, ik_all = [], []
    for n in n_list:
        x = synth.hidden_host(rng, (n * m, 128))
        ik, iks = OC.quantize_indexer(OC.merge(x, w, m))
        ik_all.append(ik)
        iks_all.append(iks)
    off = np.concatenate([[0], np.cumsum(n_list)[:-1]]).astype(np.int64)
    return np.concatenate(ik_all), np.concatenate(iks_all), off


def run(ik, iks, off, n_list, max_n, q, w, mode, k, pool_k=0, cand=None):
    import torch
    import long_context_fp4_amd as L
    topk, pool, scores = L.indexer_topk(dev(ik), dev(iks), dev(off), dev(np.asarray(n_list, np.int32)), max_n,
                                        dev(q), None if w is None else dev(w), mode,
                                        cand=None if cand is None else dev(cand), k=k, pool_k=pool_k,
                                        want_scores=True)
    torch.cuda.synchronize()
    return host(topk), None if pool is None else host(pool), host(scores)


def check_sequence(ik, iks, off, n, q, w, mode, gpu_top, gpu_scores, k, gpu_pool=None, pool_k=0, what=""):
    rows = slice(off, off + n)
    s = OI.scores(ik[rows], iks[rows], q, w, mode) if n else np.zeros(0, np.float32)
    if n:
        np.testing.assert_allclose(gpu_scores[:n], s, rtol=2e-6, atol=2e-6, err_msg=what)
    pos = np.arange(n)
    if pool_k:
        opool = OI.topk(s, pos, pool_k)
        check_topk(gpu_pool, opool, lambda p: s[p], pool_k, what + " pool")
        # the GPU's top-k is taken from the GPU's pool
        gp = gpu_pool[gpu_pool >= 0]
        otop = OI.topk(s[gp], gp, k)
        assert set(gpu_top[gpu_top >= 0]) <= set(gp)
    else:
        otop = OI.topk(s, pos, k)
    check_topk(gpu_top, otop, lambda p: s[p], k, what)


def test_tiny_dot_score():
    w = synth.workload("tiny")
    p = synth.params(w)
    (x_lat, x_idx), = synth.hidden_states_host(w, p)
    _, ik, iks = OC.cache_write(x_lat, x_idx, p["w_lat"], p["w_idx"], w.m)
    L0 = p["layers"][0]
    n = ik.shape[0]
    top, _, sc = run(ik, iks, np.zeros(1, np.int64), [n], n, L0["q_idx"], None, 0, 512)
    check_sequence(ik, iks, 0, n, L0["q_idx"][0], None, 0, top[0], sc[0], 512, what="tiny")


@pytest.mark.parametrize("n_list,Hi,use_w", [([5000, 16384, 777], 16, True), ([16000, 3], 5, False),
                                             ([1, 512, 513], 16, True)])
def test_relu_w_short_sequences(n_list, Hi, use_w):
    rng = np.random.default_rng(sum(n_list) + Hi)
    ik, iks, off = make_keys(rng, n_list)
    B = len(n_list)
    q = np.stack([synth.indexer_query(rng, Hi) for _ in range(B)])
    w = np.stack([synth.head_weights(rng, Hi) for _ in range(B)]) if use_w else None
    max_n = max(n_list)
    top, _, sc = run(ik, iks, off, n_list, max_n, q, w, 1, 512)
    for b, n in enumerate(n_list):
        check_sequence(ik, iks, off[b], n, q[b], None if w is None else w[b], 1, top[b], sc[b], 512,
                       what=f"seq{b}")


@pytest.mark.parametrize("n_list,k", [([70000, 65536, 100000, 20000, 300, 0], 512), ([40000, 99999], 2048),
                                      ([65536] * 3, 1)])
def test_relu_w_long_sequences(n_list, k):
    rng = np.random.default_rng(len(n_list) * 7 + k)
    ik, iks, off = make_keys(rng, n_list)
    B = len(n_list)
    q = np.stack([synth.indexer_query(rng, 16) for _ in range(B)])
    w = np.stack([synth.head_weights(rng, 16) for _ in range(B)])
    top, _, sc = run(ik, iks, off, n_list, max(n_list), q, w, 1, k)
    for b, n in enumerate(n_list):
        check_sequence(ik, iks, off[b], n, q[b], w[b], 1, top[b], sc[b], k, what=f"seq{b}")


def test_pool_then_topk_and_reindex():
    rng = np.random.default_rng(11)
    n_list = [200000, 50000, 16384, 9000]
    ik, iks, off = make_keys(rng, n_list)
    B = len(n_list)
    q = np.stack([synth.indexer_query(rng, 16) for _ in range(B)])
    w = np.stack([synth.head_weights(rng, 16) for _ in range(B)])
    top, pool, sc = run(ik, iks, off, n_list, max(n_list), q, w, 1, 512, pool_k=16384)
    for b, n in enumerate(n_list):
        check_sequence(ik, iks, off[b], n, q[b], w[b], 1, top[b], sc[b], 512, gpu_pool=pool[b], pool_k=16384,
                       what=f"seq{b}")
    # Reindex: rescore the GPU pool with new queries
    q2 = np.stack([synth.indexer_query(rng, 16) for _ in range(B)])
    w2 = np.stack([synth.head_weights(rng, 16) for _ in range(B)])
    top2, _, sc2 = run(ik, iks, off, n_list, max(n_list), q2, w2, 1, 512, cand=pool)
    for b, n in enumerate(n_list):
        members = pool[b][pool[b] >= 0]
        rows = slice(off[b], off[b] + n)
        s_pool = OI.scores(ik[rows][members], iks[rows][members], q2[b], w2[b], 1)
        valid = pool[b] >= 0
        np.testing.assert_allclose(sc2[b][valid], s_pool, rtol=2e-6, atol=2e-6)
        otop, _ = OI.reindex_layer(ik[rows], iks[rows], pool[b], q2[b], w2[b], 1, k=512)
        lookup = dict(zip(members.tolist(), s_pool.tolist()))
        check_topk(top2[b], otop, lambda p: np.array([lookup[int(x)] for x in p], np.float32), 512,
                   f"reindex seq{b}")


def test_reindex_unordered_candidate_list():
    """A caller's candidate list out of order, with repeated and out-of-range positions:
    only the records (greater than every earlier in-range entry) are scored, the
    top-k is ascending and distinct, as the oracle's rule gives."""
    rng = np.random.default_rng(12)
    n_list = [30000, 5000]
    ik, iks, off = make_keys(rng, n_list)
    B, S = len(n_list), 9000
    cand = np.full((B, S), -1, np.int32)
    for b, n in enumerate(n_list):
        nb = min(6000, n - 500)
        base = np.sort(rng.choice(n, size=nb, replace=False)).astype(np.int32)
        lst = np.concatenate([base, base[rng.integers(0, nb, 1500)], rng.integers(-5, n + 50, 1500)])
        seg = rng.integers(0, len(lst) - 200)
        lst[seg:seg + 200] = rng.permutation(lst[seg:seg + 200])     # a shuffled stretch
        cand[b, :len(lst)] = lst
    q = np.stack([synth.indexer_query(rng, 16) for _ in range(B)])
    w = np.stack([synth.head_weights(rng, 16) for _ in range(B)])
    top, _, _ = run(ik, iks, off, n_list, max(n_list), q, w, 1, 512, cand=cand)
    for b, n in enumerate(n_list):
        rows = slice(off[b], off[b] + n)
        used = OI.used_candidates(cand[b], n)
        assert len(used) > 512
        s_used = OI.scores(ik[rows][used], iks[rows][used], q[b], w[b], 1)
        otop, _ = OI.reindex_layer(ik[rows], iks[rows], cand[b], q[b], w[b], 1, k=512)
        lookup = dict(zip(used.tolist(), s_used.tolist()))
        check_topk(top[b], otop, lambda p: np.array([lookup[int(x)] for x in p], np.float32), 512,
                   f"unordered cand seq{b}")


@pytest.mark.parametrize("n", [3000, 40000])
def test_exact_ties_take_the_lowest_positions(n):
    """Identical rows give identical scores: the top-k must be exactly positions 0..k-1."""
    rng = np.random.default_rng(n)
    ik1, iks1, _ = make_keys(rng, [1])
    ik = np.repeat(ik1, n, axis=0)
    iks = np.repeat(iks1, n, axis=0)
    q = synth.indexer_query(rng, 16)[None]
    w = synth.head_weights(rng, 16)[None]
    top, _, _ = run(ik, iks, np.zeros(1, np.int64), [n], n, q, w, 1, 512)
    assert np.array_equal(top[0], np.arange(512))
    # all-zero query: every score is +0
    top, _, sc = run(ik, iks, np.zeros(1, np.int64), [n], n, np.zeros_like(q), w, 1, 512)
    assert np.all(sc[0][:n] == 0) and np.array_equal(top[0], np.arange(512))


def run_no_scores(ik, iks, off, n_list, max_n, q, w, k):
    """Direct top-k without scores_out: the score pass keeps no scores."""
    import torch
    import long_context_fp4_amd as L
    topk, _, _ = L.indexer_topk(dev(ik), dev(iks), dev(off), dev(np.asarray(n_list, np.int32)), max_n,
                                dev(q), dev(w), 1, k=k, want_scores=False)
    torch.cuda.synchronize()
    return host(topk)


@pytest.mark.parametrize("n", [3000, 40000])
def test_ties_without_scores_out(n):
    """Identical rows overflow every candidate list: the finish falls back and
    recomputes the scores it was not given; the top-k is positions 0..k-1."""
    rng = np.random.default_rng(n + 1)
    ik1, iks1, _ = make_keys(rng, [1])
    ik = np.repeat(ik1, n, axis=0)
    iks = np.repeat(iks1, n, axis=0)
    q = synth.indexer_query(rng, 16)[None]
    w = synth.head_weights(rng, 16)[None]
    top = run_no_scores(ik, iks, np.zeros(1, np.int64), [n], n, q, w, 512)
    assert np.array_equal(top[0], np.arange(512))


def test_fallback_recomputes_scores():
    """The 700 largest keys sit in the first chunk (their E8M0 scales raised by
    2^6), so too few keys reach the highest local cutoff: the finish falls back
    to the full score set, which it recomputes (no scores_out)."""
    rng = np.random.default_rng(11)
    n = 40000
    ik, iks, off = make_keys(rng, [n])
    iks = iks.copy()
    iks[:700] = np.minimum(iks[:700].astype(np.int32) + 6, 254).astype(np.uint8)
    q = synth.indexer_query(rng, 16)[None]
    w = synth.head_weights(rng, 16)[None]
    top = run_no_scores(ik, iks, off, [n], n, q, w, 512)
    s = OI.scores(ik, iks, q[0], w[0], 1)
    check_topk(top[0], OI.topk(s, np.arange(n), 512), lambda p: s[p], 512, "fallback")
    # and with scores_out (stored scores), the same selection
    top2, _, sc = run(ik, iks, off, [n], n, q, w, 1, 512)
    np.testing.assert_allclose(sc[0][:n], s, rtol=2e-6, atol=2e-6)
    assert np.array_equal(top[0], top2[0])


def test_workspace_reuse_across_batch_sizes():
    """One workspace reused by calls whose B and max_n shrink and grow again.

    The workspace holds no state between calls: each call lays its regions out
    afresh and sets every counter it reads, whatever an earlier call left there.
    """
    import long_context_fp4_amd as L
    ws = L.Workspace()
    rng = np.random.default_rng(5)
    for n_list, k in (([70000, 65536, 100000, 20000, 300, 0], 512), ([40000, 99999], 2048),
                      ([65536] * 3, 1), ([30000] * 7, 64), ([17000], 512)):
        ik, iks, off = make_keys(rng, n_list)
        B = len(n_list)
        q = np.stack([synth.indexer_query(rng, 16) for _ in range(B)])
        w = np.stack([synth.head_weights(rng, 16) for _ in range(B)])
        import torch
        top, _, sc = L.indexer_topk(dev(ik), dev(iks), dev(off), dev(np.asarray(n_list, np.int32)), max(n_list),
                                    dev(q), dev(w), 1, k=k, want_scores=True, workspace=ws)
        torch.cuda.synchronize()
        top, sc = host(top), host(sc)
        for b, n in enumerate(n_list):
            check_sequence(ik, iks, off[b], n, q[b], w[b], 1, top[b], sc[b], k, what=f"B{B} seq{b}")


def test_long_lists_take_the_lds_path():
    """90 and 100 copies of the sequence's best row in two chunks: those chunks'
    lists hold more than 64 candidates (all tied at the cutoff), so the finish
    copies the lists to LDS instead of keeping them in registers; the tied keys
    are taken in position order."""
    rng = np.random.default_rng(31)
    n = 40000
    ik, iks, off = make_keys(rng, [n])
    q = synth.indexer_query(rng, 16)[None]
    w = synth.head_weights(rng, 16)[None]
    s0 = OI.scores(ik, iks, q[0], w[0], 1)
    best = int(np.argmax(s0))
    ik, iks = ik.copy(), iks.copy()
    for a, cnt in ((3072, 90), (20000, 100)):
        ik[a:a + cnt] = ik[best]
        iks[a:a + cnt] = iks[best]
    s = OI.scores(ik, iks, q[0], w[0], 1)
    want = OI.topk(s, np.arange(n), 512)
    for top in (run_no_scores(ik, iks, off, [n], n, q, w, 512)[0], run(ik, iks, off, [n], n, q, w, 1, 512)[0][0]):
        check_topk(top, want, lambda p: s[p], 512, "long lists")
        assert set(range(3072, 3162)) <= set(top.tolist()) and set(range(20000, 20100)) <= set(top.tolist())
