"""GPU parity of the quantized-query scoring variant (CSA2_SCORE_QMX8).

The variant quantizes each indexer query to MXFP8 and contracts it with the
MXFP4 keys on gfx950's block-scaled FP8 x FP4 matrix instruction. The oracle
computes the same scores exactly from the same quantized query
(oracle.indexer, flag SCORE_QMX8); the GPU's scores must lie within the
instruction's accumulation bound of them (qmx_bound), and every top-k swap
must lie within twice that bound of the k-th score.
"""
import numpy as np
import pytest

from oracle import attention as OA
from oracle import cache as OC
from oracle import indexer as OI
from long_context_fp4_amd import synth
from tests.gpu_util import ATTN_REL_TOL, attn_rel_err, check_topk, dev, host

pytestmark = pytest.mark.gpu

QMX = OI.SCORE_QMX8


def qmx_bound(ik_rows, iks_rows, q_bits, w, mode):
    """Per-entry bound on |GPU score - oracle score| for the variant.

    The block-scaled instruction aligns each product of a group of 8
    consecutive channels to the binade E of the group's largest |product| and
    keeps its bits down to 2^(E - 13), dropping the rest toward zero; the group
    sums are then added (measured with single large and small products, both
    signs, and sums of small ones). A product's error is thus below
    min(|p|, 2^(E - 13)); the bound takes min(|p|, 2^(E - 12)) (one bit of
    margin) plus 2^-20 of the sum of |products| for the f32 additions, the head
    weights and the oracle's one rounding. ReLU does not increase a
    difference, so the head sum's bound is the w-weighted sum of the heads'.
    """
    k = OC.dequant_indexer(ik_rows, iks_rows)
    qd = OI.dequant_query_mx(*OI.quantize_query_mx(q_bits))
    hi = qd.shape[0]
    base = mode & ~QMX
    wh = np.zeros(hi)
    if base == OI.SCORE_DOT:
        wh[0] = 1.0
    else:
        wh[:] = 1.0 if w is None else np.asarray(w, np.float32).astype(np.float64)
    out = np.empty(k.shape[0])
    for a in range(0, k.shape[0], 2048):
        p = np.abs(k[a:a + 2048, None, :] * qd[None, :, :])            # [c, Hi, 128]
        pg = p.reshape(p.shape[0], hi, 16, 8)
        g = pg.max(axis=3, keepdims=True)
        e = np.floor(np.log2(np.where(g > 0, g, 1.0)))
        per = np.minimum(pg, np.exp2(e - 12)).sum(axis=(2, 3))
        out[a:a + 2048] = (per + 2.0 ** -20 * p.sum(axis=2)) @ wh
    return out


def make_keys(rng, n_list, m=2):
    w = synth.merge_weights(rng, m, 128)
    parts = [OC.quantize_indexer(OC.merge(synth.hidden_host(rng, (n * m, 128)), w, m)) for n in n_list]
    off = np.concatenate([[0], np.cumsum(n_list)[:-1]]).astype(np.int64)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]), off


def check_scores(gpu, ik_rows, iks_rows, q, w, mode, what):
    s = OI.scores(ik_rows, iks_rows, q, w, mode)
    bound = qmx_bound(ik_rows, iks_rows, q, w, mode)
    err = np.abs(gpu.astype(np.float64) - s.astype(np.float64))
    assert np.all(err[bound == 0] == 0), f"{what}: an all-zero contraction must score exactly"
    nz = bound > 0
    worst = np.max(err[nz] / bound[nz]) if nz.any() else 0.0
    print(f"{what}: largest error {worst:.3g} of the bound, {err.max():.3g} absolute")
    assert worst <= 1.0, f"{what}: error reaches {worst:.3g} of the bound"
    return s, bound


@pytest.mark.parametrize("mode,Hi,k", [(OI.SCORE_RELU_W, 16, 512), (OI.SCORE_DOT, 1, 64), (OI.SCORE_RELU_W, 5, 100)])
def test_qmx_full_scores_and_top_k(mode, Hi, k):
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(61 + Hi)
    n_list = [20000, 3001, 0, 700]
    ik, iks, off = make_keys(rng, n_list)
    B = len(n_list)
    q = np.stack([synth.indexer_query(rng, Hi) for _ in range(B)])
    w = np.stack([synth.head_weights(rng, Hi) for _ in range(B)]) if Hi > 1 else None
    top, _, sc = L.indexer_topk(dev(ik), dev(iks), dev(off), dev(np.asarray(n_list, np.int32)), max(n_list),
                                dev(q), None if w is None else dev(w), mode | QMX, k=k, want_scores=True)
    torch.cuda.synchronize()
    top, sc = host(top), host(sc)
    for b, n in enumerate(n_list):
        rows = slice(off[b], off[b] + n)
        if n == 0:
            assert np.all(top[b] == -1)
            continue
        wb = None if w is None else w[b]
        s, bound = check_scores(sc[b][:n], ik[rows], iks[rows], q[b], wb, mode | QMX, f"seq {b}")
        exact = OI.scores(ik[rows], iks[rows], q[b], wb, mode)
        assert np.abs(sc[b][:n].astype(np.float64) - exact).max() > 1e-4, "the variant's scores must differ"
        check_topk(top[b], OI.topk(s, np.arange(n), k), lambda p: s[p], k, f"seq {b}", tol=2 * bound.max())


def test_qmx_pool_then_reindex():
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(67)
    n_list = [30000, 9000]
    ik, iks, off = make_keys(rng, n_list)
    B, k, pool_k = len(n_list), 512, 4096
    q = np.stack([synth.indexer_query(rng, 16) for _ in range(B)])
    w = np.stack([synth.head_weights(rng, 16) for _ in range(B)])
    mode = OI.SCORE_RELU_W | QMX
    ne = dev(np.asarray(n_list, np.int32))
    top, pool, sc = L.indexer_topk(dev(ik), dev(iks), dev(off), ne, max(n_list), dev(q), dev(w), mode, k=k,
                                   pool_k=pool_k, want_scores=True)
    q2 = np.stack([synth.indexer_query(rng, 16) for _ in range(B)])
    top2, _, sc2 = L.indexer_topk(dev(ik), dev(iks), dev(off), ne, max(n_list), dev(q2), dev(w), mode,
                                  cand=pool, k=k, want_scores=True)
    torch.cuda.synchronize()
    top, pool, sc, top2, sc2 = host(top), host(pool), host(sc), host(top2), host(sc2)
    for b, n in enumerate(n_list):
        rows = slice(off[b], off[b] + n)
        s, bound = check_scores(sc[b][:n], ik[rows], iks[rows], q[b], w[b], mode, f"full seq {b}")
        tol = 2 * bound.max()
        check_topk(pool[b], OI.topk(s, np.arange(n), pool_k), lambda p: s[p], pool_k, f"pool seq {b}", tol=tol)
        gp = pool[b][pool[b] >= 0]
        check_topk(top[b], OI.topk(s[gp], gp, k), lambda p: s[p], k, f"top seq {b}", tol=tol)
        # Reindex: the pool's rows rescored with the second query
        s2, b2 = check_scores(sc2[b][:len(gp)], ik[rows][gp], iks[rows][gp], q2[b], w[b], mode, f"reindex seq {b}")
        full2 = np.full(n, -np.inf, np.float32)
        full2[gp] = s2
        check_topk(top2[b], OI.topk(s2, gp, k), lambda p: full2[p], k, f"reindex top seq {b}", tol=2 * b2.max())


def test_qmx_decode_layer_fused_and_fallback():
    """A Full decode layer with the variant: the top-k is finished inside the
    attention launch; sequence 1's largest keys are packed into its first
    chunk, so its attention workgroups recompute the variant's scores."""
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(71)
    n_list = [40000, 30000, 17000]
    m = 1
    w_lat, w_idx = synth.merge_weights(rng, m, 512), synth.merge_weights(rng, m, 128)
    parts = [OC.cache_write(synth.hidden_host(rng, (n, 512)), synth.hidden_host(rng, (n, 128)), w_lat, w_idx, m)
             for n in n_list]
    kv, ik, iks = (np.concatenate([p[i] for p in parts]) for i in range(3))
    off = np.concatenate([[0], np.cumsum(n_list)[:-1]]).astype(np.int64)
    iks = iks.copy()
    iks[off[1]:off[1] + 700] = np.minimum(iks[off[1]:off[1] + 700].astype(np.int32) + 6, 254).astype(np.uint8)
    B, H, k = len(n_list), 64, 512
    q = np.stack([synth.latent_query(rng, H) for _ in range(B)])
    qi = np.stack([synth.indexer_query(rng, 16) for _ in range(B)])
    w = np.stack([synth.head_weights(rng, 16) for _ in range(B)])
    mode = OI.SCORE_RELU_W | QMX
    top, _, out, lse = L.decode_layer(L.CSA2_FULL, dev(kv), dev(ik), dev(iks), dev(off),
                                      dev(np.asarray(n_list, np.int32)), max(n_list), dev(q), q_idx=dev(qi),
                                      w=dev(w), score_mode=mode, k=k)
    torch.cuda.synchronize()
    top, out, lse = host(top), host(out), host(lse)
    for b, n in enumerate(n_list):
        rows = slice(off[b], off[b] + n)
        s = OI.scores(ik[rows], iks[rows], qi[b], w[b], mode)
        bound = qmx_bound(ik[rows], iks[rows], qi[b], w[b], mode)
        check_topk(top[b], OI.topk(s, np.arange(n), k), lambda p: s[p], k, f"seq {b}", tol=2 * bound.max())
        ro, rl = OA.sparse_attention(kv[rows], top[b], q[b])
        err = attn_rel_err(out[b], ro)
        assert np.all(err <= ATTN_REL_TOL), f"seq {b}: attention max rel err {err.max():.3g}"
        assert np.all(np.abs(lse[b] - rl) <= 2e-3), f"seq {b}: lse"


def test_qmx_fallback_recomputes_the_variant_scores():
    """The 700 largest keys sit in the first chunk, so the finish launch falls
    back to the full score set, which it recomputes with the quantized query
    (no scores stored); the selection must equal the one taken on the stored
    scores of the same variant."""
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(73)
    n = 40000
    ik, iks, off = make_keys(rng, [n])
    iks = iks.copy()
    iks[:700] = np.minimum(iks[:700].astype(np.int32) + 6, 254).astype(np.uint8)
    q = synth.indexer_query(rng, 16)[None]
    w = synth.head_weights(rng, 16)[None]
    mode = OI.SCORE_RELU_W | QMX
    args = (dev(ik), dev(iks), dev(off), dev(np.asarray([n], np.int32)), n, dev(q), dev(w), mode)
    top, _, _ = L.indexer_topk(*args, k=512)
    top2, _, sc = L.indexer_topk(*args, k=512, want_scores=True)
    torch.cuda.synchronize()
    top, top2, sc = host(top), host(top2), host(sc)
    s, bound = check_scores(sc[0][:n], ik, iks, q[0], w[0], mode, "stored")
    check_topk(top[0], OI.topk(s, np.arange(n), 512), lambda p: s[p], 512, "fallback", tol=2 * bound.max())
    assert np.array_equal(top[0], top2[0])


def test_qmx_extreme_query_magnitudes():
    """Heads whose binary exponents are lowered by 118 (blocks whose shared
    exponent clamps at -127) and by 60, or raised by 40, an all-zero head and a
    head with a single non-zero value: the variant's scores stay within the
    bound of the oracle's."""
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(79)
    n = 5000
    ik, iks, off = make_keys(rng, [n])
    qb = synth.indexer_query(rng, 16).astype(np.uint16).copy()

    def shift(bits, d):
        """bf16 bits with the exponent field moved by d; values leaving the normal range become 0."""
        e = (bits.astype(np.int32) >> 7) & 0xFF
        ne = e + d
        out = (bits & 0x807F) | (np.clip(ne, 0, 254).astype(np.uint16) << 7)
        return np.where((e == 0) | (ne < 1), bits & 0x8000, out).astype(np.uint16)

    qb[0] = shift(qb[0], -118)
    qb[1] = shift(qb[1], -60)
    qb[2] = shift(qb[2], 40)
    qb[3] = 0
    qb[4] = 0
    qb[4, 77] = 0xC040                                   # -3.0
    w = synth.head_weights(rng, 16)
    mode = OI.SCORE_RELU_W | QMX
    _, _, sc = L.indexer_topk(dev(ik), dev(iks), dev(off), dev(np.asarray([n], np.int32)), n, dev(qb[None]),
                              dev(w[None]), mode, k=64, want_scores=True)
    torch.cuda.synchronize()
    check_scores(host(sc)[0][:n], ik, iks, qb, w, mode, "extreme magnitudes")
    # the clamped block exponent really occurs in head 0
    _, sbytes = OI.quantize_query_mx(qb)
    assert np.any(sbytes[0] == 0)
