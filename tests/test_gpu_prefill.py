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
    B, Tq, H = len(T_list), 5, 32
    pos = np.stack([np.array([0, 2 * k - 1, T // 3, T - 2, T - 1], np.int64) for T in T_list])
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
            s = OI.scores(ik[rows], iks[rows], qi[b, t], w[b, t], 1) if nv else np.zeros(0, np.float32)
            want = OI.topk(s, np.arange(nv), k)
            check_topk(top[b, t], want, lambda p: s[p], k, f"seq {b} query {t}")
            ro, rl = OA.sparse_attention(kv[off[b]:off[b] + E[b]], top[b, t], q[b, t])
            err = attn_rel_err(out[b, t], ro)
            assert np.all(err <= ATTN_REL_TOL), f"seq {b} query {t}: max rel err {err.max():.3g}"
            fin = np.isfinite(rl)
            assert np.array_equal(fin, np.isfinite(lse[b, t]))
            assert np.all(np.abs(lse[b, t][fin] - rl[fin]) <= 2e-3), f"seq {b} query {t}: lse"
