"""Pins of scoring, top-k and attention: one-hot and brute-force cases, textbook routines."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import cache as C
from oracle import formats as F
from oracle import indexer as I
from oracle import modes as M
from long_context_fp4_amd import synth


def random_cache(rng, n, m=2):
    x_lat = synth.hidden_host(rng, (n * m, 512))
    x_idx = synth.hidden_host(rng, (n * m, 128))
    w_lat = synth.merge_weights(rng, m, 512)
    w_idx = synth.merge_weights(rng, m, 128)
    return C.cache_write(x_lat, x_idx, w_lat, w_idx, m)


def decode_key_by_hand(ik_row, iks_row):
    """Nibble-by-nibble decode in plain Python (independent of the oracle's array code)."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    out = []
    for c in range(128):
        byte = int(ik_row[c // 2])
        nib = (byte >> 4) if c % 2 else (byte & 0xF)
        v = grid[nib & 7] * (-1.0 if nib & 8 else 1.0)
        out.append(v * 2.0 ** (int(iks_row[c // 32]) - 127))
    return out


def test_one_hot_query_selects_a_key_channel():
    rng = np.random.default_rng(1)
    _, ik, iks = random_cache(rng, 40)
    for c in (0, 1, 31, 32, 77, 127):
        q = np.zeros((1, 128), np.float32)
        q[0, c] = 1.0
        s = I.scores(ik, iks, synth.bf16_bits(q), None, I.SCORE_DOT)
        want = [decode_key_by_hand(ik[i], iks[i])[c] for i in range(40)]
        assert np.array_equal(s, np.float32(want))


def test_relu_weighted_score_brute_force():
    rng = np.random.default_rng(2)
    _, ik, iks = random_cache(rng, 30)
    q = synth.indexer_query(rng, 16)
    w = synth.head_weights(rng, 16)
    s = I.scores(ik, iks, q, w, I.SCORE_RELU_W)
    qf = F.bf16_bits_to_float(q)
    for i in range(30):
        k = decode_key_by_hand(ik[i], iks[i])
        tot = 0.0
        for h in range(16):
            d = sum(float(qf[h, c]) * k[c] for c in range(128))
            tot += float(w[h]) * max(0.0, d)
        assert abs(float(s[i]) - tot) <= 1e-6 * max(1.0, abs(tot))
    # ReLU: a head whose dot products are all negative contributes nothing
    s_neg = I.scores(ik, iks, q, w * 0, I.SCORE_RELU_W)
    assert np.all(s_neg == 0)


def test_topk_is_the_head_of_a_full_stable_sort():
    rng = np.random.default_rng(3)
    s = rng.integers(0, 50, size=3000).astype(np.float32)     # many exact ties
    pos = np.arange(3000)
    ref = sorted(range(3000), key=lambda i: (-float(s[i]), i))
    for k in (1, 17, 512, 2999, 3000, 4000):
        got = I.topk(s, pos, k)
        want = sorted(ref[:k])
        assert list(got[: len(want)]) == want
        assert np.all(got[len(want):] == -1)


def test_full_topk_is_inside_the_pool_and_reindex_with_same_query_agrees():
    rng = np.random.default_rng(4)
    kv, ik, iks = random_cache(rng, 3000)
    q_idx = synth.indexer_query(rng, 16)
    w = synth.head_weights(rng, 16)
    top, pool, s = I.full_layer(ik, iks, q_idx, w, I.SCORE_RELU_W, k=512, pool_k=1024)
    assert set(top) <= set(pool)
    assert np.array_equal(top, I.topk(s, np.arange(3000), 512))
    top2, _ = I.reindex_layer(ik, iks, pool, q_idx, w, I.SCORE_RELU_W, k=512)
    assert np.array_equal(top, top2)


def test_used_candidates_rule():
    """A pool (distinct, ascending, -1 padded) passes unchanged; for any list the used
    entries are the left-to-right records among the in-range ones, checked against an
    O(n^2) brute force over every prefix."""
    pool = np.array([2, 5, 9, 40, -1, -1])
    assert list(I.used_candidates(pool, 50)) == [2, 5, 9, 40]
    assert list(I.used_candidates(pool, 10)) == [2, 5, 9]          # 40 is out of range
    rng = np.random.default_rng(8)
    for trial in range(20):
        n = int(rng.integers(1, 60))
        lst = rng.integers(-3, n + 5, size=int(rng.integers(0, 80)))
        got = list(I.used_candidates(lst, n))
        want = [int(c) for i, c in enumerate(lst)
                if 0 <= c < n and all(not (0 <= d < n) or d < c for d in lst[:i])]
        assert got == want
        assert all(a < b for a, b in zip(got, got[1:]))            # distinct, ascending


def test_dense_attention_matches_torch_sdpa():
    rng = np.random.default_rng(5)
    kv, _, _ = random_cache(rng, 300)
    q = synth.latent_query(rng, 8)
    for tau in (1.0, 0.37):
        out, lse = A.sparse_attention(kv, np.arange(300), q, tau)
        c = torch.from_numpy(C.dequant_latent(kv))
        qt = torch.from_numpy(F.bf16_bits_to_float(q).astype(np.float64))
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[None, :, None, :], c[None, None].expand(1, 8, 300, 512),
            c[None, None].expand(1, 8, 300, 512), scale=tau)[0, :, 0, :]
        assert torch.allclose(torch.from_numpy(out), ref, rtol=1e-12, atol=1e-12)
        lse_ref = torch.logsumexp(tau * qt @ c.T, dim=1)
        assert np.allclose(lse, lse_ref.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(6)
    kv, _, _ = random_cache(rng, 50)
    q = synth.latent_query(rng, 4)
    c = C.dequant_latent(kv)
    # one selected entry: output is that latent, lse is its logit
    out, lse = A.sparse_attention(kv, np.array([-1, 7, -1]), q)
    assert np.array_equal(out, np.broadcast_to(c[7], (4, 512)))
    assert np.allclose(lse, F.bf16_bits_to_float(q).astype(np.float64) @ c[7])
    # zero query: equal logits give the mean, lse = log(k)
    out, lse = A.sparse_attention(kv, np.arange(0, 50, 5), np.zeros((2, 512), np.uint16))
    assert np.allclose(out, c[0:50:5].mean(axis=0)[None], rtol=1e-14, atol=1e-14)
    assert np.allclose(lse, np.log(10))
    # order of the indices does not matter
    perm = rng.permutation(50)
    o1, l1 = A.sparse_attention(kv, np.arange(50), q)
    o2, l2 = A.sparse_attention(kv, perm, q)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-13) and np.allclose(l1, l2, rtol=1e-13)
    # no valid index
    out, lse = A.sparse_attention(kv, np.array([-1, -1]), q)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_modes_reuse_with_zero_noise_equals_source_layer():
    rng = np.random.default_rng(7)
    kv, ik, iks = random_cache(rng, 2500)
    mk = lambda: {"q_idx": synth.indexer_query(rng, 16), "w": synth.head_weights(rng, 16),
                  "q": synth.latent_query(rng, 16)}
    full, rei = mk(), mk()
    layers = [dict(mode=M.FULL, **full), dict(mode=M.REINDEX, **rei),
              dict(mode=M.REUSE, q=rei["q"]), dict(mode=M.REUSE, q=synth.perturb(rng, rei["q"], 0.01))]
    res = M.decode_group(kv, ik, iks, layers, k=512, pool_k=2048)
    assert np.array_equal(res[2]["topk"], res[1]["topk"])
    assert np.array_equal(res[3]["topk"], res[1]["topk"])
    assert np.array_equal(res[2]["out"], res[1]["out"])
    assert not np.array_equal(res[3]["out"], res[1]["out"])
    assert set(res[1]["topk"]) <= set(res[0]["pool"])
