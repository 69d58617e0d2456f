"""GPU parity of the sliding-window branch against the oracle: the FP8 ring write
(bit-exact) and the window attention merged with the sparse branch."""
import numpy as np
import pytest

from oracle import attention as OA
from oracle import cache as OC
from oracle import swa as OS
from long_context_fp4_amd import synth
from tests.gpu_util import ATTN_REL_TOL, attn_rel_err, dev, host

pytestmark = pytest.mark.gpu


def window_rows(rng, B, T, spread=False):
    x = synth.hidden_host(rng, (B, T, 512))
    if spread:
        # magnitudes from 1e-4 to 1e4, all-zero and negative-zero blocks
        xf = (x.astype(np.uint32) << 16).view(np.float32).copy()
        xf *= np.exp(rng.uniform(-9, 9, (B, T, 1))).astype(np.float32)
        xf[:, ::7, 32:48] = 0.0
        xf[:, ::11, 64:80] = -0.0
        x = synth.bf16_bits(xf)
    return x


@pytest.mark.parametrize("T,spread", [(1, False), (77, False), (300, True)])
def test_window_write_bit_exact(T, spread):
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(T)
    B = 3
    x = window_rows(rng, B, T, spread)
    pos0 = np.array([0, 5, 130], np.int64)
    ring0 = rng.integers(0, 256, (B, 128, 544), dtype=np.uint8)
    win = dev(ring0)
    L.swa_write(dev(x), dev(pos0), win)
    torch.cuda.synchronize()
    got = host(win)
    for b in range(B):
        want = OS.window_write(x[b], int(pos0[b]), ring=ring0[b])
        assert np.array_equal(got[b], want), f"seq {b}"


@pytest.mark.parametrize("H", [64, 20])
def test_window_attention_merged_with_the_sparse_branch(H):
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(H)
    n_list = [3000, 2000, 2500, 1000]
    B, k = len(n_list), 256
    w_lat = synth.merge_weights(rng, 1, 512)
    w_idx = synth.merge_weights(rng, 1, 128)
    parts = [OC.cache_write(synth.hidden_host(rng, (n, 512)), synth.hidden_host(rng, (n, 128)), w_lat, w_idx, 1)
             for n in n_list]
    kv = np.concatenate([p[0] for p in parts])
    off = np.concatenate([[0], np.cumsum(n_list)[:-1]]).astype(np.int64)
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)).astype(np.int32) for n in n_list])
    idx[1, 200:] = -1                           # a short selection
    idx[3, :] = -1                              # no sparse entry: the window alone
    q = np.stack([synth.latent_query(rng, H) for _ in range(B)])
    out, lse = L.sparse_attention(dev(kv), dev(off), dev(np.asarray(n_list, np.int32)), dev(idx), dev(q))
    T = np.array([300, 77, 1, 0])                # tokens in the window of each sequence
    n_win = np.minimum(T, 128).astype(np.int32)
    xs = [window_rows(rng, 1, max(int(t), 1))[0] for t in T]
    win = torch.zeros((B, 128, 544), dtype=torch.uint8, device="cuda")
    for b in range(B):
        if T[b]:
            L.swa_write(dev(xs[b])[None], dev(np.zeros(1, np.int64)), win[b:b + 1])
    L.swa_attention(win, dev(n_win), dev(q), out, lse)
    torch.cuda.synchronize()
    out, lse = host(out), host(lse)
    for b in range(B):
        o_s, l_s = OA.sparse_attention(kv[off[b]:off[b] + n_list[b]], idx[b], q[b])
        ring = OS.window_write(xs[b][: T[b]], 0) if T[b] else np.zeros((128, 544), np.uint8)
        o_w, l_w = OS.window_attention(ring[: n_win[b]], q[b])
        o, l = OS.merge_branches(o_s, l_s, o_w, l_w)
        err = attn_rel_err(out[b], o)
        assert np.all(err <= ATTN_REL_TOL), f"seq {b}: max rel err {err.max():.3g}"
        fin = np.isfinite(l)
        assert np.array_equal(fin, np.isfinite(lse[b])), f"seq {b}: lse finiteness"
        assert np.all(np.abs(lse[b][fin] - l[fin]) <= 2e-3), f"seq {b}: lse"
