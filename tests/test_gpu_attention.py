"""GPU parity of the gather-dequant sparse attention against the oracle (float64)."""
import numpy as np
import pytest

from oracle import attention as OA
from oracle import cache as OC
from long_context_fp4_amd import synth
from tests.gpu_util import ATTN_REL_TOL, attn_rel_err, dev, host

pytestmark = pytest.mark.gpu


def make_latent(rng, n, m=2, scale_exp=None):
    x = rng.standard_normal((n * m, 512), dtype=np.float32)
    if scale_exp is not None:
        x = (x * np.ldexp(1.0, scale_exp)).astype(np.float32)
    w = synth.merge_weights(rng, m, 512)
    return OC.quantize_latent(OC.merge(synth.bf16_bits(x), w, m))


def run(kv, off, n_list, idx, q, tau=1.0):
    import torch
    import long_context_fp4_amd as L
    out, lse = L.sparse_attention(dev(kv), dev(off), dev(np.asarray(n_list, np.int32)), dev(idx), dev(q), tau)
    torch.cuda.synchronize()
    return host(out), host(lse)


def check(kv, off, n_list, idx, q, out, lse, tau=1.0, what=""):
    for b, n in enumerate(n_list):
        rows = kv[off[b]: off[b] + n]
        sel = np.where((idx[b] >= 0) & (idx[b] < n), idx[b], -1)
        ro, rl = OA.sparse_attention(rows, sel, q[b], tau)
        err = attn_rel_err(out[b], ro)
        assert np.all(err <= ATTN_REL_TOL), f"{what} seq{b}: max rel err {err.max():.3g}"
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(lse[b])), what
        assert np.all(np.abs(lse[b][fin] - rl[fin]) <= 2e-3), f"{what} seq{b}: lse"


def test_tiny_workload_heads8():
    w = synth.workload("tiny")
    p = synth.params(w)
    (x_lat, x_idx), = synth.hidden_states_host(w, p)
    kv, _, _ = OC.cache_write(x_lat, x_idx, p["w_lat"], p["w_idx"], w.m)
    rng = np.random.default_rng(0)
    idx = np.sort(rng.choice(kv.shape[0], size=512, replace=False)).astype(np.int32)[None]
    q = p["layers"][0]["q"]
    out, lse = run(kv, np.zeros(1, np.int64), [kv.shape[0]], idx, q)
    check(kv, np.zeros(1, np.int64), [kv.shape[0]], idx, q, out, lse, what="tiny")


@pytest.mark.parametrize("B,H,k", [(1, 64, 512), (4, 64, 512), (32, 64, 512), (3, 16, 100), (2, 128, 2048),
                                   (5, 1, 17), (2, 24, 1)])
def test_shapes(B, H, k):
    rng = np.random.default_rng(B * 1000 + H + k)
    n_list = [int(v) for v in rng.integers(max(k, 600), 3000, size=B)]
    kv = np.concatenate([make_latent(rng, n) for n in n_list])
    off = np.concatenate([[0], np.cumsum(n_list)[:-1]]).astype(np.int64)
    idx = np.stack([np.sort(rng.choice(n, size=k, replace=False)) for n in n_list]).astype(np.int32)
    # padding and out-of-range entries are skipped
    if k >= 8:
        idx[0, -3:] = -1
        idx[-1, 1] = n_list[-1] + 5
    q = np.stack([synth.latent_query(rng, H) for _ in range(B)])
    out, lse = run(kv, off, n_list, idx, q)
    check(kv, off, n_list, idx, q, out, lse, what=f"B{B}H{H}k{k}")


def test_degenerate_index_lists():
    rng = np.random.default_rng(3)
    kv = make_latent(rng, 1000)
    off = np.zeros(3, np.int64)
    n_list = [1000, 1000, 1000]
    idx = np.full((3, 64), -1, np.int32)
    idx[1, 10] = 123                       # a single valid entry
    idx[2, :] = 77                         # the same entry 64 times
    q = np.stack([synth.latent_query(rng, 16) for _ in range(3)])
    out, lse = run(kv, off, n_list, idx, q)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    c = OC.dequant_latent(kv[123:124])[0]
    np.testing.assert_allclose(out[1], np.broadcast_to(c, (16, 512)), rtol=0, atol=1e-6 * np.abs(c).max())
    c = OC.dequant_latent(kv[77:78])[0]
    np.testing.assert_allclose(out[2], np.broadcast_to(c, (16, 512)), rtol=0, atol=1e-6 * np.abs(c).max())
    check(kv, off, n_list, idx, q, out, lse, what="degenerate")


@pytest.mark.parametrize("scale_exp,tau", [(-9, 1.0), (-7, 1.0), (10, 0.05), (0, 3.0)])
def test_scale_ranges(scale_exp, tau):
    """Subnormal and saturated E4M3 scales, and sharp softmaxes."""
    rng = np.random.default_rng(scale_exp + 100)
    kv = make_latent(rng, 2000, scale_exp=scale_exp)
    idx = np.sort(rng.choice(2000, size=512, replace=False)).astype(np.int32)[None]
    q = synth.latent_query(rng, 64)[None]
    out, lse = run(kv, np.zeros(1, np.int64), [2000], idx, q, tau)
    check(kv, np.zeros(1, np.int64), [2000], idx, q, out, lse, tau, what=f"exp{scale_exp}")
