"""Helpers of the GPU parity tests: device transfer and the parity rules."""
import numpy as np

TOPK_SCORE_TOL = 1e-5      # swaps allowed among entries within this of the k-th oracle score
ATTN_REL_TOL = 2e-3        # max |o - r| / max |r| per (sequence, head) row


def torch_mod():
    import torch
    return torch


def dev(a):
    """numpy array -> GPU tensor (uint16 bf16 bits become int16)."""
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t):
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def check_topk(gpu_sel, oracle_sel, oracle_scores_of, k, what="", tol=TOPK_SCORE_TOL):
    """gpu_sel / oracle_sel: int arrays of k positions (ascending, -1 padded).

    oracle_scores_of(positions) -> float32 oracle scores. Sets must be equal
    except for swaps among positions whose oracle score lies within tol
    (TOPK_SCORE_TOL unless the scores carry a larger error bound) of the k-th
    best oracle score.
    """
    g = np.asarray(gpu_sel)
    o = np.asarray(oracle_sel)
    assert g.shape == o.shape == (k,), what
    gv, ov = g[g >= 0], o[o >= 0]
    assert np.all(np.diff(gv) > 0), f"{what}: GPU selection not strictly ascending"
    assert np.all(g[len(gv):] == -1), f"{what}: padding must follow the selected positions"
    assert len(gv) == len(ov), f"{what}: {len(gv)} selected vs {len(ov)}"
    diff = np.setxor1d(gv, ov)
    if diff.size == 0:
        return 0
    kth = np.min(oracle_scores_of(ov).astype(np.float64))
    ds = oracle_scores_of(diff).astype(np.float64)
    bad = np.abs(ds - kth) > tol
    assert not np.any(bad), f"{what}: {bad.sum()} swapped positions beyond the tie tolerance"
    return diff.size


def attn_rel_err(out, ref):
    """Row-wise max |o - r| / max |r| over [..., 512]."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(out - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)
