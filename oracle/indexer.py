"""Indexer scoring and top-k selection over the compressed cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

[FP4] section "Les ingrédients": the 128-channel indexer key is what scores
cached positions. [CS] section "L'architecture : trois leviers contre le
cache": a Full layer computes new top-512 indices with its own indexer; a
hierarchical sparse indexer caps the candidates at 16384 positions. [F24]
section "Tre meccanismi al posto di un solo trucco": deeper indexing layers
only look at the candidate pool that the first Full layer built.

Readings taken (the pages give no score formula):

* RELU_W score: S_i = sum_h w_h * max(0, q_h . k_i) over the indexer heads;
  DOT score (one head): S_i = q . k_i. k_i is the exact dequantized key,
  q_h the bf16 query. Computed in float64 and rounded once to float32; the
  selection then works on those float32 values, the precision the hot path
  keeps its scores in.
* Order: score descending, ties broken by the lower position. The selected
  positions are returned in ascending order, padded with -1 when fewer than
  k positions exist.
* Pool: the top-16384 positions by the same order (all positions when there
  are at most 16384). The Full layer's top-512 is taken from that pool.
* Reindex: the shared indexer key rows of the pool positions are rescored
  with the layer's own query and weights; its top-512 is taken from the pool.
* Quantized-query variant (flag SCORE_QMX8): the query is first converted to
  MXFP8 (quantize_query_mx), the input that block-scaled FP8 x FP4 matrix
  instructions take; the score is the same formula over those exact values.
"""
import numpy as np

from .cache import dequant_indexer
from .formats import bf16_bits_to_float, e4m3fn_decode, e4m3fn_round, e8m0_decode

SCORE_DOT = 0
SCORE_RELU_W = 1
SCORE_QMX8 = 0x100     # flag on either mode: the query is first quantized to MXFP8
MX_BLOCK = 32
E4M3_EMAX = 8          # largest E4M3FN binade: 448 = 1.75 * 2**8


def scores(ik_rows, iks_rows, q_idx_bits, w=None, mode=SCORE_RELU_W):
    """Scores of the given indexer rows. q_idx_bits: uint16 [Hi, 128]; w: float32 [Hi] or None (= 1).

    mode is SCORE_DOT or SCORE_RELU_W, optionally with the SCORE_QMX8 flag
    (then the query is replaced by its MXFP8 quantization, see
    quantize_query_mx, before the same exact arithmetic). Returns float32 [n].
    """
    k = dequant_indexer(ik_rows, iks_rows)                       # float64 [n, 128]
    if mode & SCORE_QMX8:
        q = dequant_query_mx(*quantize_query_mx(q_idx_bits))     # [Hi, 128], exact values
        mode &= ~SCORE_QMX8
    else:
        q = bf16_bits_to_float(q_idx_bits).astype(np.float64)    # [Hi, 128]
    d = k @ q.T                                                  # [n, Hi]
    if mode == SCORE_DOT:
        if q.shape[0] != 1:
            raise ValueError("DOT score takes exactly one indexer head")
        s = d[:, 0]
    elif mode == SCORE_RELU_W:
        wh = np.ones(q.shape[0]) if w is None else np.asarray(w, np.float32).astype(np.float64)
        s = np.maximum(d, 0.0) @ wh
    else:
        raise ValueError("unknown score mode")
    return s.astype(np.float32)


def quantize_query_mx(q_idx_bits):
    """bf16 indexer queries [Hi, 128] -> MXFP8: (E4M3FN bytes uint8 [Hi, 128], E8M0 bytes uint8 [Hi, 4]).

    The variant that feeds gfx950's block-scaled MFMA ([FP4] section "Le coût
    d'une entrée": the keys are standard MXFP4, E2M1 values with one E8M0
    scale per 32 channels). Reading taken for the query: the same OCP MX v1.0
    conversion with E4M3FN elements. Per block of 32 channels,
    X = floor(log2 amax) - 8 (8 = E4M3FN's largest exponent), clamped to
    [-127, 127]; a block whose amax is 0 takes X = -127. Each value becomes
    the nearest-even E4M3FN magnitude of |x| * 2^-X (an exact rescaling),
    saturating at 448, with the sign bit of x. The scale byte is X + 127.
    """
    x = bf16_bits_to_float(q_idx_bits).astype(np.float64)       # exact
    hi = x.shape[0]
    xb = x.reshape(hi, -1, MX_BLOCK)
    amax = np.abs(xb).max(axis=2)
    _, e2 = np.frexp(np.where(amax > 0, amax, 1.0))              # amax = f * 2**e2, f in [0.5, 1)
    X = np.where(amax > 0, (e2 - 1) - E4M3_EMAX, -127)
    X = np.clip(X, -127, 127)
    mag = e4m3fn_round(np.ldexp(np.abs(xb), -X[:, :, None]))
    sign = np.where(np.signbit(xb), 0x80, 0).astype(np.uint8)
    codes = (mag | sign).reshape(hi, -1).astype(np.uint8)
    return codes, (X + 127).astype(np.uint8)


def dequant_query_mx(codes, sbytes):
    """MXFP8 query (codes [Hi, 128], E8M0 bytes [Hi, 4]) -> float64 [Hi, 128], exact."""
    v = e4m3fn_decode(codes).reshape(codes.shape[0], -1, MX_BLOCK)
    return (v * e8m0_decode(sbytes)[:, :, None]).reshape(codes.shape[0], -1)


def order(score_values, positions):
    """Positions sorted by (score descending, position ascending)."""
    score_values = np.asarray(score_values, dtype=np.float32)
    positions = np.asarray(positions, dtype=np.int64)
    return positions[np.lexsort((positions, -score_values.astype(np.float64)))]


def topk(score_values, positions, k):
    """Top-k of (score, position) pairs; returns int32 [k] ascending, -1 padded."""
    best = order(score_values, positions)[:k]
    out = np.full(k, -1, dtype=np.int32)
    out[: best.size] = np.sort(best)
    return out


def full_layer(ik_rows, iks_rows, q_idx_bits, w, mode, k=512, pool_k=0):
    """Full layer of one sequence: score every entry, build the pool, take top-k.

    Returns (topk int32 [k], pool int32 [pool_k] or None, scores float32 [n]).
    """
    n = ik_rows.shape[0]
    s = scores(ik_rows, iks_rows, q_idx_bits, w, mode)
    pos = np.arange(n)
    if pool_k:
        pool = topk(s, pos, pool_k)
        members = pool[pool >= 0]
        top = topk(s[members], members, k)
        return top, pool, s
    return topk(s, pos, k), None, s


def used_candidates(cand, n):
    """The entries of a Reindex candidate list that a layer scores.

    Reading taken (the pages only say that deeper layers look at the Full
    layer's pool, which is a set of distinct positions and is kept in
    ascending order here): a listed position is used when it lies in [0, n)
    and is larger than every in-range position listed before it. A pool
    written by a Full layer passes unchanged; for another list this keeps the
    running record values, so the used positions are distinct and ascending.
    """
    out = []
    best = -1
    for c in np.asarray(cand).tolist():
        if 0 <= c < n:
            if c > best:
                out.append(c)
            best = max(best, c)
    return np.asarray(out, dtype=np.int64)


def reindex_layer(ik_rows, iks_rows, pool, q_idx_bits, w, mode, k=512):
    """Reindex layer of one sequence: rescore the pool rows of the shared key, take top-k.

    The rows rescored are used_candidates(pool, n). Returns (topk int32 [k],
    scores float32 [len(members)] of those rows).
    """
    members = used_candidates(pool, ik_rows.shape[0])
    s = scores(ik_rows[members], iks_rows[members], q_idx_bits, w, mode)
    return topk(s, members, k), s
