"""Sparse decode attention over the dequantized latent at the selected positions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

[TF] section "Mécanismes de compression du KV-Cache", item 1: one 512-d
latent is shared by keys and values across all heads. [FP4] section "Les
ingrédients": the main-cache latent is the part used by attention. [CS]
section "L'architecture : trois leviers contre le cache": attention reads the
top-512 positions chosen by the indexer.

Readings taken: for each query head h and each selected position i (entries
marked -1 are skipped), the logit is tau * (q_h . c_i) with c_i the exact
dequantized latent (it is both key and value; no positional part, since the
288-byte entry holds exactly the 512 latent channels). p = softmax over the
selected positions, o_h = sum_i p_i c_i, lse_h = log sum_i exp(logit). The
oracle computes in float64.
"""
import numpy as np

from .cache import dequant_latent
from .formats import bf16_bits_to_float


def sparse_attention(kv_rows, idx, q_bits, tau=1.0):
    """One sequence. kv_rows: uint8 [n, 288]; idx: int [k] (-1 = skip);
    q_bits: uint16 [H, 512]. Returns (out float64 [H, 512], lse float64 [H]).

    With no valid index the output row is 0 and lse is -inf.
    """
    idx = np.asarray(idx)
    sel = idx[idx >= 0].astype(np.int64)
    q = bf16_bits_to_float(q_bits).astype(np.float64)
    H = q.shape[0]
    if sel.size == 0:
        return np.zeros((H, 512)), np.full(H, -np.inf)
    c = dequant_latent(kv_rows[sel])                   # [k, 512]
    logits = tau * (q @ c.T)                           # [H, k]
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx)
    z = p.sum(axis=1, keepdims=True)
    out = (p @ c) / z
    lse = (mx + np.log(z))[:, 0]
    return out, lse
