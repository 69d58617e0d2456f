"""Sliding-window branch: the last 128 tokens in FP8, attended beside the sparse branch.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

[FP4] section "La contrepartie : la fenêtre glissante": besides the global cache
every layer keeps a sliding window in FP8 of 512 + 512/16 bytes per token (the
page's equation: 40 layers x 128 tokens x 544 bytes = 2.66 MiB per sequence).
[CS] section "L'architecture : trois leviers contre le cache" (its third point):
the window is 128 tokens. The pages give these sizes, not the formats.

Readings taken:

* A token's window row is its 512-channel latent row, unmerged: 512 bytes of
  E4M3FN values (channel c at byte c), then 32 scale bytes, one per block of 16
  channels (block b covers channels 16b..16b+15) - the main row's
  data-then-scales order with one byte per value.
* Scale: an E8M0 power of two per block (the page leaves the scale format of
  the FP8 cache open; an E4M3 scale of amax / 448 would fall into E4M3's
  subnormal range for ordinary magnitudes and lose most of its bits):
  s = 2^X with X the smallest integer such that amax <= 448 * 2^X, so no value
  saturates; byte X + 127, clamped to [0, 254]. Each value is the E4M3FN
  nearest-even of x * 2^-X (an exact rescaling), with the sign of x. A block
  whose amax is zero has scale byte 0 and zero values.
* Placement: a ring of 128 rows per sequence, token t in row t mod 128; with n
  tokens written the valid rows are the first min(n, 128).
* Attention: the same query heads and tau attend over the valid window rows;
  the window's (o_w, lse_w) and the sparse branch's (o_s, lse_s) merge into one
  softmax over the union of both position sets:
  o = (e^lse_s o_s + e^lse_w o_w) / (e^lse_s + e^lse_w), lse = log(e^lse_s + e^lse_w).
"""
import numpy as np

from .formats import bf16_bits_to_float, e4m3fn_decode, e4m3fn_round, e8m0_decode

WINDOW = 128
CHANNELS = 512
BLOCK = 16
ROW_BYTES = CHANNELS + CHANNELS // BLOCK     # 544
E4M3_MAX = 448.0


def block_exponent(amax):
    """Smallest X with amax <= 448 * 2^X (amax > 0), from the binary exponent: exact."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e2 = np.frexp(np.where(amax > 0, amax, 1.0))
    x0 = (e2 - 1) - 8                        # amax * 2^-x0 in [256, 512)
    return np.where(np.ldexp(amax, -x0) > E4M3_MAX, x0 + 1, x0)


def quantize_window_rows(x_bits):
    """bf16 latent rows [T, 512] -> window rows uint8 [T, 544]."""
    x = bf16_bits_to_float(x_bits).astype(np.float64).reshape(-1, CHANNELS // BLOCK, BLOCK)   # exact
    T = x.shape[0]
    amax = np.abs(x).max(axis=2)
    X = np.clip(block_exponent(amax), -127, 127)
    s_byte = np.where(amax > 0, X + 127, 0).astype(np.uint8)
    q = np.ldexp(np.abs(x), -X[:, :, None])                                     # exact rescaling
    mag = e4m3fn_round(np.minimum(q, 1e30))
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    vals = np.where((amax > 0)[:, :, None], mag | sign, 0).astype(np.uint8)
    return np.concatenate([vals.reshape(T, CHANNELS), s_byte.reshape(T, -1)], axis=1)


def dequant_window_rows(rows):
    """Window rows [n, 544] -> float64 latent [n, 512] (value times block scale, exact)."""
    rows = np.asarray(rows, dtype=np.uint8)
    v = e4m3fn_decode(rows[:, :CHANNELS]).reshape(-1, CHANNELS // BLOCK, BLOCK)
    s = e8m0_decode(rows[:, CHANNELS:])[:, :, None]
    return (v * s).reshape(-1, CHANNELS)


def window_write(x_bits, pos0, ring=None):
    """Write tokens pos0 .. pos0+T-1 (rows of x_bits [T, 512]) into a ring [128, 544]."""
    ring = np.zeros((WINDOW, ROW_BYTES), np.uint8) if ring is None else ring.copy()
    rows = quantize_window_rows(x_bits)
    for t in range(x_bits.shape[0]):
        ring[(pos0 + t) % WINDOW] = rows[t]
    return ring


def window_attention(rows, q_bits, tau=1.0):
    """Attention of q [H, 512] over window rows [n, 544]; (o [H, 512], lse [H]) in float64.

    With no row the output is 0 and lse is -inf.
    """
    q = bf16_bits_to_float(q_bits).astype(np.float64)
    H = q.shape[0]
    if len(rows) == 0:
        return np.zeros((H, CHANNELS)), np.full(H, -np.inf)
    c = dequant_window_rows(rows)
    logits = tau * (q @ c.T)
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx)
    z = p.sum(axis=1, keepdims=True)
    return (p @ c) / z, (mx + np.log(z))[:, 0]


def merge_branches(o_s, lse_s, o_w, lse_w):
    """One softmax over the union of two position sets, from each branch's (o, lse)."""
    o_s, lse_s, o_w, lse_w = (np.asarray(a, np.float64) for a in (o_s, lse_s, o_w, lse_w))
    m = np.maximum(lse_s, lse_w)
    m = np.where(np.isneginf(m), 0.0, m)
    a_s = np.exp(lse_s - m)
    a_w = np.exp(lse_w - m)
    z = a_s + a_w
    zs = np.where(z > 0, z, 1.0)
    o = (a_s[:, None] * o_s + a_w[:, None] * o_w) / zs[:, None]
    lse = np.where(z > 0, m + np.log(zs), -np.inf)
    return np.where((z > 0)[:, None], o, 0.0), lse
