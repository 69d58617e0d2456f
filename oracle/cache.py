"""Cache write: ratio-m merge, then FP4 quantization and packing.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

[TF] section "Mécanismes de compression du KV-Cache", item 2: consecutive
positions are fused into one cache entry with learned per-channel weights.
[FP4] section "Le compte par couche": a layer of ratio m stores one entry per
m tokens. [FP4] section "Le coût d'une entrée": main-cache entry = 512
channels E2M1 + one E4M3 scale per 16 channels = 256 + 32 = 288 bytes;
indexer-key entry = 128 channels E2M1 + one E8M0 scale per 32 channels =
64 + 4 = 68 bytes.

Readings taken where the pages are silent (each decides integer codes, so it
is fixed in float32, the precision of the hot path):

* Merge: e[i, c] = sum_j w[j, c] * x[m*i + j, c] with the weights already
  normalised over j (the normalisation belongs to the weights' generation).
  Evaluated in float32 as acc = w0*x0, then acc = acc + wj*xj for j = 1..m-1,
  every product and sum rounded to float32 (no fused multiply-add).
  floor(T/m) entries are written; a trailing partial group is not.
* Latent block scale: s = E4M3FN(amax / 6) with amax the largest magnitude of
  the 16 merged values, amax/6 a correctly rounded float32 division, rounded
  nearest-even to E4M3FN with saturation at 448. Codes are E2M1 of the
  float32 quotient x / s (correctly rounded division), nearest-even,
  saturating at 6; the sign bit is copied from x (so tiny negatives give the
  code 0x8). If s rounds to zero, the block's 16 codes are all 0x0.
* Indexer block scale: OCP MX rule, X = floor(log2 amax) - 2 stored as the
  E8M0 byte X + 127; codes are E2M1 of x * 2**-X (an exact rescaling). A block
  whose amax is zero gets scale byte 0 and all codes 0x0.
* Packing: two codes per byte, the even channel in the low nibble. A main row
  is the 256 code bytes followed by the 32 scale bytes (block b covers
  channels 16b..16b+15). Indexer rows are 64 code bytes; their 4 scale bytes
  live in a separate [entries, 4] array (same bytes, 68 per entry).
"""
import numpy as np

from .formats import (bf16_bits_to_float, e2m1_round_magnitude, e4m3fn_round,
                      e4m3fn_decode, e2m1_decode, e8m0_decode, mx_shared_exponent)

LATENT_CH = 512
LATENT_BLOCK = 16
INDEXER_CH = 128
INDEXER_BLOCK = 32
MAIN_ROW_BYTES = LATENT_CH // 2 + LATENT_CH // LATENT_BLOCK      # 288
INDEXER_CODE_BYTES = INDEXER_CH // 2                              # 64
INDEXER_SCALE_BYTES = INDEXER_CH // INDEXER_BLOCK                 # 4


def merge(x_bits, w_hat, m):
    """Ratio-m merge of one sequence.

    x_bits: uint16 bf16 bit patterns, shape [T, C]. w_hat: float32 [m, C].
    Returns float32 [floor(T/m), C].
    """
    x = bf16_bits_to_float(x_bits)
    w = np.asarray(w_hat, dtype=np.float32)
    T, C = x.shape
    assert w.shape == (m, C)
    E = T // m
    groups = x[: E * m].reshape(E, m, C)
    acc = w[0] * groups[:, 0, :]                   # float32 * float32 -> float32
    for j in range(1, m):
        acc = acc + w[j] * groups[:, j, :]         # two separate roundings
    return acc.astype(np.float32)


def _sign_bits(e):
    return (np.signbit(e)).astype(np.uint8) << 3


def _pack_nibbles(codes):
    """codes uint8 [..., C] (values < 16) -> bytes [..., C/2], even channel low."""
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def quantize_latent(e):
    """Merged latent float32 [E, 512] -> packed main rows uint8 [E, 288]."""
    e = np.asarray(e, dtype=np.float32)
    E = e.shape[0]
    blocks = e.reshape(E, LATENT_CH // LATENT_BLOCK, LATENT_BLOCK)
    amax = np.max(np.abs(blocks), axis=2)                          # float32
    s_in = amax / np.float32(6.0)                                  # float32 division
    s_byte = e4m3fn_round(s_in)                                    # [E, 32]
    s = e4m3fn_decode(s_byte).astype(np.float32)                   # exact
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.abs(blocks) / s[:, :, None]                         # float32 division
    zero_scale = (s == 0)[:, :, None]
    q = np.where(zero_scale, 0.0, q)
    mag = e2m1_round_magnitude(q)
    codes = np.where(zero_scale, 0, mag | _sign_bits(blocks)).astype(np.uint8)
    packed = _pack_nibbles(codes.reshape(E, LATENT_CH))
    return np.concatenate([packed, s_byte], axis=1)


def quantize_indexer(e):
    """Merged indexer key float32 [E, 128] -> (codes uint8 [E, 64], scales uint8 [E, 4])."""
    e = np.asarray(e, dtype=np.float32)
    E = e.shape[0]
    blocks = e.reshape(E, INDEXER_CH // INDEXER_BLOCK, INDEXER_BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    x_byte = mx_shared_exponent(amax)                              # [E, 4]
    X = x_byte.astype(np.int64) - 127
    r = np.ldexp(np.abs(blocks).astype(np.float64), -X[:, :, None])   # exact
    mag = e2m1_round_magnitude(r)
    zero_block = (amax == 0)[:, :, None]
    codes = np.where(zero_block, 0, mag | _sign_bits(blocks)).astype(np.uint8)
    return _pack_nibbles(codes.reshape(E, INDEXER_CH)), x_byte


def cache_write(x_lat_bits, x_idx_bits, w_lat, w_idx, m):
    """One sequence: hidden rows -> (main rows [E,288], indexer codes [E,64], indexer scales [E,4])."""
    kv = quantize_latent(merge(x_lat_bits, w_lat, m))
    ik, iks = quantize_indexer(merge(x_idx_bits, w_idx, m))
    return kv, ik, iks


def append_tokens(x_lat_bits, x_idx_bits, w_lat, w_idx, m):
    """Decode-time append of one sequence's tokens, one at a time.

    [FP4] section "Le compte par couche": one entry per m tokens. Each token
    joins the sequence's stage; when the stage holds m tokens they are merged
    and packed (exactly as cache_write packs one group) into the next entry
    and the stage empties. Returns (kv, ik, iks) of the completed groups in
    order and the staged (latent, key) rows left over.
    """
    kv, ik, iks = [], [], []
    stage = []
    for t in range(x_lat_bits.shape[0]):
        stage.append(t)
        if len(stage) == m:
            a, b, c = cache_write(x_lat_bits[stage], x_idx_bits[stage], w_lat, w_idx, m)
            kv.append(a)
            ik.append(b)
            iks.append(c)
            stage = []
    empty = lambda w: np.zeros((0, w), np.uint8)
    return (np.concatenate(kv) if kv else empty(288), np.concatenate(ik) if ik else empty(64),
            np.concatenate(iks) if iks else empty(4), x_lat_bits[stage], x_idx_bits[stage])


def unpack_nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def dequant_latent(kv_rows):
    """Main rows uint8 [n, 288] -> latent float64 [n, 512] (exact: E2M1 * E4M3)."""
    kv_rows = np.asarray(kv_rows, dtype=np.uint8)
    n = kv_rows.shape[0]
    vals = e2m1_decode(unpack_nibbles(kv_rows[:, : LATENT_CH // 2]))
    s = e4m3fn_decode(kv_rows[:, LATENT_CH // 2:])
    return (vals.reshape(n, -1, LATENT_BLOCK) * s[:, :, None]).reshape(n, LATENT_CH)


def dequant_indexer(ik_rows, iks_rows):
    """Indexer rows -> key float64 [n, 128] (exact: E2M1 * 2**X)."""
    ik_rows = np.asarray(ik_rows, dtype=np.uint8)
    n = ik_rows.shape[0]
    vals = e2m1_decode(unpack_nibbles(ik_rows))
    s = e8m0_decode(iks_rows)
    return (vals.reshape(n, -1, INDEXER_BLOCK) * s[:, :, None]).reshape(n, INDEXER_CH)
