"""ctypes binding of libcsa2fp4 (C ABI in include/csa2fp4.h).

Argument marshalling only: tensors are checked for device, dtype, layout and
shape, their device pointers and the current HIP stream are passed to the C
functions, and non-zero status codes become ``Csa2Error``. Every step of the
computation runs in the library's HIP kernels; there is no host fallback.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))

CSA2_OK = 0
CSA2_SCORE_DOT, CSA2_SCORE_RELU_W = 0, 1
CSA2_SCORE_QMX8 = 0x100          # flag: quantized-query (MXFP8) variant of either score
CSA2_FULL, CSA2_REINDEX, CSA2_REUSE = 0, 1, 2
CSA2_NOALLOC_SCRATCH_BYTES = 64 << 20   # static scratch of csa2_decode_layer_noalloc
MAIN_ROW_BYTES, INDEXER_CODE_BYTES, INDEXER_SCALE_BYTES = 288, 64, 4

_lib = None


class Csa2Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"csa2 error {code}: {msg}")
        self.code = code


def library_path():
    return os.environ.get("CSA2FP4_LIB", os.path.join(PKG, "libcsa2fp4.so"))


def lib():
    """Load libcsa2fp4.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m long_context_fp4_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.csa2_cache_write.argtypes = [vp, vp, vp, vp, i32, i64, i32, vp, vp, vp, vp, vp, vp]
    L.csa2_cache_write.restype = i32
    L.csa2_cache_append.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.csa2_cache_append.restype = i32
    L.csa2_prefill_workspace_bytes.argtypes = [i32, i32, i64, i32, i32]
    L.csa2_prefill_workspace_bytes.restype = sz
    L.csa2_prefill_layer.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, vp, vp, vp, i32, i32, vp, i32, f32, i32,
                                     vp, vp, vp, vp, sz, vp]
    L.csa2_prefill_layer.restype = i32
    L.csa2_swa_write.argtypes = [vp, i32, i64, vp, vp, vp]
    L.csa2_swa_write.restype = i32
    L.csa2_swa_attention.argtypes = [vp, vp, vp, i32, i32, f32, vp, vp, vp]
    L.csa2_swa_attention.restype = i32
    L.csa2_indexer_workspace_bytes.argtypes = [i32, i64, i32, i32, i32]
    L.csa2_indexer_workspace_bytes.restype = sz
    L.csa2_indexer_topk.argtypes = [vp, vp, vp, vp, i32, i64, vp, vp, i32, i32, vp, i32, i32, vp, i32, vp,
                                    vp, vp, sz, vp]
    L.csa2_indexer_topk.restype = i32
    L.csa2_attention_workspace_bytes.argtypes = [i32, i32, i32]
    L.csa2_attention_workspace_bytes.restype = sz
    L.csa2_sparse_attention.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, f32, vp, vp, vp, sz, vp]
    L.csa2_sparse_attention.restype = i32
    L.csa2_decode_workspace_bytes.argtypes = [i32, i64, i32, i32, i32]
    L.csa2_decode_workspace_bytes.restype = sz
    L.csa2_decode_layer.argtypes = [i32, vp, vp, vp, vp, vp, i32, i64, vp, vp, i32, i32, vp, i32, f32, i32, i32,
                                    vp, vp, vp, vp, vp, sz, vp]
    L.csa2_decode_layer.restype = i32
    L.csa2_decode_layer_noalloc.argtypes = [i32, vp, vp, vp, vp, vp, i32, i64, vp, vp, i32, i32, vp, i32, f32, i32,
                                            i32, vp, vp, vp, vp, vp]
    L.csa2_decode_layer_noalloc.restype = i32
    L.csa2_bytes_per_token.argtypes = [ctypes.POINTER(ctypes.c_int), i32, i32, i32, i32, i32, i32, i32]
    L.csa2_bytes_per_token.restype = ctypes.c_double
    L.csa2_set_profile_events.argtypes = [vp, vp]
    L.csa2_set_profile_events.restype = i32
    L.csa2_last_error.argtypes = []
    L.csa2_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc):
    if rc != CSA2_OK:
        raise Csa2Error(rc, lib().csa2_last_error().decode())


def _torch():
    import torch
    return torch


def _ptr(t, dtype=None, name="tensor"):
    """Device pointer of a contiguous CUDA/HIP tensor (None -> NULL)."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _bf16_types():
    torch = _torch()
    return (torch.int16, torch.uint16, torch.bfloat16)


class Workspace:
    """Device workspace that grows on demand (one per stream of use; needs no initialisation)."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes):
        torch = _torch()
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws = {}


def _ws(ws, device):
    if ws is not None:
        return ws
    key = str(device)
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


def cache_write(x_lat, x_idx, w_lat, w_idx, m, kv=None, ik=None, iks=None, n_tokens=None,
                out_entry_offset=None, stream=None):
    """Merge + pack B sequences of hidden rows. x_lat [B,T,512], x_idx [B,T,128] bf16 bits.

    n_tokens: i64 [B] tokens of each sequence (<= T; None = T each). out_entry_offset: i64 [B]
    first cache row of each sequence (None = b * (T // m); then the outputs are created when
    not given). Returns (kv [rows, 288] u8, ik [rows, 64] u8, iks [rows, 4] u8).
    """
    torch = _torch()
    if x_lat.dim() == 2:
        x_lat, x_idx = x_lat[None], x_idx[None]
    B, T, C = x_lat.shape
    if C != 512 or tuple(x_idx.shape) != (B, T, 128):
        raise ValueError("x_lat must be [B,T,512] and x_idx [B,T,128]")
    if tuple(w_lat.shape) != (m, 512) or tuple(w_idx.shape) != (m, 128):
        raise ValueError("w_lat must be [m,512] and w_idx [m,128]")
    for name, t in (("n_tokens", n_tokens), ("out_entry_offset", out_entry_offset)):
        if t is not None and tuple(t.shape) != (B,):
            raise ValueError(f"{name} must be [B]")
    E = T // m
    dev = x_lat.device
    if out_entry_offset is not None and (kv is None or ik is None or iks is None):
        raise ValueError("with out_entry_offset the caller provides kv, ik and iks")
    kv = torch.empty((B * E, MAIN_ROW_BYTES), dtype=torch.uint8, device=dev) if kv is None else kv
    ik = torch.empty((B * E, INDEXER_CODE_BYTES), dtype=torch.uint8, device=dev) if ik is None else ik
    iks = torch.empty((B * E, INDEXER_SCALE_BYTES), dtype=torch.uint8, device=dev) if iks is None else iks
    if out_entry_offset is None and (kv.shape[0] < B * E or ik.shape[0] < B * E or iks.shape[0] < B * E):
        raise ValueError("output buffers too small")
    bt = _bf16_types()
    _check(lib().csa2_cache_write(_ptr(x_lat, bt, "x_lat"), _ptr(x_idx, bt, "x_idx"),
                                  _ptr(w_lat, torch.float32, "w_lat"), _ptr(w_idx, torch.float32, "w_idx"),
                                  B, T, m, _ptr(n_tokens, torch.int64, "n_tokens"),
                                  _ptr(out_entry_offset, torch.int64, "out_entry_offset"),
                                  _ptr(kv, torch.uint8, "kv"), _ptr(ik, torch.uint8, "ik"),
                                  _ptr(iks, torch.uint8, "iks"), _stream(stream)))
    return kv, ik, iks


def cache_append(x_lat, x_idx, w_lat, w_idx, m, stage_lat, stage_idx, stage_count, entry_offset, n_entries,
                 capacity, kv, ik, iks, dropped=None, stream=None):
    """Append one token per sequence (x_lat [B,512], x_idx [B,128] bf16 bits) to the cache.

    stage_lat [B,m-1,512] / stage_idx [B,m-1,128] (None when m == 1), stage_count [B] i32 and
    n_entries [B] i32 are updated in place; a completed group is packed into cache row
    entry_offset[b] + n_entries[b] of kv / ik / iks while n_entries[b] < capacity[b]
    (capacity: i64 [B] device tensor). Returns dropped [B] i32 when given.
    """
    torch = _torch()
    B = x_lat.shape[0]
    if tuple(x_lat.shape) != (B, 512) or tuple(x_idx.shape) != (B, 128):
        raise ValueError("x_lat must be [B,512] and x_idx [B,128]")
    if tuple(w_lat.shape) != (m, 512) or tuple(w_idx.shape) != (m, 128):
        raise ValueError("w_lat must be [m,512] and w_idx [m,128]")
    if m > 1 and (stage_lat is None or tuple(stage_lat.shape) != (B, m - 1, 512) or
                  tuple(stage_idx.shape) != (B, m - 1, 128)):
        raise ValueError("stage_lat must be [B,m-1,512] and stage_idx [B,m-1,128]")
    if (stage_count.shape[0] != B or n_entries.shape[0] != B or entry_offset.shape[0] != B
            or tuple(capacity.shape) != (B,)):
        raise ValueError("stage_count, n_entries, entry_offset and capacity must be [B]")
    bt = _bf16_types()
    st_l = _ptr(stage_lat, bt, "stage_lat") if m > 1 else None
    st_i = _ptr(stage_idx, bt, "stage_idx") if m > 1 else None
    _check(lib().csa2_cache_append(_ptr(x_lat, bt, "x_lat"), _ptr(x_idx, bt, "x_idx"),
                                   _ptr(w_lat, torch.float32, "w_lat"), _ptr(w_idx, torch.float32, "w_idx"),
                                   B, m, st_l, st_i, _ptr(stage_count, torch.int32, "stage_count"),
                                   _ptr(entry_offset, torch.int64, "entry_offset"),
                                   _ptr(n_entries, torch.int32, "n_entries"),
                                   _ptr(capacity, torch.int64, "capacity"),
                                   _ptr(kv, torch.uint8, "kv"), _ptr(ik, torch.uint8, "ik"),
                                   _ptr(iks, torch.uint8, "iks"), _ptr(dropped, torch.int32, "dropped"),
                                   _stream(stream)))
    return dropped


SWA_WINDOW = 128
SWA_ROW_BYTES = 544


def swa_write(x_lat, pos0, win=None, stream=None):
    """Write tokens pos0[b] .. pos0[b]+T-1 (x_lat [B,T,512] bf16 bits) into the window ring.

    win: [B, 128, 544] u8 (created zeroed when None). Returns win.
    """
    torch = _torch()
    if x_lat.dim() == 2:
        x_lat = x_lat[:, None]
    B, T, C = x_lat.shape
    if C != 512 or pos0.shape[0] != B:
        raise ValueError("x_lat must be [B,T,512] and pos0 [B]")
    if win is None:
        win = torch.zeros((B, SWA_WINDOW, SWA_ROW_BYTES), dtype=torch.uint8, device=x_lat.device)
    if tuple(win.shape) != (B, SWA_WINDOW, SWA_ROW_BYTES):
        raise ValueError("win must be [B,128,544]")
    _check(lib().csa2_swa_write(_ptr(x_lat, _bf16_types(), "x_lat"), B, T, _ptr(pos0, torch.int64, "pos0"),
                                _ptr(win, torch.uint8, "win"), _stream(stream)))
    return win


def swa_attention(win, n_win, q, out, lse, softmax_scale=1.0, stream=None):
    """Attend over the window and merge into the sparse branch's out [B,H,512] / lse [B,H] in place."""
    torch = _torch()
    B, H, _ = q.shape
    if tuple(win.shape) != (B, SWA_WINDOW, SWA_ROW_BYTES) or n_win.shape[0] != B:
        raise ValueError("win must be [B,128,544] and n_win [B]")
    if tuple(out.shape) != (B, H, 512) or tuple(lse.shape) != (B, H):
        raise ValueError("out must be [B,H,512] and lse [B,H]")
    _check(lib().csa2_swa_attention(_ptr(win, torch.uint8, "win"), _ptr(n_win, torch.int32, "n_win"),
                                    _ptr(q, _bf16_types(), "q"), B, H, float(softmax_scale),
                                    _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
                                    _stream(stream)))
    return out, lse


def prefill_layer(kv, ik, iks, entry_offset, n_entries, max_n, m, pos, q_idx, q, w=None,
                  score_mode=CSA2_SCORE_RELU_W, softmax_scale=1.0, k=512, workspace=None, topk=None, out=None,
                  lse=None, stream=None):
    """Tq query tokens per sequence, each with its causal top-k and attention.

    pos [B,Tq] i64, q_idx [B,Tq,Hi,128], w [B,Tq,Hi] or None, q [B,Tq,H,512] (bf16 bits).
    Returns (topk [B,Tq,k] i32, out [B,Tq,H,512] f32, lse [B,Tq,H] f32).
    """
    torch = _torch()
    B, Tq, H, D = q.shape
    Hi = q_idx.shape[2]
    if D != 512 or tuple(pos.shape) != (B, Tq) or tuple(q_idx.shape) != (B, Tq, Hi, 128):
        raise ValueError("q must be [B,Tq,H,512], pos [B,Tq] and q_idx [B,Tq,Hi,128]")
    if w is not None and tuple(w.shape) != (B, Tq, Hi):
        raise ValueError("w must be [B,Tq,Hi]")
    dev = q.device
    topk = torch.empty((B, Tq, k), dtype=torch.int32, device=dev) if topk is None else topk
    out = torch.empty((B, Tq, H, 512), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=dev) if lse is None else lse
    nbytes = lib().csa2_prefill_workspace_bytes(B, Tq, int(max_n), H, k)
    buf = _ws(workspace, dev).get(nbytes)
    bt = _bf16_types()
    _check(lib().csa2_prefill_layer(_ptr(kv, torch.uint8, "kv"), _ptr(ik, torch.uint8, "ik"),
                                    _ptr(iks, torch.uint8, "iks"), _ptr(entry_offset, torch.int64, "entry_offset"),
                                    _ptr(n_entries, torch.int32, "n_entries"), B, int(max_n), m, Tq,
                                    _ptr(pos, torch.int64, "pos"), _ptr(q_idx, bt, "q_idx"),
                                    _ptr(w, torch.float32, "w"), Hi, score_mode, _ptr(q, bt, "q"), H,
                                    float(softmax_scale), k, _ptr(topk, torch.int32, "topk"),
                                    _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
                                    _ptr(buf, torch.uint8, "workspace"), buf.numel(), _stream(stream)))
    return topk, out, lse


def indexer_topk(ik, iks, entry_offset, n_entries, max_n, q_idx, w=None, score_mode=CSA2_SCORE_RELU_W,
                 cand=None, k=512, pool_k=0, want_scores=False, workspace=None, topk=None, pool=None,
                 stream=None):
    """Indexer pass + top-k. Returns (topk [B,k] i32, pool [B,pool_k] i32 or None, scores or None)."""
    torch = _torch()
    B = entry_offset.shape[0]
    Hi = q_idx.shape[1]
    if tuple(q_idx.shape) != (B, Hi, 128):
        raise ValueError("q_idx must be [B,Hi,128]")
    if w is not None and tuple(w.shape) != (B, Hi):
        raise ValueError("w must be [B,Hi]")
    if n_entries.shape[0] != B:
        raise ValueError("n_entries must be [B]")
    cand_stride = 0
    if cand is not None:
        if cand.dim() != 2 or cand.shape[0] != B:
            raise ValueError("cand must be [B, cand_stride]")
        cand_stride = cand.shape[1]
    dev = ik.device
    topk = torch.empty((B, k), dtype=torch.int32, device=dev) if topk is None else topk
    if pool_k and pool is None:
        pool = torch.empty((B, pool_k), dtype=torch.int32, device=dev)
    scores = None
    if want_scores:
        scores = torch.empty((B, cand_stride if cand is not None else max(int(max_n), 1)),
                             dtype=torch.float32, device=dev)
    nbytes = lib().csa2_indexer_workspace_bytes(B, int(max_n), k, pool_k, cand_stride)
    buf = _ws(workspace, dev).get(nbytes)
    _check(lib().csa2_indexer_topk(_ptr(ik, torch.uint8, "ik"), _ptr(iks, torch.uint8, "iks"),
                                   _ptr(entry_offset, torch.int64, "entry_offset"),
                                   _ptr(n_entries, torch.int32, "n_entries"), B, int(max_n),
                                   _ptr(q_idx, _bf16_types(), "q_idx"), _ptr(w, torch.float32, "w"), Hi,
                                   score_mode, _ptr(cand, torch.int32, "cand"), cand_stride, k,
                                   _ptr(topk, torch.int32, "topk"), pool_k, _ptr(pool, torch.int32, "pool"),
                                   _ptr(scores, torch.float32, "scores"), _ptr(buf), buf.numel(),
                                   _stream(stream)))
    return topk, pool, scores


def sparse_attention(kv, entry_offset, n_entries, idx, q, softmax_scale=1.0, workspace=None, out=None,
                     lse=None, stream=None):
    """Sparse attention over the selected latent rows. Returns (out [B,H,512] f32, lse [B,H] f32)."""
    torch = _torch()
    B, H, D = q.shape
    if D != 512 or idx.dim() != 2 or idx.shape[0] != B:
        raise ValueError("q must be [B,H,512] and idx [B,k]")
    k = idx.shape[1]
    dev = q.device
    out = torch.empty((B, H, 512), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=dev) if lse is None else lse
    nbytes = lib().csa2_attention_workspace_bytes(B, H, k)
    buf = _ws(workspace, dev).get(nbytes)
    _check(lib().csa2_sparse_attention(_ptr(kv, torch.uint8, "kv"), _ptr(entry_offset, torch.int64, "entry_offset"),
                                       _ptr(n_entries, torch.int32, "n_entries"), _ptr(idx, torch.int32, "idx"), k,
                                       _ptr(q, _bf16_types(), "q"), B, H, float(softmax_scale),
                                       _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
                                       _ptr(buf), buf.numel(), _stream(stream)))
    return out, lse


def _layer_outputs(mode, q, q_idx, k, pool_k, pool, topk, out, lse):
    """Output tensors of a layer call (allocated when not given) and its k, pool_k, Hi."""
    torch = _torch()
    B, H, _ = q.shape
    dev = q.device
    Hi = q_idx.shape[1] if q_idx is not None else 1
    if mode == CSA2_FULL:
        topk = torch.empty((B, k), dtype=torch.int32, device=dev) if topk is None else topk
        if pool_k and pool is None:
            pool = torch.empty((B, pool_k), dtype=torch.int32, device=dev)
    elif mode == CSA2_REINDEX:
        if pool is None:
            raise ValueError("Reindex needs the pool")
        pool_k = pool.shape[1]
        topk = torch.empty((B, k), dtype=torch.int32, device=dev) if topk is None else topk
    else:
        if topk is None:
            raise ValueError("Reuse needs topk")
        k = topk.shape[1]
    out = torch.empty((B, H, 512), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=dev) if lse is None else lse
    return topk, pool, out, lse, k, pool_k, Hi


def _layer_args(mode, kv, ik, iks, entry_offset, n_entries, max_n, q, q_idx, w, Hi, score_mode, softmax_scale, k,
                pool_k, pool, topk, out, lse):
    torch = _torch()
    B, H, _ = q.shape
    return (mode, _ptr(kv, torch.uint8, "kv"), _ptr(ik, torch.uint8, "ik"), _ptr(iks, torch.uint8, "iks"),
            _ptr(entry_offset, torch.int64, "entry_offset"), _ptr(n_entries, torch.int32, "n_entries"), B,
            int(max_n), _ptr(q_idx, _bf16_types(), "q_idx"), _ptr(w, torch.float32, "w"), Hi, score_mode,
            _ptr(q, _bf16_types(), "q"), H, float(softmax_scale), k, pool_k, _ptr(pool, torch.int32, "pool"),
            _ptr(topk, torch.int32, "topk"), _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"))


def decode_layer(mode, kv, ik, iks, entry_offset, n_entries, max_n, q, q_idx=None, w=None,
                 score_mode=CSA2_SCORE_RELU_W, softmax_scale=1.0, k=512, pool_k=0, pool=None, topk=None,
                 workspace=None, out=None, lse=None, stream=None):
    """One CSA2 layer (Full / Reindex / Reuse). Returns (topk, pool, out, lse)."""
    topk, pool, out, lse, k, pool_k, Hi = _layer_outputs(mode, q, q_idx, k, pool_k, pool, topk, out, lse)
    B, H, _ = q.shape
    nbytes = lib().csa2_decode_workspace_bytes(B, int(max_n), H, k, pool_k)
    buf = _ws(workspace, q.device).get(nbytes)
    args = _layer_args(mode, kv, ik, iks, entry_offset, n_entries, max_n, q, q_idx, w, Hi, score_mode,
                       softmax_scale, k, pool_k, pool, topk, out, lse)
    _check(lib().csa2_decode_layer(*args, _ptr(buf), buf.numel(), _stream(stream)))
    return topk, pool, out, lse


def decode_layer_noalloc(mode, kv, ik, iks, entry_offset, n_entries, max_n, q, topk, out, lse, q_idx=None, w=None,
                         score_mode=CSA2_SCORE_RELU_W, softmax_scale=1.0, k=512, pool_k=0, pool=None, stream=None):
    """decode_layer on the library's static scratch: the caller passes every output
    (topk, out, lse, and pool for a Full layer with pool_k > 0). Returns (topk, pool, out, lse)."""
    if mode == CSA2_FULL and pool_k and pool is None:
        raise ValueError("a Full layer with pool_k > 0 needs the pool output")
    topk, pool, out, lse, k, pool_k, Hi = _layer_outputs(mode, q, q_idx, k, pool_k, pool, topk, out, lse)
    args = _layer_args(mode, kv, ik, iks, entry_offset, n_entries, max_n, q, q_idx, w, Hi, score_mode,
                       softmax_scale, k, pool_k, pool, topk, out, lse)
    _check(lib().csa2_decode_layer_noalloc(*args, _stream(stream)))
    return topk, pool, out, lse


def bytes_per_token(ratios, lat=(512, 16, 1), idx=(128, 32, 1)):
    """Global-cache bytes per token (host-only accounting in the library)."""
    arr = (ctypes.c_int * len(ratios))(*ratios)
    v = lib().csa2_bytes_per_token(arr, len(ratios), lat[0], lat[1], lat[2], idx[0], idx[1], idx[2])
    if v < 0:
        raise Csa2Error(-2, lib().csa2_last_error().decode())
    return v


def set_profile_events(before, after):
    """Record two torch.cuda.Event objects around the next Full pass's scoring kernel (this thread)."""
    if before is None:
        _check(lib().csa2_set_profile_events(None, None))
        return
    _check(lib().csa2_set_profile_events(ctypes.c_void_p(before.cuda_event), ctypes.c_void_p(after.cuda_event)))
