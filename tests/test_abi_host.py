"""The C-ABI library loads without a GPU, exports every declared symbol, and rejects bad arguments on the host."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2fp4.h")


@pytest.fixture(scope="module")
def L():
    from long_context_fp4_amd import binding
    if not os.path.exists(binding.library_path()):
        pytest.skip("libcsa2fp4.so not built")
    return binding.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_api():
    names = declared_functions()
    for n in ("csa2_cache_write", "csa2_cache_append", "csa2_swa_write", "csa2_swa_attention", "csa2_prefill_layer",
              "csa2_prefill_workspace_bytes", "csa2_indexer_topk", "csa2_sparse_attention", "csa2_decode_layer",
              "csa2_indexer_workspace_bytes", "csa2_attention_workspace_bytes", "csa2_decode_workspace_bytes",
              "csa2_bytes_per_token", "csa2_last_error", "csa2_decode_layer_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n


P = 4096          # a fake, 16-byte aligned, non-null address: never dereferenced on these error paths


def err(L):
    return L.csa2_last_error().decode()


def test_cache_write_validation(L):
    def call(**kw):
        a = dict(xl=P, xi=P, wl=P, wi=P, B=1, T=10, m=2, nt=None, off=None, kv=P, ik=P, iks=P)
        a.update(kw)
        return L.csa2_cache_write(a["xl"], a["xi"], a["wl"], a["wi"], a["B"], a["T"], a["m"], a["nt"], a["off"],
                                  a["kv"], a["ik"], a["iks"], None)
    assert call(xl=None) == -1
    assert call(iks=None) == -1
    assert call(B=0) == -2 and call(B=65536) == -2
    assert call(T=-1) == -2
    assert call(m=0) == -2 and call(m=17) == -2
    assert call(xl=P + 2) == -3
    assert call(iks=P + 2) == -3 and "aligned" in err(L)     # iks needs 4 bytes
    assert call(nt=P + 8) == -3                               # token counts and offsets: 16 bytes
    assert call(off=P + 8) == -3


def test_cache_append_validation(L):
    def call(**kw):
        a = dict(xl=P, xi=P, wl=P, wi=P, B=2, m=2, sl=P, si=P, sc=P, off=P, n=P, cap=P, kv=P, ik=P, iks=P, dr=None)
        a.update(kw)
        return L.csa2_cache_append(a["xl"], a["xi"], a["wl"], a["wi"], a["B"], a["m"], a["sl"], a["si"], a["sc"],
                                   a["off"], a["n"], a["cap"], a["kv"], a["ik"], a["iks"], a["dr"], None)
    assert call(xl=None) == -1
    assert call(n=None) == -1
    assert call(sl=None) == -1            # m > 1 needs the stage
    assert call(B=0) == -2 and call(B=1025) == -2
    assert call(m=0) == -2 and call(m=17) == -2
    assert call(cap=None) == -1           # the per-sequence capacities
    assert call(cap=P + 8) == -3
    assert call(xl=P + 2) == -3
    assert call(iks=P + 2) == -3          # 4-byte alignment
    assert call(sc=P + 2) == -3
    assert call(dr=P + 2) == -3
    assert "aligned" in err(L)


def test_swa_validation(L):
    assert L.csa2_swa_write(None, 1, 10, P, P, None) == -1
    assert L.csa2_swa_write(P, 0, 10, P, P, None) == -2
    assert L.csa2_swa_write(P, 1, -1, P, P, None) == -2
    assert L.csa2_swa_write(P, 1, 10, P, P + 8, None) == -3
    assert L.csa2_swa_attention(P, None, P, 1, 8, 1.0, P, P, None) == -1
    assert L.csa2_swa_attention(P, P, P, 0, 8, 1.0, P, P, None) == -2
    assert L.csa2_swa_attention(P, P, P, 1025, 8, 1.0, P, P, None) == -2
    assert L.csa2_swa_attention(P, P, P, 1, 129, 1.0, P, P, None) == -2
    assert L.csa2_swa_attention(P, P, P, 1, 8, 1.0, P, P + 4, None) == -3
    assert "aligned" in err(L)


def test_prefill_validation(L):
    def call(**kw):
        a = dict(B=2, m=2, Tq=4, pos=P, ws=P, wsb=1 << 30)
        a.update(kw)
        return L.csa2_prefill_layer(P, P, P, P, P, a["B"], 1000, a["m"], a["Tq"], a["pos"], P, P, 16, 1, P, 64,
                                    1.0, 512, P, P, P, a["ws"], a["wsb"], None)
    assert call(pos=None) == -1
    assert call(B=0) == -2 and call(Tq=0) == -2 and call(B=2, Tq=513) == -2
    assert call(m=0) == -2 and call(m=17) == -2
    assert call(pos=P + 8) == -3
    assert call(wsb=16) == -4
    assert L.csa2_prefill_workspace_bytes(2, 4, 1000, 64, 512) > L.csa2_decode_workspace_bytes(8, 1000, 64, 512, 0)
    assert L.csa2_prefill_workspace_bytes(2, 513, 1000, 64, 512) == 0


def idx_call(L, **kw):
    a = dict(ik=P, iks=P, off=P, n=P, B=2, max_n=1000, q=P, w=P, Hi=16, mode=1, cand=None, cs=0, k=512, top=P,
             pool_k=0, pool=None, scores=None, ws=P, ws_bytes=1 << 30)
    a.update(kw)
    return L.csa2_indexer_topk(a["ik"], a["iks"], a["off"], a["n"], a["B"], a["max_n"], a["q"], a["w"], a["Hi"],
                               a["mode"], a["cand"], a["cs"], a["k"], a["top"], a["pool_k"], a["pool"], a["scores"],
                               a["ws"], a["ws_bytes"], None)


def test_indexer_validation(L):
    assert idx_call(L, ik=None) == -1
    assert idx_call(L, B=0) == -2
    assert idx_call(L, Hi=0) == -2 and idx_call(L, Hi=17) == -2
    assert idx_call(L, mode=0, Hi=2) == -2
    assert idx_call(L, mode=7) == -5
    # the quantized-query flag goes with either mode, nothing else
    assert idx_call(L, mode=0x100 | 2) == -5 and idx_call(L, mode=0x200 | 1) == -5
    assert idx_call(L, mode=0x100, Hi=2) == -2                # DOT | QMX8 still takes one head
    assert idx_call(L, mode=0x101, ws=None) == -4             # RELU_W | QMX8 passes the mode checks
    assert idx_call(L, k=0) == -2 and idx_call(L, k=4096) == -2
    assert idx_call(L, pool_k=20000, pool=P) == -2
    assert idx_call(L, pool_k=256, pool=P) == -2          # pool smaller than k
    assert idx_call(L, pool_k=1024, pool=None) == -1
    assert idx_call(L, cand=P, cs=20000) == -2
    assert idx_call(L, q=P + 8) == -3
    assert idx_call(L, ws=None) == -4
    need = L.csa2_indexer_workspace_bytes(2, 1000, 512, 0, 0)
    assert need > 0
    # the pool lists and a Reindex list longer than max_n take more room
    assert L.csa2_indexer_workspace_bytes(2, 1000, 512, 1024, 0) > need
    assert L.csa2_indexer_workspace_bytes(2, 1000, 512, 0, 4096) > need
    # the threshold path (k above the direct finish's limit) takes its bitmap and lists
    assert L.csa2_indexer_workspace_bytes(2, 1000, 2048, 0, 0) > need
    assert L.csa2_indexer_workspace_bytes(1025, 1000, 512, 0, 0) == 0
    assert L.csa2_indexer_workspace_bytes(2, 1000, 0, 0, 0) == 0
    assert idx_call(L, B=1025) == -2
    assert idx_call(L, ws_bytes=need - 1) == -4
    assert "workspace" in err(L)


def test_attention_validation(L):
    def call(**kw):
        a = dict(kv=P, off=P, n=P, idx=P, k=512, q=P, B=2, H=64, tau=1.0, out=P, lse=P, ws=P, ws_bytes=1 << 30)
        a.update(kw)
        return L.csa2_sparse_attention(a["kv"], a["off"], a["n"], a["idx"], a["k"], a["q"], a["B"], a["H"],
                                       ctypes.c_float(a["tau"]), a["out"], a["lse"], a["ws"], a["ws_bytes"], None)
    assert call(kv=None) == -1
    assert call(H=0) == -2 and call(H=129) == -2
    assert call(k=0) == -2 and call(k=2049) == -2
    assert call(out=P + 4) == -3
    assert call(ws=None) == -4


def test_decode_layer_validation(L):
    def call(mode, **kw):
        a = dict(kv=P, ik=P, iks=P, off=P, n=P, B=2, max_n=1000, qi=P, w=P, Hi=16, sm=1, q=P, H=64, tau=1.0,
                 k=512, pool_k=0, pool=None, top=P, out=P, lse=P, ws=P, ws_bytes=1 << 30)
        a.update(kw)
        return L.csa2_decode_layer(mode, a["kv"], a["ik"], a["iks"], a["off"], a["n"], a["B"], a["max_n"], a["qi"],
                                   a["w"], a["Hi"], a["sm"], a["q"], a["H"], ctypes.c_float(a["tau"]), a["k"],
                                   a["pool_k"], a["pool"], a["top"], a["out"], a["lse"], a["ws"], a["ws_bytes"], None)
    assert call(9) == -5
    assert call(1) == -1                       # Reindex without a pool
    assert call(0, qi=None) == -1
    assert call(2, ws_bytes=10) == -4


def test_bytes_per_token_matches_the_pages(L):
    from long_context_fp4_amd import bytes_per_token
    assert bytes_per_token([2, 2, 2, 1]) == 890.0
    assert bytes_per_token([2]) == 178.0 and bytes_per_token([1]) == 356.0
    assert bytes_per_token([2, 2, 2, 1], lat=(512, 32, 1)) == 850.0
    assert bytes_per_token([2, 2, 2, 1], lat=(512, 0, 1), idx=(128, 0, 1)) == 800.0
    arr = (ctypes.c_int * 1)(0)
    assert L.csa2_bytes_per_token(arr, 1, 512, 16, 1, 128, 32, 1) < 0


def test_product_path_refuses_cpu_tensors(L):
    import torch
    import long_context_fp4_amd as Lp
    x = torch.zeros((1, 4, 512), dtype=torch.int16)
    with pytest.raises(TypeError):
        Lp.cache_write(x, torch.zeros((1, 4, 128), dtype=torch.int16), torch.ones(2, 512), torch.ones(2, 128), 2)


def test_decode_noalloc_validation(L):
    """The allocation-free layer: the argument checks of the workspace one, and a
    call whose indexer scratch exceeds the static array refused before any HIP call."""
    from long_context_fp4_amd import binding

    def call(**kw):
        a = dict(mode=0, kv=P, B=2, max_n=1000, H=64, k=512, pool_k=0, pool=None, topk=P)
        a.update(kw)
        return L.csa2_decode_layer_noalloc(a["mode"], a["kv"], P, P, P, P, a["B"], a["max_n"], P, P, 16, 1, P,
                                           a["H"], 1.0, a["k"], a["pool_k"], a["pool"], a["topk"], P, P, None)
    assert call(kv=None) == -1
    assert call(mode=5) == -5
    assert call(B=0) == -2 and call(H=0) == -2 and call(k=0) == -2
    assert call(mode=1, pool=None, pool_k=0) == -1               # Reindex needs the pool
    assert call(topk=P + 4) == -3
    assert call(B=4, max_n=1 << 22) == -4 and "static scratch" in err(L)
    assert call(B=1024, max_n=1 << 20) == -4
    assert binding.CSA2_NOALLOC_SCRATCH_BYTES == 64 << 20
    hdr = open(HEADER).read()
    assert "#define CSA2_NOALLOC_SCRATCH_BYTES (64u << 20)" in hdr
