"""GPU parity at the full sizes of the hierarchical-indexer and layer-group workloads.

hsi1m: 4 sequences of 1048576 tokens (524288 ratio-2 entries), a Full layer that
keeps a 16384-candidate pool and its top-512, then two Reindex layers over that
pool, each with 64-head attention. group_ragged: 16 sequences of 32768 ..
262144 tokens at ratio 1, layers Full, Reindex, Reuse, Reuse. The caches are
written by the library from seeded device hidden states; the oracle recomputes
every sequence's scores, selections and attention from the GPU-written cache bytes,
and the bytes of sampled sequences from their hidden states.
"""
import numpy as np
import pytest

from oracle import attention as OA
from oracle import cache as OC
from oracle import indexer as OI
from long_context_fp4_amd import synth
from tests.gpu_util import ATTN_REL_TOL, attn_rel_err, check_topk, dev, host

pytestmark = pytest.mark.gpu


def build_cache(L, torch, w, p, keep, one_launch=False):
    """Writes every sequence's cache on the GPU; returns the cache and the host
    hidden states of the sequences in `keep`. one_launch: the sequences' hidden
    states are padded to the longest and written by one call with per-sequence
    token counts and entry offsets (a ragged batch into one buffer)."""
    lens = w.lengths if w.lengths is not None else [w.T] * w.B
    ents = [t // w.m for t in lens]
    off = np.concatenate([[0], np.cumsum(ents)[:-1]]).astype(np.int64)
    E = int(sum(ents))
    kv = torch.empty((E, 288), dtype=torch.uint8, device="cuda")
    ik = torch.empty((E, 64), dtype=torch.uint8, device="cuda")
    iks = torch.empty((E, 4), dtype=torch.uint8, device="cuda")
    hidden = {}
    if one_launch:
        T = max(lens)
        xl = torch.zeros((w.B, T, 512), dtype=torch.int16, device="cuda")
        xi = torch.zeros((w.B, T, 128), dtype=torch.int16, device="cuda")
    for b in range(w.B):
        x_lat, x_idx = synth.hidden_states_device(w, p, b)
        if one_launch:
            xl[b, :lens[b]] = x_lat
            xi[b, :lens[b]] = x_idx
        else:
            rows = slice(int(off[b]), int(off[b]) + ents[b])
            L.cache_write(x_lat[None], x_idx[None], dev(p["w_lat"]), dev(p["w_idx"]), w.m,
                          kv=kv[rows], ik=ik[rows], iks=iks[rows])
        if b in keep:
            hidden[b] = (host(x_lat), host(x_idx))
        del x_lat, x_idx
    if one_launch:
        L.cache_write(xl, xi, dev(p["w_lat"]), dev(p["w_idx"]), w.m, kv=kv, ik=ik, iks=iks,
                      n_tokens=dev(np.asarray(lens, np.int64)), out_entry_offset=dev(off))
        del xl, xi
    torch.cuda.synchronize()
    return kv, ik, iks, off, np.asarray(ents, np.int32), hidden


def check_attention(kv_rows, sel, q, out, lse, what):
    ro, rl = OA.sparse_attention(kv_rows, sel, q)
    err = attn_rel_err(out, ro)
    assert np.all(err <= ATTN_REL_TOL), f"{what}: max rel err {err.max():.3g}"
    assert np.all(np.abs(lse - rl) <= 2e-3), f"{what}: lse"


def check_selection_shape(sel, n, k, what):
    v = sel[sel >= 0]
    assert len(v) == min(n, k), what
    assert np.all(np.diff(v) > 0) and v[0] >= 0 and v[-1] < n, what
    assert np.all(sel[len(v):] == -1), what


def check_cache_bytes(kv, ik, iks, rows, hidden, p, m, what):
    okv, oik, oiks = OC.cache_write(hidden[0], hidden[1], p["w_lat"], p["w_idx"], m)
    assert np.array_equal(kv[rows], okv), what
    assert np.array_equal(ik[rows], oik), what
    assert np.array_equal(iks[rows], oiks), what


def test_hsi1m_full_size():
    """Every sequence end to end against the oracle on the GPU-written cache bytes (pool,
    Full top-512, both Reindex selections, three attentions); sequence 0's bytes also
    bit-exact against the oracle's cache write of its hidden states."""
    import torch
    import long_context_fp4_amd as L
    w = synth.workload("hsi1m")
    p = synth.params(w)
    kv, ik, iks, off, ents, hidden = build_cache(L, torch, w, p, keep=(0,))
    d = dict(kv=kv, ik=ik, iks=iks, entry_offset=dev(off), n_entries=dev(ents), max_n=int(ents.max()),
             workspace=L.Workspace())
    F, R1, R2 = p["layers"]
    topF, pool, outF, lseF = L.decode_layer(L.CSA2_FULL, q=dev(F["q"]), q_idx=dev(F["q_idx"]), w=dev(F["w"]),
                                            pool_k=w.pool_k, **d)
    res = []
    for R in (R1, R2):
        top, _, out, lse = L.decode_layer(L.CSA2_REINDEX, q=dev(R["q"]), q_idx=dev(R["q_idx"]), w=dev(R["w"]),
                                          pool=pool, **d)
        res.append((top, out, lse))
    torch.cuda.synchronize()
    topF, pool, outF, lseF = host(topF), host(pool), host(outF), host(lseF)
    res = [(host(t), host(o), host(l)) for t, o, l in res]
    hkv, hik, hiks = host(kv), host(ik), host(iks)
    del kv, ik, iks, d
    torch.cuda.empty_cache()
    check_cache_bytes(hkv, hik, hiks, slice(int(off[0]), int(off[0]) + int(ents[0])), hidden[0], p, w.m, "seq0 bytes")
    for b in range(w.B):
        n = int(ents[b])
        rows = slice(int(off[b]), int(off[b]) + n)
        ckv, cik, ciks = hkv[rows], hik[rows], hiks[rows]
        check_selection_shape(pool[b], n, w.pool_k, f"pool{b}")
        s = OI.scores(cik, ciks, F["q_idx"][b], F["w"][b], 1)
        check_topk(pool[b], OI.topk(s, np.arange(n), w.pool_k), lambda q: s[q], w.pool_k, f"pool{b}")
        gp = pool[b][pool[b] >= 0]
        check_topk(topF[b], OI.topk(s[gp], gp, w.k), lambda q: s[q], w.k, f"full{b}")
        check_attention(ckv, topF[b], F["q"][b], outF[b], lseF[b], f"full attention {b}")
        for j, (R, (t, o, l)) in enumerate(zip((R1, R2), res)):
            s2 = np.zeros(n, np.float32)
            s2[gp] = OI.scores(cik[gp], ciks[gp], R["q_idx"][b], R["w"][b], 1)
            check_topk(t[b], OI.topk(s2[gp], gp, w.k), lambda q: s2[q], w.k, f"reindex{j} {b}")
            check_attention(ckv, t[b], R["q"][b], o[b], l[b], f"reindex{j} attention {b}")


def test_group_ragged_full_size():
    """The 16 ragged sequences written by one cache-write call at per-sequence offsets;
    every sequence and layer end to end against the oracle on the GPU-written bytes; the
    shortest and longest sequences' bytes also bit-exact against the oracle's write."""
    import torch
    import long_context_fp4_amd as L
    w = synth.workload("group_ragged")
    p = synth.params(w)
    lens = np.asarray(w.lengths)
    keep = (int(lens.argmin()), int(lens.argmax()))
    kv, ik, iks, off, ents, hidden = build_cache(L, torch, w, p, keep=keep, one_launch=True)
    d = dict(kv=kv, ik=ik, iks=iks, entry_offset=dev(off), n_entries=dev(ents), max_n=int(ents.max()),
             workspace=L.Workspace())
    F, R, U1, U2 = p["layers"]
    topF, pool, outF, lseF = L.decode_layer(L.CSA2_FULL, q=dev(F["q"]), q_idx=dev(F["q_idx"]), w=dev(F["w"]),
                                            pool_k=w.pool_k, **d)
    topR, _, outR, lseR = L.decode_layer(L.CSA2_REINDEX, q=dev(R["q"]), q_idx=dev(R["q_idx"]), w=dev(R["w"]),
                                         pool=pool, **d)
    _, _, outU1, lseU1 = L.decode_layer(L.CSA2_REUSE, q=dev(U1["q"]), topk=topR, **d)
    _, _, outU2, lseU2 = L.decode_layer(L.CSA2_REUSE, q=dev(U2["q"]), topk=topR, **d)
    torch.cuda.synchronize()
    topF, pool, topR = host(topF), host(pool), host(topR)
    outs = [host(x) for x in (outF, lseF, outR, lseR, outU1, lseU1, outU2, lseU2)]
    hkv, hik, hiks = host(kv), host(ik), host(iks)
    del kv, ik, iks, d
    torch.cuda.empty_cache()
    for b in keep:
        check_cache_bytes(hkv, hik, hiks, slice(int(off[b]), int(off[b]) + int(ents[b])), hidden[b], p, w.m,
                          f"seq{b} bytes")
    for b in range(w.B):
        n = int(ents[b])
        rows = slice(int(off[b]), int(off[b]) + n)
        ckv, cik, ciks = hkv[rows], hik[rows], hiks[rows]
        check_selection_shape(pool[b], n, w.pool_k, f"pool{b}")
        check_selection_shape(topR[b], n, w.k, f"reindex{b}")
        s = OI.scores(cik, ciks, F["q_idx"][b], F["w"][b], 1)
        check_topk(pool[b], OI.topk(s, np.arange(n), w.pool_k), lambda q: s[q], w.pool_k, f"pool{b}")
        gp = pool[b][pool[b] >= 0]
        check_topk(topF[b], OI.topk(s[gp], gp, w.k), lambda q: s[q], w.k, f"full{b}")
        s2 = np.zeros(n, np.float32)
        s2[gp] = OI.scores(cik[gp], ciks[gp], R["q_idx"][b], R["w"][b], 1)
        check_topk(topR[b], OI.topk(s2[gp], gp, w.k), lambda q: s2[q], w.k, f"reindex{b}")
        for (q, o, l, what) in ((F["q"][b], outs[0][b], outs[1][b], "full"),
                                (R["q"][b], outs[2][b], outs[3][b], "reindex"),
                                (U1["q"][b], outs[4][b], outs[5][b], "reuse1"),
                                (U2["q"][b], outs[6][b], outs[7][b], "reuse2")):
            sel = topF[b] if what == "full" else topR[b]
            check_attention(ckv, sel, q, o, l, f"{what} attention {b}")
