"""Run-to-run and batch-size determinism of every public call.

Each call runs twice on identical inputs (the second time on a workspace the
first left behind) and must give bitwise-identical outputs; a sequence run in a
batch of three and run alone must give bitwise-identical outputs too. The
kernels use LDS and global atomics (histograms, candidate counters, bitmap ORs)
whose order depends on scheduling; their results must not.
"""
import numpy as np
import pytest

from long_context_fp4_amd import synth
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def step(msg):
    """Progress line (flushed), so that a stalled call is named in the output."""
    import sys
    print(f"[determinism] {msg}", file=sys.stderr, flush=True)


def same(a, b, what, bad=None):
    """Bitwise equality (without pytest's element diff, which is slow on large arrays).
    With `bad` (a list) the mismatch is recorded there instead of raised."""
    a, b = host(a), host(b)
    ok = a.shape == b.shape and a.dtype == b.dtype and a.tobytes() == b.tobytes()
    if ok:
        return
    n = int(np.count_nonzero(a != b)) if a.shape == b.shape else -1
    msg = f"{what}: outputs differ bitwise ({n} elements of {a.size})"
    if bad is None:
        raise AssertionError(msg)
    bad.append(msg)


def test_every_call_twice_and_alone():
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(4242)
    m, lens = 2, [80000, 46000, 140000]             # 40000, 23000, 70000 entries
    step("inputs")
    B, H, Hi, k = len(lens), 64, 16, 512
    T = max(lens)
    w_lat, w_idx = dev(synth.merge_weights(rng, m, 512)), dev(synth.merge_weights(rng, m, 128))
    x_lat = dev(synth.hidden_host(rng, (B, T, 512)))
    x_idx = dev(synth.hidden_host(rng, (B, T, 128)))
    ents = np.asarray(lens) // m
    off = np.concatenate([[0], np.cumsum(ents)[:-1]]).astype(np.int64)
    E = int(ents.sum())
    nt, offd, nbd = dev(np.asarray(lens, np.int64)), dev(off), dev(ents.astype(np.int32))

    def write():
        kv = torch.zeros((E, 288), dtype=torch.uint8, device="cuda")
        ik = torch.zeros((E, 64), dtype=torch.uint8, device="cuda")
        iks = torch.zeros((E, 4), dtype=torch.uint8, device="cuda")
        L.cache_write(x_lat, x_idx, w_lat, w_idx, m, kv=kv, ik=ik, iks=iks, n_tokens=nt, out_entry_offset=offd)
        return kv, ik, iks

    step("cache_write x2")
    c1, c2 = write(), write()
    torch.cuda.synchronize()
    for a, b, nm in zip(c1, c2, ("kv", "ik", "iks")):
        same(a, b, f"cache_write {nm}")
    kv, ik, iks = c1
    q = dev(np.stack([synth.latent_query(rng, H) for _ in range(B)]))
    qi = dev(np.stack([synth.indexer_query(rng, Hi) for _ in range(B)]))
    wh = dev(np.stack([synth.head_weights(rng, Hi) for _ in range(B)]))
    qi2 = dev(np.stack([synth.indexer_query(rng, Hi) for _ in range(B)]))
    wh2 = dev(np.stack([synth.head_weights(rng, Hi) for _ in range(B)]))
    max_n = int(ents.max())

    def calls(sel, ws):
        """Every read-path call on the sequences `sel` (their rows, offsets and queries)."""
        o, n = offd[sel].contiguous(), nbd[sel].contiguous()
        qq, qqi, ww, qqi2, ww2 = (t[sel].contiguous() for t in (q, qi, wh, qi2, wh2))
        r = {}

        def sync(what):
            torch.cuda.synchronize()
            step(f"{what} done")
        r["topk_direct"], _, r["scores"] = L.indexer_topk(ik, iks, o, n, max_n, qqi, ww, k=k, want_scores=True,
                                                          workspace=ws)
        sync("indexer direct")
        r["topk_pool"], r["pool"], _ = L.indexer_topk(ik, iks, o, n, max_n, qqi, ww, k=k, pool_k=16384, workspace=ws)
        sync("indexer pool")
        r["topk_reindex"], _, _ = L.indexer_topk(ik, iks, o, n, max_n, qqi2, ww2, cand=r["pool"], k=k, workspace=ws)
        sync("indexer reindex")
        r["attn_out"], r["attn_lse"] = L.sparse_attention(kv, o, n, r["topk_reindex"], qq, workspace=ws)
        sync("attention")
        r["full_top"], _, r["full_out"], r["full_lse"] = L.decode_layer(L.CSA2_FULL, kv, ik, iks, o, n, max_n, qq,
                                                                        q_idx=qqi, w=ww, k=k, workspace=ws)
        sync("decode full")
        r["hsi_top"], pool, r["hsi_out"], r["hsi_lse"] = L.decode_layer(L.CSA2_FULL, kv, ik, iks, o, n, max_n, qq,
                                                                        q_idx=qqi, w=ww, k=k, pool_k=16384,
                                                                        workspace=ws)
        sync("decode full + pool")
        r["rei_top"], _, r["rei_out"], r["rei_lse"] = L.decode_layer(L.CSA2_REINDEX, kv, ik, iks, o, n, max_n, qq,
                                                                     q_idx=qqi2, w=ww2, k=k, pool=pool,
                                                                     workspace=ws)
        sync("decode reindex")
        _, _, r["reuse_out"], r["reuse_lse"] = L.decode_layer(L.CSA2_REUSE, kv, ik, iks, o, n, max_n, qq,
                                                              topk=r["rei_top"], workspace=ws)
        sync("decode reuse")
        r["qmx_top"], _, r["qmx_out"], _ = L.decode_layer(L.CSA2_FULL, kv, ik, iks, o, n, max_n, qq, q_idx=qqi, w=ww,
                                                          score_mode=L.CSA2_SCORE_RELU_W | L.CSA2_SCORE_QMX8, k=k,
                                                          workspace=ws)
        sync("decode full qmx")
        nb_sel = ents[sel] if isinstance(sel, slice) else ents[np.asarray(sel)]
        pos = dev(np.stack([[2 * int(e) - 1, int(e), 3 * int(e) // 2] for e in nb_sel]).astype(np.int64))
        Tq = 3
        qp = qq[:, None].expand(-1, Tq, -1, -1).contiguous()
        qip = qqi[:, None].expand(-1, Tq, -1, -1).contiguous()
        wp = ww[:, None].expand(-1, Tq, -1).contiguous()
        r["pre_top"], r["pre_out"], r["pre_lse"] = L.prefill_layer(kv, ik, iks, o, n, max_n, m, pos, qip, qp, w=wp,
                                                                   k=k, workspace=ws)
        sync("prefill")
        return r

    ws = L.Workspace()
    step("first round")
    first = calls(slice(0, B), ws)
    step("second round")
    second = calls(slice(0, B), ws)
    torch.cuda.synchronize()
    bad = []
    for key in first:
        if key == "scores":                          # defined for positions below each n_entries[b]
            for b in range(B):
                same(first[key][b, :int(ents[b])], second[key][b, :int(ents[b])], f"scores {b} (repeat)", bad)
            continue
        same(first[key], second[key], f"{key} (repeat)", bad)
    step("sequence 2 alone")
    alone = calls([2], L.Workspace())
    torch.cuda.synchronize()
    for key in first:
        if key == "scores":
            same(first[key][2:3, :int(ents[2])], alone[key][:, :int(ents[2])], "scores (sequence 2 alone)", bad)
        else:
            same(first[key][2:3], alone[key], f"{key} (sequence 2 alone)", bad)
    assert not bad, "; ".join(bad)


def test_window_and_append_twice():
    import torch
    import long_context_fp4_amd as L
    rng = np.random.default_rng(77)
    B, H, m = 5, 64, 2
    x = dev(synth.hidden_host(rng, (B, 200, 512)))
    pos0 = dev(np.zeros(B, np.int64))
    q = dev(np.stack([synth.latent_query(rng, H) for _ in range(B)]))
    outs = []
    for _ in range(2):
        win = torch.zeros((B, 128, 544), dtype=torch.uint8, device="cuda")
        L.swa_write(x, pos0, win)
        out = torch.zeros((B, H, 512), dtype=torch.float32, device="cuda")
        lse = torch.full((B, H), float("-inf"), dtype=torch.float32, device="cuda")
        L.swa_attention(win, dev(np.full(B, 128, np.int32)), q, out, lse)
        outs.append((win, out, lse))
    torch.cuda.synchronize()
    for a, b, nm in zip(outs[0], outs[1], ("window", "window out", "window lse")):
        same(a, b, nm)
    wl, wi = dev(synth.merge_weights(rng, m, 512)), dev(synth.merge_weights(rng, m, 128))
    toks = [(dev(synth.hidden_host(rng, (B, 512))), dev(synth.hidden_host(rng, (B, 128)))) for _ in range(5)]
    res = []
    for _ in range(2):
        kv = torch.zeros((B * 4, 288), dtype=torch.uint8, device="cuda")
        ik = torch.zeros((B * 4, 64), dtype=torch.uint8, device="cuda")
        iks = torch.zeros((B * 4, 4), dtype=torch.uint8, device="cuda")
        st_l = torch.zeros((B, m - 1, 512), dtype=torch.int16, device="cuda")
        st_i = torch.zeros((B, m - 1, 128), dtype=torch.int16, device="cuda")
        cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
        ne = torch.zeros(B, dtype=torch.int32, device="cuda")
        for tl, ti in toks:
            L.cache_append(tl, ti, wl, wi, m, st_l, st_i, cnt, dev(np.arange(B, dtype=np.int64) * 4), ne,
                           dev(np.full(B, 4, np.int64)), kv, ik, iks)
        res.append((kv, ik, iks, st_l, st_i, cnt, ne))
    torch.cuda.synchronize()
    for a, b in zip(res[0], res[1]):
        same(a, b, "append")
