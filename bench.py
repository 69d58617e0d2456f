"""Decode benchmark of the FP4 compressed-KV sparse decode path on one MI355X.

One step = one Full CSA2 layer for every sequence of the batch: the indexer
scores all cached entries (packed MXFP4 keys), the top-512 is selected, and all
query heads attend over the dequantized FP4 latent at those positions. The
workload is 32 sequences of 131072 tokens (65536 ratio-2 entries each), 64
query heads, 16 indexer heads; every step is one query token per sequence.

The cache is written once, from seeded synthetic hidden states, by the
library's own cache-write kernel, then copied so that consecutive steps read
different copies (4 copies of the 142.6 MB indexer stream exceed the 256 MB
last-level cache, so the timed passes read HBM). The scoring kernel is timed
by itself with HIP events that the library records around its launch on the
step's stream; the whole step is timed with events around K steps.

The same run also times the cache write on its own workload (8 sequences of
131072 tokens merged at ratio 2, the write128k configuration) and reports it
beside the step as "cache_write", the decode-time append of one token for
each of the 32 sequences (ratio 2: every other call completes a group and
packs 32 entries) as "append", and the sliding-window branch at the step's
shape (the window write of one token per sequence; the attention over 128
window tokens merged into the sparse result) as "swa", and a multi-query
prefill of 32 query tokens of one sequence as "prefill", and the same step
with the quantized-query scoring variant (MXFP8 queries, block-scaled MFMA;
its scores differ from the exact ones) as "score_qmx8". None of these is part
of the timed step, which is the one Full layer the metric is quoted on, scored
exactly.

`traffic` in the roofline object is the HBM traffic of one scoring launch from
rocprofv3 FETCH_SIZE and WRITE_SIZE counters, each scaled by what the same
counter reads for a plain copy of known size (`--copy-calibration` runs that
copy). The figures are kept below with the hash of the kernel source they were
taken on; when the source has changed since, `traffic` is null.

Prints one JSON line. `--gpus N` with N > 1 exits: this path runs on one GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0     # dense bf16 / fp16 matrix peak of MI355X


def call_roofline(nbytes, flops, us):
    """A latency-bound call against both rooflines: its algorithmic bytes and
    matrix flops over its time, as fractions of the HBM and bf16 MFMA peaks."""
    gbs = nbytes / (us * 1e-6) / 1e9
    out = {"bound": "latency", "bytes": nbytes, "achieved_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
    if flops:
        tfl = flops / (us * 1e-6) / 1e12
        out.update({"flops": flops, "achieved_tflops": tfl, "mfma_frac": tfl / MFMA_F16_PEAK_TFLOPS})
    return out
COPIES = 4
SCORE_SOURCES = [os.path.join(ROOT, "long_context_fp4_amd", "csrc", f)
                 for f in ("indexer.hip", "select_dev.h", "device.h", "kernels.h")]
# Counter readings of one scoring launch at the decode128k size (KiB per
# dispatch, medians over the timed launches) and the counters' scale factors
# from the copy calibration; valid for the kernel sources with this hash.
TRAFFIC = {"source_sha": "a248f18cd9b54cc9", "fetch_kib": 70245.0, "write_kib": 606.7,
           "fetch_scale": 2.0, "write_scale": 1.0}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle timing budget")
    ap.add_argument("--no-cache-write", action="store_true",
                    help="skip the legs beside the step (quantized-query scoring, prefill, cache write, window, append)")
    ap.add_argument("--legs", default="all",
                    help="comma-separated legs beside the step to run (qmx8, prefill, fallback, clustered, hsi1m, "
                         "group_ragged, cache_write, swa, append) or 'all'")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB five times (counter calibration)")
    return ap.parse_args()


def source_hash():
    h = hashlib.sha256()
    for path in SCORE_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_bytes():
    """HBM bytes of one scoring launch from the recorded counters, or None."""
    if TRAFFIC is None or TRAFFIC.get("source_sha") != source_hash():
        return None
    return (TRAFFIC["fetch_kib"] * 1024 * TRAFFIC["fetch_scale"] +
            TRAFFIC["write_kib"] * 1024 * TRAFFIC["write_scale"])


def copy_calibration():
    import torch
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 5}), flush=True)


def cache_write_leg(L, synth, torch):
    """Cache write of the write128k workload: one launch over 8 x 131072 tokens."""
    import numpy as np
    w = synth.workload("write128k")
    p = synth.params(w)
    E = w.T // w.m
    xs = [synth.hidden_states_device(w, p, b) for b in range(w.B)]
    x_lat = torch.stack([x[0] for x in xs])
    x_idx = torch.stack([x[1] for x in xs])
    del xs
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    wl, wi = d(p["w_lat"]), d(p["w_idx"])
    kv = torch.empty((w.B * E, 288), dtype=torch.uint8, device="cuda")
    ik = torch.empty((w.B * E, 64), dtype=torch.uint8, device="cuda")
    iks = torch.empty((w.B * E, 4), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        L.cache_write(x_lat, x_idx, wl, wi, w.m, kv=kv, ik=ik, iks=iks)
    n = 10
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record()
        L.cache_write(x_lat, x_idx, wl, wi, w.m, kv=kv, ik=ik, iks=iks)
        e1.record()
    torch.cuda.synchronize()
    us = 1e3 * float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    nbytes = x_lat.numel() * 2 + x_idx.numel() * 2 + kv.numel() + ik.numel() + iks.numel()
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "write128k: 8 sequences x 131072 bf16 tokens (1% outlier channels x20), ratio-2 "
                        "merge, packed to 288 + 68 B per entry",
            "bound": "hbm", "bytes_per_launch": nbytes, "avg_launch_us": us, "achieved": gbs,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}


def append_leg(L, synth, torch):
    """Decode-time append: one token for each of 32 sequences per call, ratio 2."""
    import numpy as np
    B, m, cap, n = 32, 2, 4096, 200
    rng = np.random.default_rng(20261210)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    wl, wi = d(synth.merge_weights(rng, m, 512)), d(synth.merge_weights(rng, m, 128))
    toks = [(d(synth.hidden_host(rng, (B, 512)).view(np.int16)), d(synth.hidden_host(rng, (B, 128)).view(np.int16)))
            for _ in range(8)]
    kv = torch.zeros((B * cap, 288), dtype=torch.uint8, device="cuda")
    ik = torch.zeros((B * cap, 64), dtype=torch.uint8, device="cuda")
    iks = torch.zeros((B * cap, 4), dtype=torch.uint8, device="cuda")
    st_l = torch.zeros((B, m - 1, 512), dtype=torch.int16, device="cuda")
    st_i = torch.zeros((B, m - 1, 128), dtype=torch.int16, device="cuda")
    cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
    ne = torch.zeros(B, dtype=torch.int32, device="cuda")
    off = d(np.arange(B, dtype=np.int64) * cap)
    caps = d(np.full(B, cap, np.int64))
    call = lambda i: L.cache_append(toks[i % 8][0], toks[i % 8][1], wl, wi, m, st_l, st_i, cnt, off, ne, caps,
                                    kv, ik, iks)
    for i in range(10):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # a long first kernel keeps the GPU busy while the host enqueues the calls,
    # so the events time the appends back to back, not the host's call rate
    torch.cuda._sleep(100_000_000)
    e0.record()
    for i in range(n):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / n
    # per pair of calls: 2 tokens read per sequence, one staged (written, then read) and one entry written
    pair_bytes = B * (2 * 1280 + 2 * 1280 + 356)
    return {"workload": f"append: one token for each of {B} sequences per call, ratio {m} (every other call "
                        f"packs {B} entries)", "bound": "latency", "avg_call_us": us, "calls": n,
            "bytes_per_call": pair_bytes / 2, "roofline": call_roofline(pair_bytes / 2, 0, us)}


def swa_leg(L, synth, torch, w):
    """Sliding window at the decode128k shape: 32 sequences, 64 heads, 128 window tokens.

    Times the window write of one token per sequence and the window attention
    merged into a sparse result, each back to back behind a long first kernel.
    """
    import numpy as np
    rng = np.random.default_rng(20261211)
    B, H = w.B, w.H
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    win = torch.zeros((B, 128, 544), dtype=torch.uint8, device="cuda")
    L.swa_write(d(synth.hidden_host(rng, (B, 128, 512)).view(np.int16)), d(np.zeros(B, np.int64)), win)
    toks = d(synth.hidden_host(rng, (B, 1, 512)).view(np.int16))
    q = d(np.stack([synth.latent_query(rng, H) for _ in range(B)]).view(np.int16))
    n_win = d(np.full(B, 128, np.int32))
    out = torch.zeros((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H), float("-inf"), dtype=torch.float32, device="cuda")
    pos = d(np.full(B, 128, np.int64))

    def timed(fn, n=100):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(100_000_000)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / n

    write_us = timed(lambda: L.swa_write(toks, pos, win))
    attn_us = timed(lambda: L.swa_attention(win, n_win, q, out, lse))
    # write: a bf16 token read, a 544-byte row written per sequence; attention:
    # the window rows, the queries, the sparse (out, lse) read and written back,
    # QK and PV over 128 tokens x 512 dims per head
    write_bytes = B * (512 * 2 + 544)
    attn_bytes = B * 128 * 544 + B * H * 512 * 2 + 2 * B * H * (512 + 1) * 4
    attn_flops = 2 * (2 * B * H * 128 * 512)
    return {"workload": f"window of 128 FP8 tokens for each of {B} sequences, {H} heads, merged into the "
                        f"sparse result", "bound": "latency", "write_one_token_us": write_us,
            "attention_us": attn_us, "window_bytes_read": B * 128 * 544,
            "roofline_write": call_roofline(write_bytes, 0, write_us),
            "roofline_attention": call_roofline(attn_bytes, attn_flops, attn_us)}


def prefill_leg(L, synth, torch, w, p, kv, ik, iks):
    """Multi-query prefill on the decode128k cache: 32 query tokens of one sequence
    (its last 32 positions), each with its causal top-512 and attention."""
    import numpy as np
    E = w.T // w.m
    Tq = 32
    rng = np.random.default_rng(20261212)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    pos = d(np.arange(w.T - Tq, w.T, dtype=np.int64)[None])
    q = d(np.stack([synth.latent_query(rng, w.H) for _ in range(Tq)])[None].view(np.int16))
    qi = d(np.stack([synth.indexer_query(rng, w.Hi) for _ in range(Tq)])[None].view(np.int16))
    wh = d(np.stack([synth.head_weights(rng, w.Hi) for _ in range(Tq)])[None])
    off, nb = d(np.zeros(1, np.int64)), d(np.full(1, E, np.int32))
    ws = L.Workspace()
    call = lambda: L.prefill_layer(kv, ik, iks, off, nb, E, w.m, pos, qi, q, w=wh, k=w.k, workspace=ws)
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 20
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / n
    # the sequence's keys once, the gathered rows, queries and outputs; scoring
    # every visible entry for 16 heads and the 64-head attention over k rows
    vis = [min(E, (w.T - Tq + t + 1) // w.m) for t in range(Tq)]
    nbytes = (E * 68 + Tq * w.k * 288 + Tq * (w.H * 512 * 2 + w.Hi * (128 * 2 + 4))
              + Tq * (w.H * (512 + 1) * 4 + w.k * 4))
    flops = sum(vis) * w.Hi * 128 * 2 + Tq * 2 * (2 * w.H * w.k * 512)
    return {"workload": f"prefill: {Tq} query tokens of one 131072-token sequence (65536 entries), each with "
                        f"its causal top-{w.k} and {w.H}-head attention", "avg_call_us": us,
            "query_tokens_per_s": Tq / (us * 1e-6), "roofline": call_roofline(nbytes, flops, us)}


def group_leg(L, synth, torch, name, steps, warmup, copies=3):
    """A layer group at full size, as the decode step of its workload runs it:
    hsi1m (4 x 1048576 tokens at ratio 2: Full with a 16384-candidate pool and its
    top-512, then two Reindex layers over that pool, each with 64-head attention) or
    group_ragged (16 sequences of 32768..262144 tokens at ratio 1: Full, Reindex,
    Reuse, Reuse). The cache is written by the library, then copied so that
    consecutive steps read different copies (more than the 256 MB last-level
    cache). Reports the step time from events around K steps, each layer's time
    from events between the layers (a separate pass), and the step's algorithmic
    cache bytes over its time against the HBM peak."""
    import numpy as np
    w = synth.workload(name)
    p = synth.params(w)
    lens = w.lengths if w.lengths is not None else [w.T] * w.B
    ents = np.asarray([t // w.m for t in lens], np.int64)
    off = np.concatenate([[0], np.cumsum(ents)[:-1]]).astype(np.int64)
    E = int(ents.sum())
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kv = torch.empty((E, 288), dtype=torch.uint8, device="cuda")
    ik = torch.empty((E, 64), dtype=torch.uint8, device="cuda")
    iks = torch.empty((E, 4), dtype=torch.uint8, device="cuda")
    wl, wi = d(p["w_lat"]), d(p["w_idx"])
    for b in range(w.B):
        x_lat, x_idx = synth.hidden_states_device(w, p, b)
        r = slice(int(off[b]), int(off[b] + ents[b]))
        L.cache_write(x_lat[None], x_idx[None], wl, wi, w.m, kv=kv[r], ik=ik[r], iks=iks[r])
        del x_lat, x_idx
    torch.cuda.synchronize()
    cs = [(kv, ik, iks)] + [(kv.clone(), ik.clone(), iks.clone()) for _ in range(copies - 1)]
    offd, nbd = d(off), d(ents.astype(np.int32))
    max_n = int(ents.max())
    ws = L.Workspace()
    layers = []
    for Lr in p["layers"]:
        layers.append({"mode": Lr["mode"], "q": d(Lr["q"].view(np.int16)),
                       "q_idx": d(Lr["q_idx"].view(np.int16)) if "q_idx" in Lr else None,
                       "w": d(Lr["w"]) if Lr.get("w") is not None else None,
                       "topk": torch.empty((w.B, w.k), dtype=torch.int32, device="cuda"),
                       "out": torch.empty((w.B, w.H, 512), dtype=torch.float32, device="cuda"),
                       "lse": torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")})
    pool = torch.empty((w.B, w.pool_k), dtype=torch.int32, device="cuda")

    def step(i, evs=None):
        c = cs[i % copies]
        src = None                                   # the layer whose indices a Reuse layer takes
        for j, y in enumerate(layers):
            if evs is not None:
                evs[j].record()
            if y["mode"] == 0:
                L.decode_layer(L.CSA2_FULL, c[0], c[1], c[2], offd, nbd, max_n, y["q"], q_idx=y["q_idx"], w=y["w"],
                               k=w.k, pool_k=w.pool_k, pool=pool, topk=y["topk"], out=y["out"], lse=y["lse"],
                               workspace=ws)
                src = y
            elif y["mode"] == 1:
                L.decode_layer(L.CSA2_REINDEX, c[0], c[1], c[2], offd, nbd, max_n, y["q"], q_idx=y["q_idx"],
                               w=y["w"], k=w.k, pool=pool, topk=y["topk"], out=y["out"], lse=y["lse"], workspace=ws)
                src = y
            else:
                L.decode_layer(L.CSA2_REUSE, c[0], c[1], c[2], offd, nbd, max_n, y["q"], topk=src["topk"],
                               out=y["out"], lse=y["lse"], workspace=ws)
        if evs is not None:
            evs[len(layers)].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    step_us = 1e3 * e0.elapsed_time(e1) / steps
    per = np.zeros(len(layers))
    for i in range(steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(layers) + 1)]
        step(i, evs)
        torch.cuda.synchronize()
        per += [1e3 * evs[j].elapsed_time(evs[j + 1]) for j in range(len(layers))]
    per /= steps
    names = {0: "full", 1: "reindex", 2: "reuse"}
    idx_bytes = int(ents.sum()) * 68
    n_rei = sum(1 for y in layers if y["mode"] == 1)
    rei_bytes = n_rei * int(np.minimum(ents, w.pool_k).sum()) * 68
    gather_bytes = len(layers) * int(np.minimum(ents, w.k).sum()) * 288
    nbytes = idx_bytes + rei_bytes + gather_bytes
    gbs = nbytes / (step_us * 1e-6) / 1e9
    del cs, kv, ik, iks
    torch.cuda.empty_cache()
    return {"workload": f"{name}: {w.B} sequences, " + (f"{w.T} tokens each" if w.lengths is None else
                                                        f"{min(lens)}..{max(lens)} tokens") +
                        f" at ratio {w.m}, layers " + ", ".join(names[y["mode"]] for y in layers) +
                        f", pool {w.pool_k}, top-{w.k}, {w.H} heads",
            "ms_per_step": step_us / 1e3, "query_tokens_per_s": w.B / (step_us * 1e-6),
            "layer_us": {f"{j}:{names[y['mode']]}": float(per[j]) for j, y in enumerate(layers)},
            "bytes_per_step": nbytes, "bytes": {"indexer_full": idx_bytes, "indexer_reindex": rei_bytes,
                                                "gathered_rows": gather_bytes},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS}}


def fallback_leg(L, torch, w, E, copies, off, nb, q, wh, ws, steps):
    """The decode128k step with an all-zero indexer query: every score is 0, so every
    local candidate list overflows and the top-k finish takes its fallback (a rescore
    and a histogram of the whole sequence); the top-512 is then positions 0..511."""
    q_idx0 = torch.zeros((w.B, w.Hi, 128), dtype=torch.int16, device="cuda")
    topk = torch.empty((w.B, w.k), dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    call = lambda i: L.decode_layer(L.CSA2_FULL, *copies[i % len(copies)], off, nb, E, q, q_idx=q_idx0, w=wh,
                                    k=w.k, topk=topk, out=out, lse=lse, workspace=ws)
    call(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / steps
    ok = bool((topk == torch.arange(w.k, device="cuda", dtype=torch.int32)[None]).all())
    return {"workload": "decode128k with an all-zero indexer query (every score ties at 0): the top-k "
                        "finish's fallback path", "ms_per_step": us / 1e3, "topk_is_first_512": ok}


def clustered_leg(L, torch, w, E, copies, off, nb, q, q_idx, wh, ws, steps):
    """The decode128k step with the top keys of every sequence clustered in one
    chunk: the E8M0 scales of 700 rows at the start of each sequence's last chunk
    of 1024 entries are raised by 2^6, so those rows hold the sequence's top-512
    and that chunk's local cutoff lies far above every other chunk's. Too few
    keys reach the highest cutoff; the finish rescores that chunk alone and
    takes every other chunk's listed keys. Checks that the top-512 lies in the
    cluster."""
    lo = E - 1024
    cl = []
    for kv, ik, iks in copies:
        x = iks.clone().view(w.B, E, 4)
        x[:, lo:lo + 700] = torch.clamp(x[:, lo:lo + 700].to(torch.int32) + 6, max=254).to(torch.uint8)
        cl.append((kv, ik, x.view(-1, 4)))
    topk = torch.empty((w.B, w.k), dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    call = lambda i: L.decode_layer(L.CSA2_FULL, *cl[i % len(cl)], off, nb, E, q, q_idx=q_idx, w=wh,
                                    k=w.k, topk=topk, out=out, lse=lse, workspace=ws)
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / steps
    inside = bool(((topk >= lo) & (topk < lo + 700)).all())
    del cl
    return {"workload": "decode128k with each sequence's top keys clustered in its last chunk (700 rows with "
                        "E8M0 scales raised by 2^6): the finish rescores that chunk only",
            "ms_per_step": us / 1e3, "query_tokens_per_s": w.B / (us * 1e-6), "topk_in_cluster": inside}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_cache(L, synth, torch, w, p):
    E = w.T // w.m
    kv = torch.empty((w.B * E, 288), dtype=torch.uint8, device="cuda")
    ik = torch.empty((w.B * E, 64), dtype=torch.uint8, device="cuda")
    iks = torch.empty((w.B * E, 4), dtype=torch.uint8, device="cuda")
    d = lambda a: torch.from_numpy(a).cuda()
    for b in range(w.B):
        x_lat, x_idx = synth.hidden_states_device(w, p, b)
        L.cache_write(x_lat[None], x_idx[None], d(p["w_lat"]), d(p["w_idx"]), w.m,
                      kv=kv[b * E:(b + 1) * E], ik=ik[b * E:(b + 1) * E], iks=iks[b * E:(b + 1) * E])
    torch.cuda.synchronize()
    return kv, ik, iks


def _oracle_steps(args):
    """One host worker of the CPU baseline: the oracle's decode step (scores, top-k,
    attention) on one sequence, repeated for `budget` seconds with BLAS on one thread.
    Returns (steps done, seconds)."""
    kv, ik, iks, q_idx, wh, q, k, budget = args
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attention as OA
    from oracle import indexer as OI
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            n = ik.shape[0]
            s = OI.scores(ik, iks, q_idx, wh, OI.SCORE_RELU_W)
            top = OI.topk(s, np.arange(n), k)
            OA.sparse_attention(kv, top, q, 1.0)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return done, el


def host_cpu():
    """(usable cores, model name) of this host."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def cpu_baseline(w, p, budget_s):
    """The oracle's decode step (scores, top-512, attention) on a sample of the same
    workload: on one core, then on all usable host cores (one oracle process per core,
    each on one sequence of the sample, BLAS on one thread; up to 16 processes, this
    host's share of a one-GPU machine)."""
    import multiprocessing as mp
    import numpy as np
    from long_context_fp4_amd import synth
    from oracle import cache as OC
    import torch

    Lr = p["layers"][0]
    seqs = [0, 1]
    caches = []
    for b in seqs:
        x_lat, x_idx = synth.hidden_states_device(w, p, b)
        xl = x_lat.cpu().numpy().view(np.uint16)
        xi = x_idx.cpu().numpy().view(np.uint16)
        caches.append(OC.cache_write(xl, xi, p["w_lat"], p["w_idx"], w.m))
    del x_lat, x_idx
    torch.cuda.empty_cache()
    job = lambda i, budget: (*caches[i % 2], Lr["q_idx"][seqs[i % 2]], Lr["w"][seqs[i % 2]],
                             Lr["q"][seqs[i % 2]], w.k, budget)
    one_done, one_s = _oracle_steps(job(0, budget_s / 2))
    cores, model = host_cpu()
    nproc = max(1, min(cores, 16))
    with mp.get_context("spawn").Pool(nproc) as pool:
        res = pool.map(_oracle_steps, [job(i, budget_s / 2) for i in range(nproc)])
    all_rate = sum(d / s for d, s in res)
    return {"value": all_rate, "unit": "query-tokens/s", "cores": nproc, "kind": "oracle",
            "cpu_model": model, "host_cores": cores,
            "one_core": {"value": one_done / one_s, "cores": 1, "steps": one_done, "seconds": one_s},
            "sample": f"decode steps (one query token each) of the decode128k workload on sequences {seqs} "
                      f"(65536 entries, 64 heads, 16 indexer heads, top-512): the numpy oracle in {nproc} "
                      f"processes at once (BLAS on one thread each, sequences alternating), "
                      f"{sum(d for d, _ in res)} steps in {max(s for _, s in res):.1f} s; one core alone: "
                      f"{one_done} steps in {one_s:.1f} s"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              f"(the path shards by whole sequences, with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration()
        return
    import numpy as np
    import torch
    import long_context_fp4_amd as L
    from long_context_fp4_amd import synth

    w = synth.workload("decode128k")
    p = synth.params(w)
    E = w.T // w.m
    log("writing the cache")
    kv, ik, iks = build_cache(L, synth, torch, w, p)
    copies = [(kv, ik, iks)] + [(kv.clone(), ik.clone(), iks.clone()) for _ in range(COPIES - 1)]
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    Lr = p["layers"][0]
    q = d(Lr["q"].view(np.int16))
    q_idx = d(Lr["q_idx"].view(np.int16))
    wh = d(Lr["w"])
    off = d(np.arange(w.B, dtype=np.int64) * E)
    nb = d(np.full(w.B, E, np.int32))
    ws = L.Workspace()
    topk = torch.empty((w.B, w.k), dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")

    def step(i, evs=None, score_mode=L.CSA2_SCORE_RELU_W):
        c = copies[i % COPIES]
        if evs is not None:
            L.set_profile_events(*evs)
        L.decode_layer(L.CSA2_FULL, c[0], c[1], c[2], off, nb, E, q, q_idx=q_idx, w=wh, k=w.k,
                       score_mode=score_mode, topk=topk, out=out, lse=lse, workspace=ws)

    def timed_steps(score_mode):
        """(ms per step over K steps, average scoring-launch time in us)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(a.steps):
            step(i, score_mode=score_mode)
        e1.record()
        torch.cuda.synchronize()
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(a.steps)]
        for x, y in pairs:
            x.record()
            y.record()
        torch.cuda.synchronize()
        for i in range(a.steps):
            step(i, pairs[i], score_mode=score_mode)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / a.steps, 1e3 * float(np.mean([x.elapsed_time(y) for x, y in pairs]))

    log(f"warmup {a.warmup}")
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    # whole-step timing: events around K steps
    ev_s = torch.cuda.Event(enable_timing=True)
    ev_e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev_s.record()
    for i in range(a.steps):
        step(i)
    ev_e.record()
    torch.cuda.synchronize()
    total_ms = ev_s.elapsed_time(ev_e)

    # scoring kernel alone: events recorded by the library around its launch
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    for e0, e1 in pairs:
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    for i in range(a.steps):
        step(i, pairs[i])
    torch.cuda.synchronize()
    score_ms = [e0.elapsed_time(e1) for e0, e1 in pairs]
    score_avg_us = 1e3 * float(np.mean(score_ms))
    pct = lambda v: {"p10": float(np.percentile(v, 10)), "median": float(np.median(v)),
                     "p90": float(np.percentile(v, 90))}

    steps_per_s = a.steps / (total_ms / 1e3)
    qtok_s = w.B * steps_per_s
    idx_bytes = w.B * E * 68                      # packed indexer keys read by one scoring launch
    gather_bytes = w.B * w.k * 288                # latent rows read by the attention
    achieved = idx_bytes / (score_avg_us * 1e-6) / 1e9
    step_gbs = (idx_bytes + gather_bytes) / (total_ms / a.steps * 1e-3) / 1e9
    res = {
        "metric": "decode query-tokens/sec at 128K ctx; cache-read HBM GB/s vs peak (1 GPU)",
        "value": qtok_s,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": total_ms / a.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4 storage (E2M1 + E4M3/E8M0 scales); bf16 x bf16 MFMA scoring and fp16 x fp16 MFMA "
                 "attention, f32 accumulation and softmax",
        "data": "synthetic: seeded N(0,1) bf16 hidden states packed to FP4 by the library; seeded queries",
        "config": {"workload": "decode128k: 32 sequences x 131072 tokens (65536 ratio-2 entries), one Full "
                               "layer: indexer over all entries (16 heads), top-512, attention with 64 heads "
                               "over the 512-d FP4 latent",
                   "batch": w.B, "context_tokens": w.T, "entries_per_seq": E, "heads": w.H,
                   "indexer_heads": w.Hi, "k": w.k, "cache_copies": COPIES},
        "roofline": {"bound": "hbm", "kernel": "score_kernel (indexer scoring pass)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_bytes(),
                     "bytes_per_launch": idx_bytes, "avg_launch_us": score_avg_us,
                     "launch_us": pct(1e3 * np.array(score_ms))},
        "step_cache_read_gbs": step_gbs,
    }
    log(f"step {total_ms / a.steps * 1e3:.1f} us, scoring kernel {score_avg_us:.1f} us "
        f"({achieved:.0f} GB/s), {qtok_s:.0f} query-tokens/s")
    legs = set(("qmx8 prefill fallback clustered hsi1m group_ragged cache_write swa append".split()
                 if a.legs == "all" else a.legs.split(",")) if not a.no_cache_write else [])
    if "qmx8" in legs:
        log("quantized-query scoring leg")
        qmode = L.CSA2_SCORE_RELU_W | L.CSA2_SCORE_QMX8
        for i in range(a.warmup):
            step(i, score_mode=qmode)
        ms, sus = timed_steps(qmode)
        res["score_qmx8"] = {
            "workload": "the same decode128k step with the quantized-query variant: MXFP8 indexer queries "
                        "and one block-scaled FP8 x FP4 MFMA per 16 entries (not the exact path)",
            "ms_per_step": ms, "query_tokens_per_s": w.B / (ms * 1e-3), "score_avg_launch_us": sus,
            "score_achieved_gbs": idx_bytes / (sus * 1e-6) / 1e9,
            "score_frac": idx_bytes / (sus * 1e-6) / 1e9 / HBM_PEAK_GBS}
        log(f"quantized-query step {ms * 1e3:.1f} us, scoring {sus:.1f} us")
    if "prefill" in legs:
        log("prefill leg")
        res["prefill"] = prefill_leg(L, synth, torch, w, p, kv, ik, iks)
        log(f"prefill {res['prefill']['avg_call_us']:.1f} us for 32 query tokens")
    if "fallback" in legs:
        log("fallback leg")
        res["fallback"] = fallback_leg(L, torch, w, E, copies, off, nb, q, wh, ws, min(a.steps, 20))
        log(f"fallback step {res['fallback']['ms_per_step'] * 1e3:.1f} us")
    if "clustered" in legs:
        log("clustered leg")
        res["clustered"] = clustered_leg(L, torch, w, E, copies, off, nb, q, q_idx, wh, ws, min(a.steps, 50))
        log(f"clustered step {res['clustered']['ms_per_step'] * 1e3:.1f} us")
    del copies, kv, ik, iks
    torch.cuda.empty_cache()
    for name in ("hsi1m", "group_ragged"):
        if name in legs:
            log(f"{name} leg")
            res[name] = group_leg(L, synth, torch, name, min(a.steps, 50), min(a.warmup, 5))
            log(f"{name} step {res[name]['ms_per_step'] * 1e3:.1f} us, layers {res[name]['layer_us']}")
    if "cache_write" in legs:
        log("cache write leg (write128k)")
        res["cache_write"] = cache_write_leg(L, synth, torch)
        log(f"cache write {res['cache_write']['avg_launch_us']:.1f} us "
            f"({res['cache_write']['achieved']:.0f} GB/s)")
    if "swa" in legs:
        log("sliding-window leg")
        res["swa"] = swa_leg(L, synth, torch, w)
        log(f"window attention {res['swa']['attention_us']:.2f} us")
    if "append" in legs:
        log("append leg")
        res["append"] = append_leg(L, synth, torch)
        log(f"append {res['append']['avg_call_us']:.2f} us per call")
    if not a.no_cpu_baseline:
        log("timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline(w, p, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
