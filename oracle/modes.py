"""CSA2 layer modes composed over one shared cache (one sequence).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

[CS] section "L'architecture : trois leviers contre le cache": each CSA2
layer has one static mode. Full: own main KV, own indexer, new top-512.
Reindex: main KV from elsewhere, own rescoring. Reuse: main KV and indices
both taken over. [F24] section "Tre meccanismi al posto di un solo trucco":
the layers share the main KV and the indexer key; deeper indexing layers
rescore only the pool built by the first Full layer. [TF] section
"Mécanismes de compression du KV-Cache", item 3: Reuse relies on a light
perturbation of the query.

Readings taken: Reindex rescores the shared indexer key (only source layers
store keys) at the Full layer's pool positions; Reuse takes the indices of
the nearest preceding layer that produced indices; every layer runs its own
attention with its own query (a Reuse layer's perturbed query is an input).
"""
from . import attention, indexer

FULL, REINDEX, REUSE = 0, 1, 2


def decode_group(kv, ik, iks, layers, k=512, pool_k=16384, tau=1.0):
    """Run a list of layers over one sequence's shared cache.

    ``layers``: list of dicts with key "mode" and, as the mode needs,
    "q_idx" (uint16 [Hi,128]), "w" (float32 [Hi] or None), "score_mode",
    "q" (uint16 [H,512]). Returns one dict per layer with "topk", "pool"
    (Full only), "out", "lse".
    """
    results = []
    pool = None
    idx = None
    for L in layers:
        r = {}
        if L["mode"] == FULL:
            idx, pool, _ = indexer.full_layer(ik, iks, L["q_idx"], L.get("w"),
                                              L.get("score_mode", indexer.SCORE_RELU_W),
                                              k=k, pool_k=pool_k)
            r["pool"] = pool
        elif L["mode"] == REINDEX:
            if pool is None:
                raise ValueError("Reindex needs a preceding Full layer's pool")
            idx, _ = indexer.reindex_layer(ik, iks, pool, L["q_idx"], L.get("w"),
                                           L.get("score_mode", indexer.SCORE_RELU_W), k=k)
        elif L["mode"] == REUSE:
            if idx is None:
                raise ValueError("Reuse needs indices from a preceding layer")
        else:
            raise ValueError("unknown layer mode")
        r["topk"] = idx
        r["out"], r["lse"] = attention.sparse_attention(kv, idx, L["q"], tau)
        results.append(r)
    return results
