"""The static Full / Reindex / Reuse layer plan of a CSA2 group.

TEST INFRASTRUCTURE: see oracle/__init__.py for who may use this package.

What the pages fix (agentnet.co.il "DeepSeek launches V4.1-Flash ...",
section "CSA2: compression along the layer axis"; tgviewer.app sof_news24
"DeepSeek V4.1 Flash: new architecture ...", section "Layers no longer store
everything independently"): every layer has one fixed mode.  Full brings its
own main KV and indexer K and picks fresh indices; Reindex keeps the main KV
and indexer K of the last Full layer but ranks them with its own indexer Q;
Reuse keeps both the KV and the latest indices and runs no indexer.  The
decoder groups are Full + 3 Reuse, then Reindex + 3 Reuse.

Readings:
  * ai-wave.ru ("DeepSeek V4.1-Flash: 1M context ...", third paragraph) says
    Reindex keeps the indices too; the two other pages say it ranks afresh,
    which is what is done here;
  * "latest indices" are those of the most recent Full or Reindex layer, also
    from an earlier call on the same state;
  * every layer has its own attention Q and its own sliding-window rows;
  * a Full layer receives its KV already encoded (the projection that makes it
    needs model weights).
"""

import numpy as np

from .attention import sparse_swa_attention
from .indexer import TOP_K, index_flat, index_flat_pool, index_hier, index_pool, visible_entries

FULL, REINDEX, REUSE = 0, 1, 2


def new_state():
    return {"kv": None, "indices": None, "pool": None}


def _index_one(kind, kv, b, idx_q, idx_w, n_vis, k):
    if kind == "flat":
        return index_flat(idx_q, idx_w, kv["k8"][b], kv["ks"][b], n_vis, k), None
    if kind == "hier":
        return index_hier(idx_q, idx_w, kv["k8"][b], kv["ks"][b], kv["bk8"][b],
                          kv["bks"][b], n_vis, k)
    if kind == "flatpool":
        return index_flat_pool(idx_q, idx_w, kv["k8"][b], kv["ks"][b], n_vis, k)
    raise ValueError(kind)


def run_group(layers, state, q_pos0, n_entries, swa_pos0, ratio=1,
              softmax_scale=1.0, kind="flat", reindex_kind="flat", k=TOP_K):
    """Run a plan of layers in order; returns one float32 [B, n_q, 16, 512] per layer.

    layers: list of dicts with "mode", "q" (u16 [B, n_q, 16, 512]), "swa"
    (u16 [B, rows, 512]), "idx_q" (u8 [B, n_q, 4, 64]) and "idx_w"
    (f32 [B, n_q, 4] or None) for Full and Reindex, and "kv" for Full: per
    sequence lists "nib", "scale", "k8", "ks" (+ "bk8", "bks" for kind "hier").
    state: dict from new_state(), updated in place.
    kind "flatpool" indexes Full layers flat and keeps the pool of the blocks
    their token scores rank highest (index_flat_pool).  reindex_kind "pool"
    ranks only the pool kept by the last Full layer instead of every visible
    position; a Full layer that keeps no pool (kind "flat") drops the pool
    of an earlier one, which belonged to the KV it replaces."""
    outs = []
    for layer in layers:
        mode = layer["mode"]
        q = layer["q"]
        B, n_q = q.shape[0], q.shape[1]
        if mode == FULL:
            state["kv"] = layer["kv"]
        elif state["kv"] is None:
            raise RuntimeError("Reindex/Reuse layer before any Full layer")
        kv = state["kv"]
        if mode in (FULL, REINDEX):
            idx = np.full((B, n_q, k), -1, dtype=np.int32)
            keeps_pool = mode == FULL and kind in ("hier", "flatpool")
            pools = [[None] * n_q for _ in range(B)] if keeps_pool else None
            for b in range(B):
                for i in range(n_q):
                    n_vis = min(int(n_entries[b]), visible_entries(int(q_pos0[b]) + i, ratio))
                    w = None if layer.get("idx_w") is None else layer["idx_w"][b, i]
                    if mode == REINDEX and reindex_kind == "pool":
                        if state["pool"] is None:
                            raise RuntimeError("pool Reindex needs a Full layer that keeps a pool")
                        idx[b, i] = index_pool(layer["idx_q"][b, i], w, kv["k8"][b],
                                               kv["ks"][b], state["pool"][b][i], k)
                        continue
                    this_kind = kind if mode == FULL else "flat"
                    idx[b, i], pool = _index_one(this_kind, kv, b, layer["idx_q"][b, i],
                                                 w, n_vis, k)
                    if pools is not None:
                        pools[b][i] = pool
            state["indices"] = idx
            if mode == FULL:
                state["pool"] = pools
        elif state["indices"] is None:
            raise RuntimeError("Reuse layer before any indices exist")
        idx = state["indices"]
        out = np.empty(q.shape, dtype=np.float32)
        for b in range(B):
            for i in range(n_q):
                out[b, i] = sparse_swa_attention(
                    q[b, i], kv["nib"][b], kv["scale"][b], idx[b, i], layer["swa"][b],
                    int(swa_pos0[b]), int(q_pos0[b]) + i, softmax_scale)
        outs.append(out)
    return outs
