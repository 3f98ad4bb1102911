"""Indexer of the CSA2 step: scores, top-k selection, flat and hierarchical.

TEST INFRASTRUCTURE: see oracle/__init__.py for who may use this package.

What the pages fix (agentnet.co.il "DeepSeek launches V4.1-Flash ...",
section "CSA2: compression along the layer axis"): a Full layer projects an
indexer K and picks 512 fresh positions; a Reindex layer ranks the last Full
layer's indexer K with its own indexer Q; the decoder's hierarchical sparse
indexer lets a Full layer build a pool of at most 16,384 candidate positions
made of 2,048 blocks of 8.

Readings (the pages give no formula):
  * score of position p for one query: s_p = ks_p * sum_h w_h * max(0, q_h . k_p)
    over the 4 indexer heads h, with q_h and k_p the E4M3 code values (the
    indexer key k_p is shared by the heads; w_h defaults to 1).  With
    per-head keys (k8 of shape [n, 4, 64]) head h dots its own key:
    s_p = ks_p * sum_h w_h * max(0, q_h . k_{p,h}).  The inner
    dot of E4M3 values is exact in float64 (every value is an integer times
    2**-9 below 2**18, so 64 products stay below 2**42 units), the rest is
    float64 arithmetic;
  * top-k: order by score descending, then position ascending; keep the first
    min(k, n); report them in ascending position, padded with -1;
  * hierarchical: the same score over the block keys, top 2,048 blocks (ties
    to the lower block), the pool is every visible position of those blocks,
    then top-512 positions inside the pool;
  * flat with a pool (the other reading of the same section: the pool comes
    from the Full layer's own token scores, aggregated per block): every
    visible position is scored and the top 512 are the indices; a block of 8
    scores the largest score among its visible positions (so the blocks of
    the 512 indices are always kept), top 2,048 blocks (ties to the lower
    block), the pool is every visible position of those blocks.
"""

import numpy as np

from .formats import e4m3_value

TOP_K = 512
N_BLOCKS = 2048
BLOCK = 8


def scores(idx_q, idx_w, k8, ks):
    """Scores of one query against keys.

    idx_q u8[4, 64] E4M3 codes; idx_w f32[4] or None; k8 u8[n, 64] (shared
    key) or u8[n, 4, 64] (per-head keys); ks f32[n] -> float64[n]."""
    q = e4m3_value(np.asarray(idx_q))                          # [4, 64]
    w = np.ones(q.shape[0]) if idx_w is None else np.asarray(idx_w, dtype=np.float64)
    k = e4m3_value(np.asarray(k8))                             # [n, 64] or [n, 4, 64]
    if k.ndim == 3:
        dots = (k * q[None, :, :]).sum(axis=2)                 # [n, 4], exact
    else:
        dots = k @ q.T                                         # [n, 4], exact
    per_head = np.maximum(dots, 0.0) * w[None, :]
    return np.asarray(ks, dtype=np.float64) * per_head.sum(axis=1)


def scores_many(idx_q, idx_w, k8, ks):
    """Scores of n queries against the same keys, float64 [n, m]: row i is
    scores(idx_q[i], idx_w[i], k8, ks) (idx_w None: all weights 1), with the
    keys decoded once for all queries.

    idx_q u8[n, 4, 64]; idx_w f32[n, 4] or None; k8 u8[m, 64] or per-head
    u8[m, 4, 64]; ks f32[m]."""
    q = e4m3_value(np.asarray(idx_q))                          # [n, 4, 64]
    n, h, c = q.shape
    w = np.ones((n, h)) if idx_w is None else np.asarray(idx_w, dtype=np.float64)
    k = e4m3_value(np.asarray(k8))                             # [m, 64] or [m, 4, 64]
    if k.ndim == 3:
        dots = np.stack([k[:, j, :] @ q[:, j, :].T for j in range(h)], axis=2)  # [m, n, 4], exact
    else:
        dots = (k @ q.reshape(n * h, c).T).reshape(-1, n, h)   # [m, n, 4], exact
    per_head = np.maximum(dots, 0.0) * w[None, :, :]
    return (np.asarray(ks, dtype=np.float64)[:, None] * per_head.sum(axis=2)).T


def top_k(score, positions, k):
    """Top-k positions of (score, position) pairs: score descending, position
    ascending on ties; returned ascending, padded with -1 to length k."""
    score = np.asarray(score, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    order = np.lexsort((positions, -score))                    # last key is primary
    chosen = np.sort(positions[order[:k]])
    out = np.full(k, -1, dtype=np.int32)
    out[: len(chosen)] = chosen
    return out


def visible_entries(q_pos, ratio):
    """Number of entries a query at token position q_pos may see: entry j
    covers tokens ratio*j .. ratio*j + ratio - 1 and is visible once its last
    token is at or before the query."""
    return (q_pos + 1) // ratio


def index_flat(idx_q, idx_w, k8, ks, n_visible, k=TOP_K):
    """Flat indexer: score every visible entry, keep the top k."""
    s = scores(idx_q, idx_w, k8[:n_visible], ks[:n_visible])
    return top_k(s, np.arange(n_visible), k)


def index_pool(idx_q, idx_w, k8, ks, pool, k=TOP_K):
    """Top-k restricted to a candidate pool of positions (-1 entries ignored)."""
    pool = np.asarray(pool, dtype=np.int64)
    pool = pool[pool >= 0]
    s = scores(idx_q, idx_w, k8[pool], ks[pool])
    return top_k(s, pool, k)


def index_hier(idx_q, idx_w, k8, ks, bk8, bks, n_visible, k=TOP_K,
               n_blocks=N_BLOCKS, block=BLOCK):
    """Hierarchical indexer: blocks first, then positions inside the pool.

    Returns (indices i32[k], pool i32[n_blocks * block] ascending, -1 padded)."""
    nb_visible = -(-n_visible // block)
    bs = scores(idx_q, idx_w, bk8[:nb_visible], bks[:nb_visible])
    chosen_blocks = top_k(bs, np.arange(nb_visible), n_blocks)
    chosen_blocks = chosen_blocks[chosen_blocks >= 0]
    pos = (chosen_blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    pos = pos[pos < n_visible]
    pool = np.full(n_blocks * block, -1, dtype=np.int32)
    pool[: len(pos)] = pos
    return index_pool(idx_q, idx_w, k8, ks, pos, k), pool


def index_flat_pool(idx_q, idx_w, k8, ks, n_visible, k=TOP_K, n_blocks=N_BLOCKS, block=BLOCK):
    """Flat indexer that also keeps a pool built from the same token scores:
    block b (positions b*block .. b*block + block - 1) scores the largest
    score of its visible positions; the top n_blocks blocks are kept.

    Returns (indices i32[k] as index_flat, pool i32[n_blocks * block] ascending, -1 padded)."""
    s = scores(idx_q, idx_w, k8[:n_visible], ks[:n_visible])
    indices = top_k(s, np.arange(n_visible), k)
    nb_visible = -(-n_visible // block)
    padded = np.full(nb_visible * block, -np.inf)
    padded[:n_visible] = s
    bs = padded.reshape(nb_visible, block).max(axis=1)        # block max over visible positions
    chosen_blocks = top_k(bs, np.arange(nb_visible), n_blocks)
    chosen_blocks = chosen_blocks[chosen_blocks >= 0]
    pos = (chosen_blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    pos = pos[pos < n_visible]
    pool = np.full(n_blocks * block, -1, dtype=np.int32)
    pool[: len(pos)] = pos
    return indices, pool
