"""Comparison rules shared by the GPU parity tests.

Top-k (the rule the GPU path is held to): with the oracle's scores s over the
visible items, s_k and s_k+1 the k-th and (k+1)-th largest and
gap = (s_k - s_k+1) / |s_k|:
  * gap > 1e-5: the GPU set equals the oracle set;
  * otherwise: the GPU set has k members, holds every item scoring above
    s_k (1 + 1e-5), and every member scores at least s_k (1 - 1e-5).
Attention: |gpu - oracle| <= 2e-3 + 2e-3 |oracle| elementwise.
"""

import numpy as np

REL_GAP = 1e-5
ATOL = RTOL = 2e-3


def check_topk(gpu, ref, score_of, k, n_visible, what=""):
    """gpu, ref: int arrays [k] (ascending, -1 padded); score_of: dict or
    array mapping position -> oracle score for every visible position.
    Returns "exact" or "tie"."""
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    if n_visible <= k:
        assert np.array_equal(gpu, ref), f"{what}: all visible positions expected"
        return "exact"
    g = gpu[gpu >= 0]
    assert len(g) == k and np.all(np.diff(g) > 0), f"{what}: GPU set not k ascending positions"
    if isinstance(score_of, dict):
        pos = np.fromiter(score_of.keys(), dtype=np.int64)
        sc = np.fromiter(score_of.values(), dtype=np.float64)
    else:
        pos = np.arange(len(score_of))
        sc = np.asarray(score_of, dtype=np.float64)
    srt = np.sort(sc)[::-1]
    sk, sk1 = srt[k - 1], srt[k]
    gap = (sk - sk1) / abs(sk) if sk != 0 else 0.0
    if gap > REL_GAP:
        assert np.array_equal(gpu, ref), f"{what}: sets differ with gap {gap:.3g}"
        return "exact"
    lookup = dict(zip(pos.tolist(), sc.tolist())) if not isinstance(score_of, dict) else score_of
    must = pos[sc > sk * (1 + REL_GAP) if sk >= 0 else sc > sk * (1 - REL_GAP)]
    assert set(must.tolist()) <= set(g.tolist()), f"{what}: a clear winner is missing"
    lo = sk * (1 - REL_GAP) if sk >= 0 else sk * (1 + REL_GAP)
    assert all(lookup[int(p)] >= lo for p in g), f"{what}: a member scores below the tie band"
    return "tie"


def check_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance, "
                           f"max err {err.max():.3g}")
    return float(err.max())


def check_hier(gpu_idx, gpu_pool, q, w, k8, ks, bk8, bks, n_vis, k=512, n_blocks=2048, what=""):
    """Hierarchical selection of one query, with nothing skipped on ties.

    The block stage: the GPU's kept blocks (read from its pool) against the
    oracle's block scores, tie-aware like any top-k.  The pool must then be
    exactly the visible positions of those blocks, ascending, -1 padded.  The
    token stage: the GPU's indices against the oracle's top-k of the GPU's
    own pool (so a legitimate block-stage tie cannot hide a token-stage
    error).  k8 / ks / bk8 / bks are the oracle's codes of the sequence.
    Returns (block kind, token kind), each "exact" or "tie"."""
    import oracle
    nb = -(-n_vis // 8)
    bscore = oracle.scores(q, w, bk8[:nb], bks[:nb])
    gpool = np.asarray(gpu_pool)
    gblocks = np.unique(gpool[gpool >= 0] // 8)
    gb = np.full(n_blocks, -1, dtype=np.int64)
    assert len(gblocks) <= n_blocks, f"{what}: more than {n_blocks} blocks in the pool"
    gb[: len(gblocks)] = gblocks
    rb = oracle.top_k(bscore, np.arange(nb), n_blocks)
    kind_b = check_topk(gb, rb, bscore, n_blocks, nb, f"{what} blocks")
    want = (gblocks[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    want = want[want < n_vis]
    assert np.array_equal(gpool[: len(want)], want) and np.all(gpool[len(want):] == -1), \
        f"{what}: the pool is not the visible positions of its blocks"
    ref = oracle.index_pool(q, w, k8, ks, want, k)
    sc = oracle.scores(q, w, k8[want], ks[want])
    kind_t = check_topk(gpu_idx, ref, dict(zip(want.tolist(), sc.tolist())), k, len(want), f"{what} pool")
    return kind_b, kind_t


def check_flat_pool(gpu_idx, gpu_pool, q, w, k8, ks, n_vis, k=512, n_blocks=2048, what=""):
    """Flat selection that also keeps a pool (FLAT_POOL), with nothing
    skipped on ties.  The indices: the flat top-k, tie-aware.  The blocks:
    the GPU's kept blocks (read from its pool) against block scores that are
    the largest oracle score among each block's visible positions,
    tie-aware.  The pool must be exactly the visible positions of those
    blocks, ascending, -1 padded.  Returns (block kind, token kind)."""
    import oracle
    sc = oracle.scores(q, w, k8[:n_vis], ks[:n_vis])
    kind_t = check_topk(gpu_idx, oracle.index_flat(q, w, k8, ks, n_vis, k), sc, k, n_vis, f"{what} indices")
    nb = -(-n_vis // 8)
    bscore = np.array([sc[8 * b: min(8 * b + 8, n_vis)].max() for b in range(nb)])
    gpool = np.asarray(gpu_pool)
    gblocks = np.unique(gpool[gpool >= 0] // 8)
    assert len(gblocks) <= n_blocks, f"{what}: more than {n_blocks} blocks in the pool"
    gb = np.full(n_blocks, -1, dtype=np.int64)
    gb[: len(gblocks)] = gblocks
    rb = oracle.top_k(bscore, np.arange(nb), n_blocks)
    kind_b = check_topk(gb, rb, bscore, n_blocks, nb, f"{what} blocks")
    want = (gblocks[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    want = want[want < n_vis]
    assert np.array_equal(gpool[: len(want)], want) and np.all(gpool[len(want):] == -1), \
        f"{what}: the pool is not the visible positions of its blocks"
    return kind_b, kind_t
