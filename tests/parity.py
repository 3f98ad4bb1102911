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
