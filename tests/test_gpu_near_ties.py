"""Top-k sets on keys built to be near-ties under float32 arithmetic.

The keys are E4M3 codes of +-448 in most channels, so each dot product is a
sum of large products that nearly cancel (the sum of |products| is 10 to 50
times the score), and the float32 error of a score (an fp8 MFMA's or a
binary32 dot's) is of the order of the gaps between the scores around the
512th.  Around the 512th the scores are spaced 1.5e-5 .. 6e-5 apart
(relative), so the 512th / 513th gap exceeds 1e-5 and the GPU set must
equal the oracle's exactly: the select has to settle the near ties on exact
scores.  One, two and four query rows per sequence (the VALU scan, and the
MFMA scan shared by two and by four queries; the rows of a sequence carry
the same query, so each row has the construction's gaps)."""

import numpy as np
import pytest
import torch

import oracle
from parity import check_topk

@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_decode_fp4_amd as m
    return m


def near_tie_keys(seed, n, n_high=489, chain_min=40):
    """(query codes [4, 64], key codes [n, 64], key scales [n]): n_high keys
    scoring far above the rest (scale 4), a chain of keys whose scores step
    down by 1.5e-5 .. 6e-5 relative (scale 1), the others near zero (scale
    1e-3), at positions drawn by the seed."""
    rng = np.random.default_rng(seed)
    q = oracle.e4m3_encode(rng.standard_normal((4, 64)))
    base = np.where(rng.random(64) < 0.5, 0x7E, 0xFE).astype(np.uint8)
    var = []
    for j in range(64):
        for c in range(0x7F):
            for sgn in (0, 0x80):
                v = base.copy()
                v[j] = c | sgn
                var.append(v)
    V = np.unique(np.stack(var), axis=0)
    s = oracle.scores(q, None, V, np.ones(len(V), np.float32))
    order = np.argsort(-s, kind="stable")
    best = []
    for start in range(0, min(len(order), 4000), 25):
        chain = [order[start]]
        for i in order[start + 1:]:
            g = (s[chain[-1]] - s[i]) / abs(s[chain[-1]])
            if g > 6e-5:
                break
            if g >= 1.5e-5:
                chain.append(i)
        if len(chain) > len(best):
            best = chain
    assert len(best) >= chain_min, "construction: chain too short"
    k8 = oracle.e4m3_encode(rng.standard_normal((n, 64)) * 30.0)
    ks = np.full(n, 1e-3, np.float32)
    slots = rng.permutation(n - 8)[: n_high + len(best)]
    hi_keys = V[order[rng.integers(0, len(V), n_high)]]
    k8[slots[:n_high]] = hi_keys
    ks[slots[:n_high]] = 4.0
    k8[slots[n_high:]] = V[np.array(best)]
    ks[slots[n_high:]] = 1.0
    return q, k8, ks


@pytest.mark.parametrize("seed", [61, 62, 63])
def test_construction_has_the_intended_gaps(seed):
    # a CPU test of the test data itself
    q, k8, ks = near_tie_keys(seed, 40000)
    s = np.sort(oracle.scores(q, None, k8, ks))[::-1]
    gaps = (s[500:530] - s[501:531]) / np.abs(s[500:530])
    assert 1e-5 < gaps.min() and gaps.max() < 7e-5
    dq, dk = oracle.e4m3_value(q), oracle.e4m3_value(k8)
    order = np.argsort(-oracle.scores(q, None, k8, ks))[505:520]
    ratio = np.abs(dk[order][:, None, :] * dq[None]).sum(axis=(1, 2)) / (s[505:520] / ks[order])
    assert ratio.min() > 5.0


@pytest.mark.gpu
@pytest.mark.parametrize("n_q", [1, 2, 4])
def test_near_ties_select_the_oracle_set(csa2, n_q):
    n = 40000
    kinds = []
    for seed in (61, 62, 63):
        q, k8h, ksh = near_tie_keys(seed, n)
        k8 = torch.from_numpy(k8h).cuda()
        ks = torch.from_numpy(ksh).cuda()
        qd = torch.from_numpy(np.broadcast_to(q, (1, n_q, 4, 64)).copy()).cuda()
        ws = csa2.Workspace(1, n_q, n)
        out = csa2.csa2_index_topk(ws, qd, k8, ks, [n], [n - n_q], n)
        torch.cuda.synchronize()
        s = oracle.scores(q, None, k8h, ksh)
        for i in range(n_q):
            nv = n - n_q + i + 1
            ref = oracle.index_flat(q, None, k8h, ksh, nv)
            kinds.append(check_topk(out[0, i].cpu().numpy(), ref, s[:nv], 512, nv, f"seed {seed} q {i}"))
            assert np.array_equal(out[0, i].cpu().numpy(), ref), f"seed {seed} q {i}: not the oracle's set"
    print(n_q, kinds)
