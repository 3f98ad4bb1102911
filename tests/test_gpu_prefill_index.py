"""GPU parity of the prefill-chunk indexer (fp8 MFMA scoring, sampled
threshold, exact selection) against the oracle, including the exact
recompute taken when the sampled threshold cannot bound a row."""

import numpy as np
import pytest
import torch

import csa2_inputs as gen
import oracle
import oracle_side
from parity import check_topk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_decode_fp4_amd as m
    return m


def _keys(csa2, k_f32):
    """GPU keys of fp32 draws, and the oracle's codes of the same draws."""
    n = k_f32.shape[0]
    x = torch.zeros((n, 512), dtype=torch.float32, device="cuda")
    _, _, k8, ks = csa2.csa2_quantize_kv(x, k_in=k_f32)
    _keys.oracle_codes = oracle_side.keys(k_f32, k8, ks)
    return k8, ks


def _check_rows(out, q, w, k8h, ksh, n_entries, q_pos0, ratio, k, stride, rows=None):
    kinds = []
    B, n_q = q.shape[0], q.shape[1]
    for b in range(B):
        for i in (range(n_q) if rows is None else rows):
            nv = min(n_entries[b], oracle.visible_entries(q_pos0[b] + i, ratio))
            wi = None if w is None else w[b, i]
            kb, sb = k8h[b * stride: b * stride + nv], ksh[b * stride: b * stride + nv]
            ref = oracle.index_flat(q[b, i], wi, kb, sb, nv, k)
            sc = oracle.scores(q[b, i], wi, kb, sb)
            kinds.append(check_topk(out[b, i], ref, sc, k, nv, f"seq {b} query {i}"))
    return kinds


@pytest.mark.parametrize("B,n_entries,n_q,ratio,with_w,k", [
    (1, [20000], 300, 1, False, 512),       # ratio 1, queries at the end of the context
    (2, [9000, 14000], 64, 1, True, 512),   # two sequences, head weights
    (1, [5000], 257, 2, False, 512),        # ratio 2, a partial second row tile
    (1, [3000], 40, 1, False, 2048),        # large k
])
def test_prefill_index_matches_oracle(csa2, B, n_entries, n_q, ratio, with_w, k):
    stride = max(n_entries)
    kf = gen.index_key(B * stride, 17, device="cuda")
    k8, ks = _keys(csa2, kf)
    q = gen.index_query((B, n_q), 17, device="cuda")
    w = torch.rand((B, n_q, 4), device="cuda", generator=torch.Generator("cuda").manual_seed(5)) if with_w else None
    q_pos0 = [ratio * n - n_q for n in n_entries]
    ws = csa2.Workspace(B, n_q, stride)
    out = csa2.csa2_index_topk(ws, q, k8, ks, n_entries, q_pos0, stride, ratio=ratio, idx_w=w, k=k)
    torch.cuda.synchronize()
    kinds = _check_rows(out.cpu().numpy(), q.cpu().numpy(), None if w is None else w.cpu().numpy(),
                        *_keys.oracle_codes, n_entries, q_pos0, ratio, k, stride)
    assert kinds.count("exact") >= 0.9 * len(kinds)
    out2 = csa2.csa2_index_topk(ws, q, k8, ks, n_entries, q_pos0, stride, ratio=ratio, idx_w=w, k=k)
    assert torch.equal(out, out2)


def test_prefill_equal_scores_take_the_exact_recompute(csa2):
    # a zero query scores every key 0: the sampled threshold admits every key,
    # the list overflows, and the row is recomputed exactly
    n = 12000
    k8, ks = _keys(csa2, gen.index_key(n, 3, device="cuda"))
    q = torch.zeros((1, 40, 4, 64), dtype=torch.uint8, device="cuda")
    ws = csa2.Workspace(1, 40, n)
    out = csa2.csa2_index_topk(ws, q, k8, ks, [n], [n + 100], n)
    assert np.array_equal(out.cpu().numpy()[0], np.tile(np.arange(512), (40, 1)))


def test_prefill_misleading_sample_takes_the_exact_recompute(csa2):
    # every sampled key scores far above the rest, so the sampled threshold
    # admits fewer than k keys and the rows are recomputed exactly
    n = 20000
    kf = gen.index_key(n, 8, device="cuda")
    sampled = torch.arange(2048, device="cuda") * n // 2048
    kf[sampled] *= 1000.0
    k8, ks = _keys(csa2, kf)
    q = gen.index_query((1, 48), 8, device="cuda")
    ws = csa2.Workspace(1, 48, n)
    out = csa2.csa2_index_topk(ws, q, k8, ks, [n], [n + 500], n)
    torch.cuda.synchronize()
    _check_rows(out.cpu().numpy(), q.cpu().numpy(), None, *_keys.oracle_codes, [n],
                [n + 500], 1, 512, n, rows=[0, 1, 47])
