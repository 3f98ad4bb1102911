"""GPU parity of the indexer + top-k against the oracle (tie-aware rule)."""

import numpy as np
import pytest
import torch

import csa2_inputs as gen
import oracle
import oracle_side
from parity import check_flat_pool, check_hier, check_topk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_decode_fp4_amd as m
    return m


def _keys(csa2, seed, batch, stride):
    """GPU keys of fp32 draws, and the oracle's codes of the same draws."""
    dev = "cuda"
    k = gen.index_key(batch * stride, seed, device=dev)
    x = torch.zeros((batch * stride, 512), dtype=torch.float32, device=dev)
    _, _, k8, ks = csa2.csa2_quantize_kv(x, k_in=k)
    k8h, ksh = oracle_side.keys(k, k8, ks)
    return k8, ks, k8h, ksh


@pytest.mark.parametrize("n_entries,n_q,ratio,k", [
    ([4096], 1, 1, 512),                 # the smallest decode workload
    ([5000, 700, 4097, 513], 1, 1, 512),  # ragged batch, several scan tiles, tail chunks
    ([20000, 9000], 1, 1, 2048),         # large k
    ([300], 1, 1, 512),                  # fewer entries than k: all of them, -1 padded
    ([3000], 7, 2, 512),                 # several queries per sequence, ratio-2 visibility
    ([9000, 5000], 2, 1, 512),           # two queries share each scan workgroup
    ([40000], 4, 1, 512),                # four queries share each scan workgroup
    ([20000, 12000], 6, 2, 512),         # a full and a partial group of four, ratio 2
    ([1], 1, 1, 5),
])
def test_flat_topk(csa2, n_entries, n_q, ratio, k):
    batch = len(n_entries)
    stride = max(n_entries)
    k8, ks, k8h, ksh = _keys(csa2, 100 + stride, batch, stride)
    q = gen.index_query((batch, n_q), 5 + n_q, device="cuda")
    w = None
    if n_q > 1:
        w = torch.rand((batch, n_q, 4), device="cuda", generator=torch.Generator("cuda").manual_seed(3))
    q_pos0 = [ratio * n - n_q for n in n_entries] if ratio == 2 else [n - 1 for n in n_entries]
    ws = csa2.Workspace(batch, n_q, stride)
    out = csa2.csa2_index_topk(ws, q, k8, ks, n_entries, q_pos0, stride, ratio=ratio, idx_w=w, k=k)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    wh = None if w is None else w.cpu().numpy()
    kinds = []
    for b, n in enumerate(n_entries):
        for i in range(n_q):
            nv = oracle.visible_entries(q_pos0[b] + i, ratio)
            nv = min(nv, n)
            wi = None if wh is None else wh[b, i]
            ref = oracle.index_flat(qh[b, i], wi, k8h[b * stride:], ksh[b * stride:], nv, k)
            sc = oracle.scores(qh[b, i], wi, k8h[b * stride: b * stride + nv], ksh[b * stride: b * stride + nv])
            kinds.append(check_topk(out[b, i].cpu().numpy(), ref, sc, k, nv, f"b{b} q{i}"))
    # workspace left clean: a second call gives the same answer
    out2 = csa2.csa2_index_topk(ws, q, k8, ks, n_entries, q_pos0, stride, ratio=ratio, idx_w=w, k=k)
    assert torch.equal(out, out2)
    # random keys: every row's candidate list holds its answer (no exact recompute)
    assert ws.fallbacks() == 0


def test_zero_query_picks_first_positions(csa2):
    k8, ks, _, _ = _keys(csa2, 9, 1, 5000)
    q = torch.zeros((1, 1, 4, 64), dtype=torch.uint8, device="cuda")
    ws = csa2.Workspace(1, 1, 5000)
    out = csa2.csa2_index_topk(ws, q, k8, ks, [5000], [4999], 5000)
    assert np.array_equal(out[0, 0].cpu().numpy(), np.arange(512))
    # every score is 0: all 5,000 keys reach the threshold, the segments
    # overflow and the row is recomputed exactly (this covers that path)
    assert ws.fallbacks() == 1


def test_equal_scores_tie_to_lower_position(csa2):
    # every key identical: all scores equal, the lowest 512 positions win
    dev = "cuda"
    k = gen.index_key(1, 4, device=dev).repeat(3000, 1)
    x = torch.zeros((3000, 512), dtype=torch.float32, device=dev)
    _, _, k8, ks = csa2.csa2_quantize_kv(x, k_in=k)
    q = gen.index_query((1, 1), 4, device=dev)
    ws = csa2.Workspace(1, 1, 3000)
    out = csa2.csa2_index_topk(ws, q, k8, ks, [3000], [2999], 3000)
    assert np.array_equal(out[0, 0].cpu().numpy(), np.arange(512))


@pytest.mark.parametrize("n_entries", [[40000, 30001], [12000]])
def test_hierarchical_topk(csa2, n_entries):
    batch = len(n_entries)
    stride = max(n_entries)
    k8, ks, k8h, ksh = _keys(csa2, 77, batch, stride)
    bk8, bks = csa2.csa2_build_block_keys(k8, ks, n_entries, stride)
    bst = (stride + 7) // 8
    q = gen.index_query((batch, 1), 13, device="cuda")
    ws = csa2.Workspace(batch, 1, stride)
    out, pool = csa2.csa2_index_topk(ws, q, k8, ks, n_entries, [n - 1 for n in n_entries], stride,
                                     kind=csa2.INDEX_HIER, bk8=bk8, bkscale=bks, bk_stride=bst,
                                     want_pool=True)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    bk8h, bksh = oracle_side.block_keys(k8h, ksh, n_entries, stride, bk8, bks)
    for b, n in enumerate(n_entries):
        kb, sb = k8h[b * stride: b * stride + n], ksh[b * stride: b * stride + n]
        bkb, bsb = bk8h[b * bst: b * bst + (n + 7) // 8], bksh[b * bst: b * bst + (n + 7) // 8]
        ref_idx, ref_pool = oracle.index_hier(qh[b, 0], None, kb, sb, bkb, bsb, n)
        gpool = pool[b, 0].cpu().numpy()
        kinds = check_hier(out[b, 0].cpu().numpy(), gpool, qh[b, 0], None, kb, sb, bkb, bsb, n, what=f"b{b}")
        if kinds[0] == "exact":
            assert np.array_equal(gpool, ref_pool)
        if n <= 16384:
            flat = oracle.index_flat(qh[b, 0], None, kb, sb, n)
            assert np.array_equal(ref_idx, flat)
    assert ws.fallbacks() == 0


@pytest.mark.parametrize("n_entries,n_q", [
    ([20000, 9000, 16500], 1),   # 2,500 blocks (a strict subset kept), and rows that keep every block
    ([40000], 2),                # two queries share each scan workgroup (fp8 MFMA scores)
    ([131072, 70001], 4),        # four queries, 16,384 blocks of 8 at the longest row
])
def test_flat_pool_topk(csa2, n_entries, n_q):
    """FLAT_POOL: the flat indices, and the pool of the blocks whose largest
    token score ranks highest, against the oracle for every row."""
    batch = len(n_entries)
    stride = max(n_entries)
    k8, ks, k8h, ksh = _keys(csa2, 91, batch, stride)
    q = gen.index_query((batch, n_q), 17, device="cuda")
    ws = csa2.Workspace(batch, n_q, stride)
    q_pos0 = [n - n_q for n in n_entries]
    out, pool = csa2.csa2_index_topk(ws, q, k8, ks, n_entries, q_pos0, stride, kind=csa2.INDEX_FLAT_POOL,
                                     want_pool=True)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    for b, n in enumerate(n_entries):
        kb, sb = k8h[b * stride: b * stride + n], ksh[b * stride: b * stride + n]
        for i in range(n_q):
            n_vis = min(n, q_pos0[b] + i + 1)
            gpool = pool[b, i].cpu().numpy()
            kinds = check_flat_pool(out[b, i].cpu().numpy(), gpool, qh[b, i], None, kb, sb, n_vis,
                                    what=f"b{b} q{i}")
            if kinds[0] == "exact":
                _, ref_pool = oracle.index_flat_pool(qh[b, i], None, kb, sb, n_vis)
                assert np.array_equal(gpool, ref_pool)
            if -(-n_vis // 8) <= 2048:  # every block kept: the pool is every visible position
                assert np.array_equal(gpool[:n_vis], np.arange(n_vis)) and np.all(gpool[n_vis:] == -1)
    assert ws.fallbacks() == 0


def test_pool_topk(csa2):
    stride = 9000
    k8, ks, k8h, ksh = _keys(csa2, 5, 2, stride)
    rng = np.random.default_rng(1)
    cand = np.full((2, 1, 3000), -1, np.int32)
    cand[0, 0, :2500] = np.sort(rng.choice(stride, 2500, replace=False))
    cand[1, 0, :300] = np.sort(rng.choice(stride, 300, replace=False))
    q = gen.index_query((2, 1), 8, device="cuda")
    ws = csa2.Workspace(2, 1, stride)
    out = csa2.csa2_index_topk(ws, q, k8, ks, [stride, stride], [stride - 1] * 2, stride,
                               kind=csa2.INDEX_POOL, cand=torch.from_numpy(cand).cuda())
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    for b in range(2):
        c = cand[b, 0]
        c = c[c >= 0]
        ref = oracle.index_pool(qh[b, 0], None, k8h[b * stride:], ksh[b * stride:], c)
        sc = dict(zip(c.tolist(), oracle.scores(qh[b, 0], None, k8h[b * stride + c], ksh[b * stride + c]).tolist()))
        check_topk(out[b, 0].cpu().numpy(), ref, sc, 512, len(c), f"b{b}")
