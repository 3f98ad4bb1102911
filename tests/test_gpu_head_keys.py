"""GPU parity of the per-head 4 x 64 indexer-key layout (key_heads = 4)
against the oracle: the encoder bit for bit, flat / flat-pool / pool top-k
tie-aware for every row, near-ties settled exactly, and a group plan."""

import numpy as np
import pytest
import torch

import csa2_inputs as gen
import oracle
from parity import check_close, check_flat_pool, check_topk
from test_gpu_near_ties import near_tie_keys

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_decode_fp4_amd as m
    return m


def _head_keys(csa2, seed, n_tok, ratio=1):
    """GPU per-head keys of N(0,1) draws (with one all-zero token pair), and
    the oracle's codes of the same draws, checked equal bit for bit."""
    k = gen.normal((n_tok, 4, 64), seed, "idxk4", device="cuda")
    k[ratio * 3: ratio * 4] = 0.0
    k[ratio * 5] *= 40.0                                  # one head sets the shared scale
    k8, ks = csa2.csa2_quantize_head_keys(k, ratio=ratio)
    torch.cuda.synchronize()
    kh = k.cpu().numpy()
    e = oracle.compress_pairs(kh.reshape(n_tok, -1), ratio).reshape(-1, 4, 64)
    rk8, rks = oracle.index_key_encode_heads(e)
    assert np.array_equal(k8.cpu().numpy(), rk8), "per-head key codes"
    assert np.array_equal(ks.cpu().numpy().view(np.uint32), rks.view(np.uint32)), "per-head key scales"
    return k8, ks, rk8, rks


@pytest.mark.parametrize("ratio", [1, 2])
def test_head_key_encoder_is_bit_exact(csa2, ratio):
    _head_keys(csa2, 3, 6002, ratio)


@pytest.mark.parametrize("n_entries,n_q,ratio", [
    ([5000, 700, 4097], 1, 1),      # ragged batch, tail chunks
    ([20000], 3, 1),                # several queries per sequence (one scan each)
    ([3001], 2, 2),                 # ratio-2 visibility
])
def test_head_keys_flat_topk(csa2, n_entries, n_q, ratio):
    batch, stride = len(n_entries), max(n_entries)
    k8, ks, rk8, rks = _head_keys(csa2, 5, batch * stride)
    q = gen.index_query((batch, n_q), 21, device="cuda")
    ws = csa2.Workspace(batch, n_q, stride)
    q_pos0 = [ratio * n - n_q for n in n_entries]
    out = csa2.csa2_index_topk(ws, q, k8, ks, n_entries, q_pos0, stride, ratio=ratio, key_heads=4)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    for b, n in enumerate(n_entries):
        kb, sb = rk8[b * stride: b * stride + n], rks[b * stride: b * stride + n]
        for i in range(n_q):
            nv = min(n, oracle.visible_entries(q_pos0[b] + i, ratio))
            ref = oracle.index_flat(qh[b, i], None, kb, sb, nv)
            check_topk(out[b, i].cpu().numpy(), ref, oracle.scores(qh[b, i], None, kb[:nv], sb[:nv]), 512, nv,
                       f"b{b} q{i}")
    assert ws.fallbacks() == 0


def test_head_keys_flat_pool_and_pool(csa2):
    n_entries, stride = [40000, 9000], 40000
    k8, ks, rk8, rks = _head_keys(csa2, 7, 2 * stride)
    q = gen.index_query((2, 1), 23, device="cuda")
    ws = csa2.Workspace(2, 1, stride)
    out, pool = csa2.csa2_index_topk(ws, q, k8, ks, n_entries, [n - 1 for n in n_entries], stride,
                                     kind=csa2.INDEX_FLAT_POOL, want_pool=True, key_heads=4)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    for b, n in enumerate(n_entries):
        kb, sb = rk8[b * stride: b * stride + n], rks[b * stride: b * stride + n]
        check_flat_pool(out[b, 0].cpu().numpy(), pool[b, 0].cpu().numpy(), qh[b, 0], None, kb, sb, n, what=f"b{b}")
    # POOL over random candidates
    rng = np.random.default_rng(2)
    cand = np.full((2, 1, 3000), -1, np.int32)
    cand[0, 0, :2600] = np.sort(rng.choice(n_entries[0], 2600, replace=False))
    cand[1, 0, :400] = np.sort(rng.choice(n_entries[1], 400, replace=False))
    out = csa2.csa2_index_topk(ws, q, k8, ks, n_entries, [n - 1 for n in n_entries], stride,
                               kind=csa2.INDEX_POOL, cand=torch.from_numpy(cand).cuda(), key_heads=4)
    torch.cuda.synchronize()
    for b, n in enumerate(n_entries):
        kb, sb = rk8[b * stride: b * stride + n], rks[b * stride: b * stride + n]
        c = cand[b, 0][cand[b, 0] >= 0]
        ref = oracle.index_pool(qh[b, 0], None, kb, sb, c)
        sc = dict(zip(c.tolist(), oracle.scores(qh[b, 0], None, kb[c], sb[c]).tolist()))
        check_topk(out[b, 0].cpu().numpy(), ref, sc, 512, len(c), f"pool b{b}")
    assert ws.fallbacks() == 0


@pytest.mark.parametrize("seed", [61, 62])
def test_head_keys_near_ties_select_the_oracle_set(csa2, seed):
    """The near-tie keys of test_gpu_near_ties with each head's key a
    different channel permutation of the shared key (and each head's query
    permuted alike): the exact scores are those of the shared construction,
    so the 512th / 513th gap is above 1e-5 and the sets must be equal; a
    head reading another head's key would score differently."""
    n = 40000
    q, k8, ks = near_tie_keys(seed, n)
    rng = np.random.default_rng(seed + 100)
    perms = [rng.permutation(64) for _ in range(4)]
    qh = np.ascontiguousarray(np.stack([q[h, perms[h]] for h in range(4)]))
    kh = np.ascontiguousarray(np.stack([k8[:, perms[h]] for h in range(4)], axis=1))  # [n, 4, 64]
    s_shared = oracle.scores(q, None, k8, ks)
    assert np.array_equal(oracle.scores(qh, None, kh, ks), s_shared)
    ref = oracle.index_flat(qh, None, kh, ks, n)
    ws = csa2.Workspace(1, 1, n)
    out = csa2.csa2_index_topk(ws, torch.from_numpy(qh[None, None]).cuda(), torch.from_numpy(kh).cuda(),
                               torch.from_numpy(ks).cuda(), [n], [n - 1], n, key_heads=4)
    torch.cuda.synchronize()
    assert np.array_equal(out[0, 0].cpu().numpy(), ref)
    assert ws.fallbacks() == 0


def test_head_keys_group_plan(csa2):
    """[F, U, U, U] then [R, U, U, U] on a per-head-key cache, against the
    oracle's plan on the same codes (indices tie-aware, every layer's
    attention on the GPU's own index set)."""
    n_entries, stride = [20011, 7000], 20016
    B = len(n_entries)
    x = gen.latent(B * stride, 41, device="cuda")
    nib, sc = csa2.csa2_quantize_kv(x)
    k8, ks, rk8, rks = _head_keys(csa2, 41, B * stride)
    dkv = csa2.make_kv(nib, sc, k8, ks, stride, key_heads=4)
    nh, sh = nib.cpu().numpy(), sc.cpu().numpy()
    hkv = {"nib": [nh[b * stride: b * stride + n] for b, n in enumerate(n_entries)],
           "scale": [sh[b * stride: b * stride + n] for b, n in enumerate(n_entries)],
           "k8": [rk8[b * stride: b * stride + n] for b, n in enumerate(n_entries)],
           "ks": [rks[b * stride: b * stride + n] for b, n in enumerate(n_entries)]}
    q_pos0 = [n - 1 for n in n_entries]
    swa_pos0 = [p - 127 for p in q_pos0]
    ws = csa2.Workspace(B, 1, stride)
    st = csa2.State(B, 1)
    for run, plan in enumerate(["FUUU", "RUUU"]):
        dl = []
        for j, m in enumerate(plan):
            d = dict(mode={"F": csa2.MODE_FULL, "R": csa2.MODE_REINDEX, "U": csa2.MODE_REUSE}[m],
                     q=gen.attn_query((B, 1), 41, 10 * run + j, device="cuda"),
                     swa=gen.window_rows(B, 128, 41, 10 * run + j, device="cuda"))
            if m in "FR":
                d["idx_q"] = gen.index_query((B, 1), 41, 10 * run + j, device="cuda")
            if m == "F":
                d["kv"] = dkv
            dl.append(d)
        outs = csa2.csa2_run_group(ws, st, dl, q_pos0, n_entries, swa_pos0)
        torch.cuda.synchronize()
        gi = st.indices.cpu().numpy()
        iq = dl[0]["idx_q"].cpu().numpy()
        for b, n in enumerate(n_entries):
            ref = oracle.index_flat(iq[b, 0], None, hkv["k8"][b], hkv["ks"][b], n)
            check_topk(gi[b, 0], ref, oracle.scores(iq[b, 0], None, hkv["k8"][b], hkv["ks"][b]), 512, n,
                       f"run {run} seq {b}")
            for j, L in enumerate(dl):
                ref_out = oracle.sparse_swa_attention(gen.bf16_bits(L["q"])[b, 0], hkv["nib"][b], hkv["scale"][b],
                                                      gi[b, 0], gen.bf16_bits(L["swa"])[b], swa_pos0[b], q_pos0[b])
                check_close(outs[j][b, 0].cpu().numpy(), ref_out, f"run {run} layer {j} seq {b}")
    assert ws.fallbacks() == 0


def test_binding_refuses_strided_keys(csa2):
    """A strided key tensor (numpy's stack along axis 1 of fancy-indexed
    arrays makes one) is refused by the binding instead of being read as if
    it were contiguous."""
    strided = torch.zeros((100, 64, 4), dtype=torch.uint8, device="cuda").permute(0, 2, 1)
    assert not strided.is_contiguous()
    ws = csa2.Workspace(1, 1, 100)
    q = torch.zeros((1, 1, 4, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        csa2.csa2_index_topk(ws, q, strided, torch.ones(100, device="cuda"), [100], [99], 100, key_heads=4)
