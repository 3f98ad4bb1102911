"""Paged caches on the GPU: the caches as a pool of fixed-size pages with a
page table per sequence (pages placed in a random order).  Every result
must equal, bit for bit, the one the same cache gives laid out contiguously
(whose parity with the oracle the other tests establish), and the indices
are also checked against the oracle here."""

import numpy as np
import pytest
import torch

import csa2_inputs as gen
import oracle
import oracle_side
from parity import check_close, check_topk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_decode_fp4_amd as m
    return m


def _contiguous(csa2, n_entries, stride, seed, dev="cuda"):
    B = len(n_entries)
    nib = torch.zeros((B * stride, 256), dtype=torch.uint8, device=dev)
    sc = torch.zeros((B * stride, 32), dtype=torch.uint8, device=dev)
    k8 = torch.zeros((B * stride, 64), dtype=torch.uint8, device=dev)
    ks = torch.zeros((B * stride,), dtype=torch.float32, device=dev)
    for b, n in enumerate(n_entries):
        if n == 0:
            continue
        x = gen.latent(n, seed, seq=b, device=dev)
        k = gen.index_key(n, seed, seq=b, device=dev)
        e0 = b * stride
        csa2.csa2_quantize_kv(x, k_in=k, out=[nib[e0:e0 + n], sc[e0:e0 + n], k8[e0:e0 + n], ks[e0:e0 + n]])
    return nib, sc, k8, ks


def _paginate(csa2, arrays, n_entries, stride, page, seed, extra_pages=3):
    """The contiguous caches scattered over a pool, page by page in a random
    order (plus unused pages); returns the pools and the page table."""
    rng = np.random.default_rng(seed)
    B = len(n_entries)
    table_stride = max(1, max((stride + page - 1) // page, 1))
    n_pages = B * table_stride + extra_pages
    order = rng.permutation(n_pages)
    table = np.zeros((B, table_stride), dtype=np.int32)
    pools = [torch.zeros((n_pages * page,) + a.shape[1:], dtype=a.dtype, device=a.device) for a in arrays]
    i = 0
    for b in range(B):
        for j in range(table_stride):
            pg = int(order[i]); i += 1
            table[b, j] = pg
            lo, hi = j * page, min((j + 1) * page, stride)
            if lo >= hi:
                continue
            for a, pool in zip(arrays, pools):
                pool[pg * page: pg * page + (hi - lo)] = a[b * stride + lo: b * stride + hi]
    t = torch.from_numpy(table).to(arrays[0].device)
    return pools, csa2.make_pages(t, page, n_pages * page), t


@pytest.mark.parametrize("n_q,page", [(1, 256), (4, 128)])
def test_paged_index_matches_contiguous(csa2, n_q, page):
    seed = 71 + n_q
    n_entries = [9000, 40000, 1500]  # the last row is short: every key is a candidate
    stride = 40000
    nib, sc, k8, ks = _contiguous(csa2, n_entries, stride, seed)
    (pk8, pks), pages, _ = _paginate(csa2, [k8, ks], n_entries, stride, page, seed)
    q = gen.index_query((3, n_q), seed, device="cuda")
    q_pos0 = [n - n_q for n in n_entries]
    ws = csa2.Workspace(3, n_q, stride)
    ref = csa2.csa2_index_topk(ws, q, k8, ks, n_entries, q_pos0, stride)
    got = csa2.csa2_index_topk(ws, q, pk8, pks, n_entries, q_pos0, 0, pages=pages)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert ws.fallbacks() == 0
    qh, gh = q.cpu().numpy(), got.cpu().numpy()
    for b, n in enumerate(n_entries):
        e0 = b * stride
        k8h, ksh = oracle_side.keys(gen.index_key(n, seed, seq=b, device="cuda"), k8[e0:e0 + n], ks[e0:e0 + n])
        for i in range(n_q):
            vis = min(n, q_pos0[b] + i + 1)
            r = oracle.index_flat(qh[b, i], None, k8h, ksh, vis)
            check_topk(gh[b, i], r, oracle.scores(qh[b, i], None, k8h[:vis], ksh[:vis]), 512, vis,
                       f"seq {b} q{i}")


@pytest.mark.parametrize("n_q", [1, 3])
def test_paged_attention_matches_contiguous(csa2, n_q):
    """n_q 1 takes the tile form, 3 the walk form."""
    seed, B, stride, page = 29 + n_q, 2, 6000, 512
    n_entries = [6000, 4100]
    nib, sc, k8, ks = _contiguous(csa2, n_entries, stride, seed)
    (pnib, psc), pages, _ = _paginate(csa2, [nib, sc], n_entries, stride, page, seed)
    rng = np.random.default_rng(seed)
    idx = np.stack([np.stack([np.sort(rng.choice(n_entries[b], 512, replace=False)) for _ in range(n_q)])
                    for b in range(B)]).astype(np.int32)
    idx[1, 0, -5:] = -1  # a few empty slots
    idx_d = torch.from_numpy(idx).cuda()
    q_pos0 = [n - n_q for n in n_entries]
    swa_pos0 = [p - 127 for p in q_pos0]
    q = gen.attn_query((B, n_q), seed, device="cuda")
    swa = gen.window_rows(B, 127 + n_q, seed, device="cuda")
    ws = csa2.Workspace(B, n_q, stride)
    ref = csa2.csa2_sparse_swa_attn(ws, q, nib, sc, idx_d, swa, q_pos0, swa_pos0, stride)
    got = csa2.csa2_sparse_swa_attn(ws, q, pnib, psc, idx_d, swa, q_pos0, swa_pos0, 0, pages=pages)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    nh, sh = oracle_side.fp4(gen.latent(n_entries[0], seed, seq=0, device="cuda"), nib[:n_entries[0]], sc[:n_entries[0]])
    r = oracle.sparse_swa_attention(gen.bf16_bits(q[0, 0]), nh, sh, idx[0, 0],
                                    gen.bf16_bits(swa[0]), swa_pos0[0], q_pos0[0])
    check_close(got[0, 0].cpu().numpy(), r, "b0 q0")


def test_paged_group_matches_contiguous(csa2):
    """Full + 3 Reuse, then Reindex + 3 Reuse, at batch 4 (the decode group's
    window tiles run in the select launch)."""
    seed, B, stride, page = 53, 4, 20000, 1024
    n_entries = [20000, 17000, 9000, 12345]
    nib, sc, k8, ks = _contiguous(csa2, n_entries, stride, seed)
    pools, pages, _ = _paginate(csa2, [nib, sc, k8, ks], n_entries, stride, page, seed)
    kv_c = csa2.make_kv(nib, sc, k8, ks, stride)
    kv_p = csa2.make_kv(*pools, 0, pages=pages)
    q_pos0 = [n - 1 for n in n_entries]
    swa_pos0 = [p - 127 for p in q_pos0]

    def plan(kv, first):
        ls = []
        for j, m in enumerate([first] + [csa2.MODE_REUSE] * 3):
            d = dict(mode=m, q=gen.attn_query((B, 1), seed + (first == csa2.MODE_REINDEX), j, device="cuda"),
                     swa=gen.window_rows(B, 128, seed, j, device="cuda"))
            if m != csa2.MODE_REUSE:
                d["idx_q"] = gen.index_query((B, 1), seed + (first == csa2.MODE_REINDEX), j, device="cuda")
            if m == csa2.MODE_FULL:
                d["kv"] = kv
            ls.append(d)
        return ls

    res = []
    for kv in (kv_c, kv_p):
        ws, st = csa2.Workspace(B, 1, stride), csa2.State(B, 1)
        o1 = csa2.csa2_run_group(ws, st, plan(kv, csa2.MODE_FULL), q_pos0, n_entries, swa_pos0)
        i1 = st.indices.clone()
        o2 = csa2.csa2_run_group(ws, st, plan(kv, csa2.MODE_REINDEX), q_pos0, n_entries, swa_pos0)
        torch.cuda.synchronize()
        assert ws.fallbacks() == 0
        res.append((o1, i1, o2, st.indices.clone()))
    (a1, ai1, a2, ai2), (b1, bi1, b2, bi2) = res
    assert torch.equal(ai1, bi1) and torch.equal(ai2, bi2)
    for x, y in zip(a1 + a2, b1 + b2):
        assert torch.equal(x, y)


@pytest.mark.parametrize("ratio", [1, 2])
def test_paged_append_matches_contiguous(csa2, ratio):
    """Decode steps appended into a paged pool leave every page holding the
    bytes the contiguous cache holds for it (block keys stay per sequence)."""
    seed, B, page, steps = 61 + ratio, 3, 128, 300
    prefix = [0, 40, 200]
    n_tok = [p + steps for p in prefix]
    stride = max(n_tok) // ratio + 8
    bst = (stride + 7) // 8
    xs = [gen.latent(n, seed, seq=b, device="cuda") for b, n in enumerate(n_tok)]
    kk = [gen.index_key(n, seed, seq=b, device="cuda") for b, n in enumerate(n_tok)]

    def run(paged):
        nib = torch.zeros((B * stride, 256), dtype=torch.uint8, device="cuda")
        sc = torch.zeros((B * stride, 32), dtype=torch.uint8, device="cuda")
        k8 = torch.zeros((B * stride, 64), dtype=torch.uint8, device="cuda")
        ks = torch.zeros((B * stride,), dtype=torch.float32, device="cuda")
        bk8 = torch.zeros((B * bst, 64), dtype=torch.uint8, device="cuda")
        bks = torch.zeros((B * bst,), dtype=torch.float32, device="cuda")
        pend = torch.zeros((B, 576), dtype=torch.float32, device="cuda")
        for b, p in enumerate(prefix):
            if p:
                e0, e1 = b * stride, b * stride + p // ratio
                csa2.csa2_quantize_kv(xs[b][:p].contiguous(), ratio=ratio, k_in=kk[b][:p].contiguous(),
                                      out=[nib[e0:e1], sc[e0:e1], k8[e0:e1], ks[e0:e1]])
        csa2.csa2_build_block_keys(k8, ks, [p // ratio for p in prefix], stride, bk8, bks, bst)
        arrays, pages, table = [nib, sc, k8, ks], None, None
        if paged:
            arrays, pages, table = _paginate(csa2, [nib, sc, k8, ks], [stride] * B, stride, page, seed)
        for t in range(steps):
            pos = [p + t for p in prefix]
            x = torch.stack([xs[b][pos[b]] for b in range(B)]).contiguous()
            k = torch.stack([kk[b][pos[b]] for b in range(B)]).contiguous()
            csa2.csa2_append(x, k, pos, *arrays, stride if not paged else 0, ratio=ratio, bk8=bk8, bkscale=bks,
                             bk_stride=bst, pending=pend, pages=pages)
        torch.cuda.synchronize()
        return arrays, table, bk8, bks

    (cn, cs, ck, cks), _, cbk, cbks = run(False)
    (pn, ps, pk, pks), table, pbk, pbks = run(True)
    assert torch.equal(cbk, pbk) and torch.equal(cbks, pbks)
    tab = table.cpu().numpy()
    for b in range(B):
        for j in range(tab.shape[1]):
            lo, hi = j * page, min((j + 1) * page, stride)
            if lo >= hi:
                continue
            pg = int(tab[b, j])
            for c, p in ((cn, pn), (cs, ps), (ck, pk)):
                assert torch.equal(c[b * stride + lo: b * stride + hi], p[pg * page: pg * page + hi - lo]), (b, j)
            assert torch.equal(cks[b * stride + lo: b * stride + hi].view(torch.int32),
                               pks[pg * page: pg * page + hi - lo].view(torch.int32)), (b, j)


def test_paged_decode_steps_match_oracle(csa2):
    """Three decode steps on a paged pool with window rings, ratio 2: append
    each new token (cache pages, window ring), then a Full + Reuse group; the
    last step's indices and outputs match the oracle over the token history,
    and equal those of the same steps on a contiguous cache."""
    dev, B, ratio, page, ring, seed = "cuda", 2, 2, 128, 128, 83
    prefix, steps = 5000, 4                      # even prefix: whole pairs
    n_tok = prefix + steps
    stride = n_tok // ratio + 8
    xs = [gen.latent(n_tok, seed, seq=b, device=dev) for b in range(B)]
    kk = [gen.index_key(n_tok, seed, seq=b, device=dev) for b in range(B)]

    def run(paged):
        nib = torch.zeros((B * stride, 256), dtype=torch.uint8, device=dev)
        sc = torch.zeros((B * stride, 32), dtype=torch.uint8, device=dev)
        k8 = torch.zeros((B * stride, 64), dtype=torch.uint8, device=dev)
        ks = torch.zeros((B * stride,), dtype=torch.float32, device=dev)
        pend = torch.zeros((B, 576), dtype=torch.float32, device=dev)
        swa = [torch.zeros((B, ring, 512), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        for b in range(B):
            e0 = b * stride
            csa2.csa2_quantize_kv(xs[b][:prefix].contiguous(), ratio=ratio, k_in=kk[b][:prefix].contiguous(),
                                  out=[nib[e0:e0 + prefix // ratio], sc[e0:e0 + prefix // ratio],
                                       k8[e0:e0 + prefix // ratio], ks[e0:e0 + prefix // ratio]])
            for L in range(2):
                for tok in range(prefix - ring, prefix):
                    swa[L][b, tok % ring] = xs[b][tok].to(torch.bfloat16)
        arrays, pages = [nib, sc, k8, ks], None
        if paged:
            arrays, pages, _ = _paginate(csa2, arrays, [stride] * B, stride, page, seed)
        kv = csa2.make_kv(*arrays, 0 if paged else stride, pages=pages)
        ws, st = csa2.Workspace(B, 1, stride), csa2.State(B, 1)
        for t in range(steps):
            pos = prefix + t
            x = torch.stack([xs[b][pos] for b in range(B)]).contiguous()
            k = torch.stack([kk[b][pos] for b in range(B)]).contiguous()
            for L in range(2):
                csa2.csa2_append(x, k, [pos] * B, *arrays, 0 if paged else stride, ratio=ratio,
                                 pending=pend if L == 0 else pend.clone(), swa=swa[L], swa_ring=ring, pages=pages)
            layers = [dict(mode=csa2.MODE_FULL, q=gen.attn_query((B, 1), seed + t, 0, device=dev), swa=swa[0],
                           idx_q=gen.index_query((B, 1), seed + t, 0, device=dev), kv=kv),
                      dict(mode=csa2.MODE_REUSE, q=gen.attn_query((B, 1), seed + t, 1, device=dev), swa=swa[1])]
            n_ent = (pos + 1) // ratio
            outs = csa2.csa2_run_group(ws, st, layers, [pos] * B, [n_ent] * B, None, ratio=ratio, swa_ring=ring)
        torch.cuda.synchronize()
        assert ws.fallbacks() == 0
        return outs, st.indices.clone(), layers

    outs_c, idx_c, _ = run(False)
    outs_p, idx_p, layers = run(True)
    assert torch.equal(idx_c, idx_p)
    for a, b in zip(outs_c, outs_p):
        assert torch.equal(a, b)
    pos = prefix + steps - 1
    n_ent = (pos + 1) // ratio
    idx = idx_p.cpu().numpy()
    for b in range(B):
        xh, kh = xs[b][:2 * n_ent].cpu().numpy(), kk[b][:2 * n_ent].cpu().numpy()
        rn, rs, rk, rks = oracle.quantize_kv(xh, ratio, kh)
        iq = layers[0]["idx_q"][b, 0].cpu().numpy()
        ref = oracle.index_flat(iq, None, rk, rks, n_ent)
        check_topk(idx[b, 0], ref, oracle.scores(iq, None, rk, rks), 512, n_ent, f"seq {b}")
        win = gen.bf16_bits(xs[b][pos - 127: pos + 1].to(torch.bfloat16))
        for j, L in enumerate(layers):  # on the GPU's own index set
            r = oracle.sparse_swa_attention(gen.bf16_bits(L["q"][b, 0]), rn, rs, idx[b, 0], win, pos - 127, pos)
            check_close(outs_p[j][b, 0].cpu().numpy(), r, f"seq {b} layer {j}")


def test_paged_multi_token_group_matches_contiguous(csa2):
    """Four query tokens per sequence (shared scan, walk-form attention) on a
    paged pool: Full + 3 Reuse equals the contiguous run."""
    seed, B, n_q, stride, page = 97, 3, 4, 12000, 256
    n_entries = [12000, 7000, 300]
    nib, sc, k8, ks = _contiguous(csa2, n_entries, stride, seed)
    pools, pages, _ = _paginate(csa2, [nib, sc, k8, ks], n_entries, stride, page, seed)
    q_pos0 = [max(n - n_q, 0) for n in n_entries]
    swa_pos0 = [max(p - 127, 0) for p in q_pos0]
    res = []
    for kv in (csa2.make_kv(nib, sc, k8, ks, stride), csa2.make_kv(*pools, 0, pages=pages)):
        ls = []
        for j, m in enumerate([csa2.MODE_FULL] + [csa2.MODE_REUSE] * 3):
            d = dict(mode=m, q=gen.attn_query((B, n_q), seed, j, device="cuda"),
                     swa=gen.window_rows(B, 127 + n_q, seed, j, device="cuda"))
            if m == csa2.MODE_FULL:
                d["idx_q"], d["kv"] = gen.index_query((B, n_q), seed, j, device="cuda"), kv
            ls.append(d)
        ws, st = csa2.Workspace(B, n_q, stride), csa2.State(B, n_q)
        outs = csa2.csa2_run_group(ws, st, ls, q_pos0, n_entries, swa_pos0)
        torch.cuda.synchronize()
        assert ws.fallbacks() == 0
        res.append((outs, st.indices.clone()))
    (oc, ic), (op, ip) = res
    assert torch.equal(ic, ip)
    for a, b in zip(oc, op):
        assert torch.equal(a, b)
