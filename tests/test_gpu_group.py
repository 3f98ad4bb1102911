"""GPU parity of the Full / Reindex / Reuse plan (csa2_run_group)."""

import numpy as np
import pytest
import torch

import csa2_inputs as gen
import oracle
from parity import check_close, check_flat_pool, check_hier, check_topk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_decode_fp4_amd as m
    return m


def _kv(csa2, seed, n_entries, stride, hier):
    """The GPU cache of fp32 draws, and the oracle's own encoding of the same
    draws (checked equal to the GPU's bit for bit, so the oracle's inputs are
    its own)."""
    dev = "cuda"
    B = len(n_entries)
    x = gen.latent(B * stride, seed, device=dev)
    k = gen.index_key(B * stride, seed, device=dev)
    nib, sc, k8, ks = csa2.csa2_quantize_kv(x, k_in=k)
    bk8 = bks = None
    bst = 0
    if hier:
        bst = (stride + 7) // 8
        bk8, bks = csa2.csa2_build_block_keys(k8, ks, n_entries, stride)
    dkv = csa2.make_kv(nib, sc, k8, ks, stride, bk8, bks, bst)
    hkv = {"nib": [], "scale": [], "k8": [], "ks": [], "bk8": [], "bks": []}
    xh, kh = x.cpu().numpy(), k.cpu().numpy()
    g = [t.cpu().numpy() for t in (nib, sc, k8, ks)]
    for b, n in enumerate(n_entries):
        sl = slice(b * stride, b * stride + n)
        rn, rs, rk, rks = oracle.quantize_kv(xh[sl], 1, kh[sl])
        for name, arr, gpu in zip(("nib", "scale", "k8", "ks"), (rn, rs, rk, rks), g):
            assert np.array_equal(gpu[sl].view(np.uint8), arr.view(np.uint8)), f"seq {b}: {name}"
            hkv[name].append(arr)
        if hier:
            rbk, rbks = oracle.block_keys(rk, rks)
            nb = (n + 7) // 8
            assert np.array_equal(bk8[b * bst: b * bst + nb].cpu().numpy(), rbk), f"seq {b}: block keys"
            hkv["bk8"].append(rbk)
            hkv["bks"].append(rbks)
    return dkv, hkv


def _layers(csa2, seed, plan, B, rows, dkv, hkv, layer0, n_q=1):
    dev_layers, host_layers = [], []
    for j, m in enumerate(plan):
        mode = {"F": csa2.MODE_FULL, "R": csa2.MODE_REINDEX, "U": csa2.MODE_REUSE}[m]
        q = gen.attn_query((B, n_q), seed, layer0 + j, device="cuda")
        swa = gen.window_rows(B, rows, seed, layer0 + j, device="cuda")
        d = dict(mode=mode, q=q, swa=swa)
        h = dict(mode=mode, q=gen.bf16_bits(q), swa=gen.bf16_bits(swa))
        if m in "FR":
            iq = gen.index_query((B, n_q), seed, layer0 + j, device="cuda")
            d["idx_q"], h["idx_q"], h["idx_w"] = iq, iq.cpu().numpy(), None
        if m == "F":
            d["kv"], h["kv"] = dkv, hkv
        dev_layers.append(d)
        host_layers.append(h)
    return dev_layers, host_layers


def _compare(outs, st, hkv, host_layers, n_entries, q_pos0, swa_pos0, plan, kind, reindex_kind="flat"):
    """Indices tie-aware (hierarchical Full rows and pool Reindex rows
    against the oracle's ranking of the GPU's own pool); every layer's
    attention against the oracle on the GPU's own index set."""
    st_idx = st.indices.cpu().numpy()
    gpool = st.pool.cpu().numpy() if st.pool is not None else None
    n_q = st_idx.shape[1]
    last = max(j for j, m in enumerate(plan) if m in "FR")
    L = host_layers[last]
    kinds = []
    for b, n in enumerate(n_entries):
        for i in range(n_q):
            nv = min(n, oracle.visible_entries(q_pos0[b] + i, 1))
            iq = L["idx_q"][b, i]
            if kind == "hier" and plan[last] == "F":
                kinds.append(check_hier(st_idx[b, i], gpool[b, i], iq, None, hkv["k8"][b], hkv["ks"][b],
                                        hkv["bk8"][b], hkv["bks"][b], nv, what=f"seq {b} q {i}"))
            elif kind == "flatpool" and plan[last] == "F":
                kinds.append(check_flat_pool(st_idx[b, i], gpool[b, i], iq, None, hkv["k8"][b], hkv["ks"][b], nv,
                                             what=f"seq {b} q {i}"))
            elif plan[last] == "R" and reindex_kind == "pool":
                pool = gpool[b, i][gpool[b, i] >= 0]
                ref = oracle.index_pool(iq, None, hkv["k8"][b], hkv["ks"][b], pool)
                sc = dict(zip(pool.tolist(), oracle.scores(iq, None, hkv["k8"][b][pool], hkv["ks"][b][pool]).tolist()))
                kinds.append(check_topk(st_idx[b, i], ref, sc, 512, len(pool), f"seq {b} q {i} pool reindex"))
            else:
                ref = oracle.index_flat(iq, None, hkv["k8"][b], hkv["ks"][b], nv)
                sc = oracle.scores(iq, None, hkv["k8"][b][:nv], hkv["ks"][b][:nv])
                kinds.append(check_topk(st_idx[b, i], ref, sc, 512, nv, f"seq {b} q {i}"))
            for j, H in enumerate(host_layers):
                ref_out = oracle.sparse_swa_attention(H["q"][b, i], hkv["nib"][b], hkv["scale"][b], st_idx[b, i],
                                                      H["swa"][b], swa_pos0[b], q_pos0[b] + i)
                check_close(outs[j][b, i].cpu().numpy(), ref_out, f"layer {j} seq {b} q {i}")
    return kinds


@pytest.mark.parametrize("kind", ["flat", "hier"])
def test_group_full_reuse_then_reindex_reuse(csa2, kind):
    n_entries = [20011, 7000, 513]
    stride = 20016
    B = len(n_entries)
    hier = kind == "hier"
    dkv, hkv = _kv(csa2, 31, n_entries, stride, hier)
    rows = 128
    q_pos0 = [n - 1 for n in n_entries]
    swa_pos0 = [p - 127 for p in q_pos0]
    ws = csa2.Workspace(B, 1, stride)
    st = csa2.State(B, 1, with_pool=hier)
    ik = csa2.INDEX_HIER if hier else csa2.INDEX_FLAT
    for run, plan in enumerate(["FUUU", "RUUU"]):
        dl, hl = _layers(csa2, 31, plan, B, rows, dkv, hkv, 10 * run)
        outs = csa2.csa2_run_group(ws, st, dl, q_pos0, n_entries, swa_pos0, index_kind=ik)
        torch.cuda.synchronize()
        print(plan, _compare(outs, st, hkv, hl, n_entries, q_pos0, swa_pos0, plan, kind))
        # the Reuse layers attended with exactly the state's indices
        solo = csa2.csa2_sparse_swa_attn(ws, dl[2]["q"], dkv._tensors[0], dkv._tensors[1], st.indices,
                                         dl[2]["swa"], q_pos0, swa_pos0, stride)
        assert torch.equal(solo, outs[2])
    assert ws.fallbacks() == 0


def test_hier_full_then_pool_reindex(csa2):
    """[F(hier), U, U, U] then [R(pool), U, U, U]: the Reindex layer ranks only
    the 16,384-position pool the hierarchical Full layer kept, against the
    oracle's plan with reindex_kind "pool" (40,000 and 65,536 entries: 5,000
    and 8,192 blocks, so the 2,048 kept blocks are a strict subset)."""
    n_entries = [40000, 65536]
    stride = 65536
    B = len(n_entries)
    dkv, hkv = _kv(csa2, 37, n_entries, stride, True)
    q_pos0 = [n - 1 for n in n_entries]
    swa_pos0 = [p - 127 for p in q_pos0]
    ws = csa2.Workspace(B, 1, stride)
    st = csa2.State(B, 1, with_pool=True)
    ref_st = oracle.new_state()
    for run, plan in enumerate(["FUUU", "RUUU"]):
        dl, hl = _layers(csa2, 37, plan, B, 128, dkv, hkv, 10 * run)
        outs = csa2.csa2_run_group(ws, st, dl, q_pos0, n_entries, swa_pos0, index_kind=csa2.INDEX_HIER,
                                   reindex_kind=csa2.INDEX_POOL)
        torch.cuda.synchronize()
        kinds = _compare(outs, st, hkv, hl, n_entries, q_pos0, swa_pos0, plan, "hier", "pool")
        print(plan, kinds)
        ref_outs = oracle.run_group(hl, ref_st, q_pos0, n_entries, swa_pos0, kind="hier", reindex_kind="pool")
        gi = st.indices.cpu().numpy()
        for b in range(B):
            # where the block stage had no tie the GPU's pool is the oracle's,
            # and then the whole plan's indices are the oracle's plan's
            if run == 0 and kinds[b][0] == "exact":
                assert np.array_equal(st.pool[b, 0].cpu().numpy(), ref_st["pool"][b][0])
            if np.array_equal(gi[b, 0], ref_st["indices"][b, 0]):
                for j in range(4):
                    check_close(outs[j][b, 0].cpu().numpy(), ref_outs[j][b, 0], f"plan run {run} layer {j} seq {b}")
        # the Reindex indices lie inside the Full layer's pool
        if run == 1:
            for b in range(B):
                pool = set(st.pool[b, 0].cpu().numpy().tolist()) - {-1}
                assert set(gi[b, 0].tolist()) <= pool
    assert ws.fallbacks() == 0


def test_flat_pool_full_then_pool_reindex(csa2):
    """[F(flat pool), U, U, U] then [R(pool), U, U, U]: the Full layer indexes
    flat and keeps the 2,048 blocks its token scores rank highest; the
    Reindex layer ranks only that pool (the oracle's plan with kind
    "flatpool"); 40,000 and 65,536 entries, so the kept blocks are a strict
    subset."""
    n_entries = [40000, 65536]
    stride = 65536
    B = len(n_entries)
    dkv, hkv = _kv(csa2, 39, n_entries, stride, False)
    q_pos0 = [n - 1 for n in n_entries]
    swa_pos0 = [p - 127 for p in q_pos0]
    ws = csa2.Workspace(B, 1, stride)
    st = csa2.State(B, 1, with_pool=True)
    ref_st = oracle.new_state()
    for run, plan in enumerate(["FUUU", "RUUU"]):
        dl, hl = _layers(csa2, 39, plan, B, 128, dkv, hkv, 10 * run)
        outs = csa2.csa2_run_group(ws, st, dl, q_pos0, n_entries, swa_pos0, index_kind=csa2.INDEX_FLAT_POOL,
                                   reindex_kind=csa2.INDEX_POOL)
        torch.cuda.synchronize()
        kinds = _compare(outs, st, hkv, hl, n_entries, q_pos0, swa_pos0, plan, "flatpool", "pool")
        print(plan, kinds)
        ref_outs = oracle.run_group(hl, ref_st, q_pos0, n_entries, swa_pos0, kind="flatpool", reindex_kind="pool")
        gi = st.indices.cpu().numpy()
        for b in range(B):
            if run == 0 and kinds[b][0] == "exact":
                assert np.array_equal(st.pool[b, 0].cpu().numpy(), ref_st["pool"][b][0])
            if np.array_equal(gi[b, 0], ref_st["indices"][b, 0]):
                for j in range(4):
                    check_close(outs[j][b, 0].cpu().numpy(), ref_outs[j][b, 0], f"plan run {run} layer {j} seq {b}")
            pool = set(st.pool[b, 0].cpu().numpy().tolist()) - {-1}
            assert set(gi[b, 0].tolist()) <= pool  # Full's indices and Reindex's both lie in the pool
    assert ws.fallbacks() == 0


@pytest.mark.timeout(900)
def test_multi_token_group_128k(csa2):
    """Four query tokens per sequence at the 128K decode shape (16 sequences
    of 131,072 entries), Full + 3 Reuse then Reindex + 3 Reuse, every query
    row's top-k and every layer's attention against the oracle."""
    B, ctx, n_q = 16, 131072, 4
    seed = 1002
    dev = "cuda"
    nib = torch.empty((B * ctx, 256), dtype=torch.uint8, device=dev)
    sc = torch.empty((B * ctx, 32), dtype=torch.uint8, device=dev)
    k8 = torch.empty((B * ctx, 64), dtype=torch.uint8, device=dev)
    ks = torch.empty((B * ctx,), dtype=torch.float32, device=dev)
    for b in range(B):
        sl = slice(b * ctx, (b + 1) * ctx)
        csa2.csa2_quantize_kv(gen.latent(ctx, seed, seq=b, device=dev), k_in=gen.index_key(ctx, seed, seq=b, device=dev),
                              out=[nib[sl], sc[sl], k8[sl], ks[sl]])
    dkv = csa2.make_kv(nib, sc, k8, ks, ctx)
    q_pos0 = [ctx - n_q] * B
    swa_pos0 = [ctx - n_q - 127] * B
    ws = csa2.Workspace(B, n_q, ctx)
    st = csa2.State(B, n_q)
    host = {}
    for run, plan in enumerate(["FUUU", "RUUU"]):
        dl = []
        for j, m in enumerate(plan):
            d = dict(mode={"F": csa2.MODE_FULL, "R": csa2.MODE_REINDEX, "U": csa2.MODE_REUSE}[m],
                     q=gen.attn_query((B, n_q), seed, 10 * run + j, name="mq", device=dev),
                     swa=gen.window_rows(B, n_q + 127, seed, 10 * run + j, name="mswa", device=dev))
            if m in "FR":
                d["idx_q"] = gen.index_query((B, n_q), seed, 10 * run + j, name="midxq", device=dev)
            if m == "F":
                d["kv"] = dkv
            dl.append(d)
        outs = csa2.csa2_run_group(ws, st, dl, q_pos0, [ctx] * B, swa_pos0)
        torch.cuda.synchronize()
        gi = st.indices.cpu().numpy()
        outs_h = [o.cpu().numpy() for o in outs]
        qb = [gen.bf16_bits(L["q"]) for L in dl]
        sb = [gen.bf16_bits(L["swa"]) for L in dl]
        iq = dl[0]["idx_q"].cpu().numpy()
        kinds = []
        for b in range(B):
            if b not in host:
                kf = gen.index_key(ctx, seed, seq=b, device=dev).cpu().numpy()
                rk, rks = oracle.index_key_encode(kf)
                assert np.array_equal(k8[b * ctx:(b + 1) * ctx].cpu().numpy(), rk), f"seq {b}: indexer codes"
                host[b] = (rk, rks)
            rk, rks = host[b]
            s_many = oracle.scores_many(iq[b], None, rk, rks)
            x = gen.latent(ctx, seed, seq=b, device=dev)
            for i in range(n_q):
                nv = q_pos0[b] + i + 1
                ref = oracle.top_k(s_many[i, :nv], np.arange(nv), 512)
                kinds.append(check_topk(gi[b, i], ref, s_many[i, :nv], 512, nv, f"run {run} seq {b} q {i}"))
                sel = gi[b, i][gi[b, i] >= 0]
                sn, ss = oracle.fp4_encode_rows(x[torch.from_numpy(sel.astype(np.int64)).cuda()].cpu().numpy())
                for j in range(4):
                    r = oracle.sparse_swa_attention(qb[j][b, i], sn, ss, np.arange(len(sel)), sb[j][b],
                                                    swa_pos0[b], q_pos0[b] + i)
                    check_close(outs_h[j][b, i], r, f"run {run} layer {j} seq {b} q {i}")
            del x
        print(plan, kinds.count("exact"), "exact,", kinds.count("tie"), "tie", flush=True)
    assert ws.fallbacks() == 0


def test_reindex_with_full_query_reproduces_full(csa2):
    n_entries = [9000, 9000]
    stride = 9000
    dkv, hkv = _kv(csa2, 41, n_entries, stride, False)
    q_pos0 = [n - 1 for n in n_entries]
    swa_pos0 = [p - 127 for p in q_pos0]
    ws = csa2.Workspace(2, 1, stride)
    st = csa2.State(2, 1)
    dl, _ = _layers(csa2, 41, "F", 2, 128, dkv, hkv, 0)
    csa2.csa2_run_group(ws, st, dl, q_pos0, n_entries, swa_pos0)
    full_idx = st.indices.clone()
    dr, _ = _layers(csa2, 41, "RU", 2, 128, dkv, hkv, 5)
    dr[0]["idx_q"] = dl[0]["idx_q"]
    csa2.csa2_run_group(ws, st, dr, q_pos0, n_entries, swa_pos0)
    assert torch.equal(st.indices, full_idx)


def test_state_errors(csa2):
    ws = csa2.Workspace(1, 1, 1000)
    st = csa2.State(1, 1)
    q = gen.attn_query((1, 1), 1, device="cuda")
    swa = gen.window_rows(1, 128, 1, device="cuda")
    with pytest.raises(csa2.Csa2Error) as e:
        csa2.csa2_run_group(ws, st, [dict(mode=csa2.MODE_REUSE, q=q, swa=swa)], [999], [1000], [872])
    assert e.value.code == csa2.ERR_STATE
    iq = gen.index_query((1, 1), 1, device="cuda")
    with pytest.raises(csa2.Csa2Error) as e:
        csa2.csa2_run_group(ws, st, [dict(mode=csa2.MODE_REINDEX, q=q, swa=swa, idx_q=iq)], [999], [1000], [872])
    assert e.value.code == csa2.ERR_STATE


def test_group_odd_layers_and_rows(csa2):
    """Plans whose last layer pair holds one layer (F+2U, R+U, F alone) over
    9 sequences (more than 8 rows, not a multiple of 8), so the decode select
    that attends over its own winners maps its grid the linear way and runs a
    pair of one layer; two of the sequences hold fewer entries than k (300)
    or a single one.  Every layer is compared with the oracle, and a Reuse
    layer with the standalone attention call, bit for bit."""
    n_entries = [3001 + 997 * b for b in range(7)] + [300, 1]
    stride = max(n_entries) + 15
    B = len(n_entries)
    dkv, hkv = _kv(csa2, 43, n_entries, stride, False)
    rows = 128
    q_pos0 = [n - 1 for n in n_entries]
    swa_pos0 = [p - 127 for p in q_pos0]
    ws = csa2.Workspace(B, 1, stride)
    st = csa2.State(B, 1)
    for run, plan in enumerate(["FUU", "RU", "F"]):
        dl, hl = _layers(csa2, 43, plan, B, rows, dkv, hkv, 10 * run)
        outs = csa2.csa2_run_group(ws, st, dl, q_pos0, n_entries, swa_pos0)
        torch.cuda.synchronize()
        print(plan, _compare(outs, st, hkv, hl, n_entries, q_pos0, swa_pos0, plan, "flat"))
        if len(plan) > 1:
            solo = csa2.csa2_sparse_swa_attn(ws, dl[-1]["q"], dkv._tensors[0], dkv._tensors[1], st.indices,
                                             dl[-1]["swa"], q_pos0, swa_pos0, stride)
            assert torch.equal(solo, outs[-1])
    assert ws.fallbacks() == 0
