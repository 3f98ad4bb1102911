"""GPU parity at the full workload sizes, on sampled sequences.

The GPU runs the whole batch exactly as bench.py does; the oracle then
recomputes sampled sequences from the same fp32 draws: the indexer keys of
the whole sequence (bit-exact), the top-k (tie-aware), and attention on the
main-KV rows it needs, which it encodes itself from the fp32 source."""

import numpy as np
import pytest
import torch

import csa2_inputs as gen
import oracle
from parity import check_close, check_topk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_decode_fp4_amd as m
    return m


def _caches(csa2, B, ctx, seed, lognormal, hier):
    dev = "cuda"
    nib = torch.empty((B * ctx, 256), dtype=torch.uint8, device=dev)
    sc = torch.empty((B * ctx, 32), dtype=torch.uint8, device=dev)
    k8 = torch.empty((B * ctx, 64), dtype=torch.uint8, device=dev)
    ks = torch.empty((B * ctx,), dtype=torch.float32, device=dev)
    for b in range(B):
        x = gen.latent(ctx, seed, seq=b, lognormal=lognormal, device=dev)
        k = gen.index_key(ctx, seed, seq=b, device=dev)
        sl = slice(b * ctx, (b + 1) * ctx)
        csa2.csa2_quantize_kv(x, k_in=k, out=[nib[sl], sc[sl], k8[sl], ks[sl]])
        del x, k
    bk8 = bks = None
    bst = 0
    if hier:
        bst = ctx // 8
        bk8, bks = csa2.csa2_build_block_keys(k8, ks, [ctx] * B, ctx)
    return csa2.make_kv(nib, sc, k8, ks, ctx, bk8, bks, bst), (nib, sc, k8, ks, bk8, bks)


def _check_sequence(b, ctx, seed, lognormal, gpu_t, layers_dev, outs, idx_gpu, hier, sample_rows=2048):
    nib, sc, k8, ks, bk8, bks = gpu_t
    sl = slice(b * ctx, (b + 1) * ctx)
    x = gen.latent(ctx, seed, seq=b, lognormal=lognormal, device="cuda")
    kf = gen.index_key(ctx, seed, seq=b, device="cuda").cpu().numpy()
    rk, rks = oracle.index_key_encode(kf)
    assert np.array_equal(k8[sl].cpu().numpy(), rk), f"seq {b}: indexer codes"
    assert np.array_equal(ks[sl].cpu().numpy().view(np.uint32), rks.view(np.uint32)), f"seq {b}: key scales"
    # main KV: bit-exact on a sample of rows
    rng = np.random.default_rng(b)
    rows = np.sort(rng.choice(ctx, size=min(sample_rows, ctx), replace=False))
    xr = x[torch.from_numpy(rows).cuda()].cpu().numpy()
    rn, rs = oracle.fp4_encode_rows(xr)
    assert np.array_equal(nib[sl][torch.from_numpy(rows).cuda()].cpu().numpy(), rn), f"seq {b}: nibbles"
    assert np.array_equal(sc[sl][torch.from_numpy(rows).cuda()].cpu().numpy(), rs), f"seq {b}: scales"
    L0 = layers_dev[0]
    iq = L0["idx_q"][b, 0].cpu().numpy()
    if hier:
        rbk, rbks = oracle.block_keys(rk, rks)
        bst = ctx // 8
        assert np.array_equal(bk8[b * bst:(b + 1) * bst].cpu().numpy(), rbk), f"seq {b}: block keys"
        ref_idx, ref_pool = oracle.index_hier(iq, None, rk, rks, rbk, rbks, ctx)
        bscore = oracle.scores(iq, None, rbk, rbks)
        srt = np.sort(bscore)[::-1]
        gap = (srt[2047] - srt[2048]) / abs(srt[2047])
        if gap <= 1e-5:
            return "block-tie"
        valid = ref_pool[ref_pool >= 0]
        score = dict(zip(valid.tolist(), oracle.scores(iq, None, rk[valid], rks[valid]).tolist()))
        n_vis = len(valid)
    else:
        ref_idx = oracle.index_flat(iq, None, rk, rks, ctx)
        score = oracle.scores(iq, None, rk, rks)
        n_vis = ctx
    kind = check_topk(idx_gpu[b, 0], ref_idx, score, 512, n_vis, f"seq {b}")
    if not np.array_equal(idx_gpu[b, 0], ref_idx):
        return kind
    # attention of every layer on these indices: encode just the selected rows
    sel = ref_idx[ref_idx >= 0]
    xs = x[torch.from_numpy(sel.astype(np.int64)).cuda()].cpu().numpy()
    sn, ss = oracle.fp4_encode_rows(xs)
    for j, L in enumerate(layers_dev):
        ref = oracle.sparse_swa_attention(gen.bf16_bits(L["q"][b:b + 1])[0, 0], sn, ss, np.arange(len(sel)),
                                          gen.bf16_bits(L["swa"][b:b + 1])[0], ctx - 128, ctx - 1)
        check_close(outs[j][b, 0].cpu().numpy(), ref, f"seq {b} layer {j}")
    return kind


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_config_full_size(csa2, cfg):
    c = gen.CONFIGS[cfg]
    B, ctx = c["batch"], c["ctx"]
    seed = 1000 + cfg
    hier = c["index"] == "hier"
    kv, gpu_t = _caches(csa2, B, ctx, seed, c["lognormal"], hier)
    ws = csa2.Workspace(B, 1, ctx)
    st = csa2.State(B, 1, with_pool=hier)
    q_pos0, n_entries, swa_pos0 = [ctx - 1] * B, [ctx] * B, [ctx - 128] * B
    samples = [0, B - 1] if B > 1 else [0]
    kinds = []
    for run, plan in enumerate(c["plans"]):
        layers = []
        for j, m in enumerate(plan):
            li = 4 * run + j
            d = dict(mode={"F": csa2.MODE_FULL, "R": csa2.MODE_REINDEX, "U": csa2.MODE_REUSE}[m],
                     q=gen.attn_query((B, 1), seed, li, device="cuda"),
                     swa=gen.window_rows(B, 128, seed, li, lognormal=c["lognormal"], device="cuda"))
            if m in "FR":
                d["idx_q"] = gen.index_query((B, 1), seed, li, device="cuda")
            if m == "F":
                d["kv"] = kv
            layers.append(d)
        outs = csa2.csa2_run_group(ws, st, layers, q_pos0, n_entries, swa_pos0,
                                   index_kind=csa2.INDEX_HIER if hier else csa2.INDEX_FLAT)
        torch.cuda.synchronize()
        idx = st.indices.cpu().numpy()
        if run == 0:
            for b in samples:
                kinds.append(_check_sequence(b, ctx, seed, c["lognormal"], gpu_t, layers, outs, idx, hier))
        else:
            # Reindex run: same KV, fresh indexer query; Reuse layers keep its indices
            for b in samples:
                kf = gen.index_key(ctx, seed, seq=b, device="cuda").cpu().numpy()
                rk, rks = oracle.index_key_encode(kf)
                iq = layers[0]["idx_q"][b, 0].cpu().numpy()
                ref_idx = oracle.index_flat(iq, None, rk, rks, ctx)
                kinds.append(check_topk(idx[b, 0], ref_idx, oracle.scores(iq, None, rk, rks), 512, ctx,
                                        f"reindex seq {b}"))
    print(f"config {cfg}: {kinds}")
    # the threshold pass held every row's answer: no exact recompute
    assert ws.fallbacks() == 0


def test_prefill_full_size(csa2):
    """The full prefill chunk (262,144-token prefix + 4,096 queries, ratio 2):
    sampled query rows against the oracle, the chunk's encoding bit-exact."""
    c = gen.CONFIGS[4]
    P, T = c["prefix_tokens"], c["chunk"]
    seed = 1004
    n_ent = (P + T) // 2
    dev = "cuda"
    x = gen.latent(P + T, seed, device=dev)
    kin = gen.index_key(P + T, seed, device=dev)
    nib, sc, k8, ks = csa2.csa2_quantize_kv(x, ratio=2, k_in=kin)
    kv = csa2.make_kv(nib, sc, k8, ks, n_ent)
    swa_pos0 = P - 127
    layers = []
    for j, m in enumerate(c["plans"][0]):
        d = dict(mode=csa2.MODE_FULL if m == "F" else csa2.MODE_REUSE,
                 q=gen.attn_query((1, T), seed, j, device=dev),
                 swa=gen.window_rows(1, P + T - swa_pos0, seed, j, device=dev))
        if m == "F":
            d["idx_q"], d["kv"] = gen.index_query((1, T), seed, j, device=dev), kv
        layers.append(d)
    ws = csa2.Workspace(1, T, n_ent)
    st = csa2.State(1, T)
    outs = csa2.csa2_run_group(ws, st, layers, [P], [n_ent], [swa_pos0], ratio=2)
    torch.cuda.synchronize()
    kh = kin.cpu().numpy()
    rk, rks = oracle.index_key_encode(oracle.compress_pairs(kh, 2))
    assert np.array_equal(k8.cpu().numpy(), rk) and np.array_equal(ks.cpu().numpy().view(np.uint32), rks.view(np.uint32))
    iq = layers[0]["idx_q"].cpu().numpy()
    idx = st.indices.cpu().numpy()
    xh = x.cpu().numpy()
    kinds = []
    for i in [0, 1, 2, 777, 2048, 4094, 4095]:
        nv = oracle.visible_entries(P + i, 2)
        ref = oracle.index_flat(iq[0, i], None, rk, rks, nv)
        kinds.append(check_topk(idx[0, i], ref, oracle.scores(iq[0, i], None, rk[:nv], rks[:nv]), 512, nv, f"query {i}"))
        if not np.array_equal(idx[0, i], ref):
            continue
        sel = ref[ref >= 0]
        rows = np.concatenate([2 * sel[:, None], 2 * sel[:, None] + 1], axis=1).reshape(-1)
        sn, ss = oracle.fp4_encode_rows(oracle.compress_pairs(xh[rows], 2))
        for j, L in enumerate(layers):
            r = oracle.sparse_swa_attention(gen.bf16_bits(L["q"][:, i:i + 1])[0, 0], sn, ss, np.arange(len(sel)),
                                            gen.bf16_bits(L["swa"])[0], swa_pos0, P + i)
            check_close(outs[j][0, i].cpu().numpy(), r, f"query {i} layer {j}")
    nfb = ws.fallbacks()
    print("prefill full size:", kinds, "exact recomputes:", nfb)
    assert nfb <= T // 100
