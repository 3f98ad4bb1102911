"""GPU parity of the decode-step write side (csa2_append) and of attention
over a window ring.  Appending tokens one step at a time must give the bytes
the oracle's bulk encoders give for the whole token history (FP4 main KV,
fp8 indexer keys, block keys; pair means at ratio 2), and the window ring
must hold bf16(x) of the last tokens, which attention then reads exactly as
it reads a linear window."""

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


def _bf16_bits(x):
    return x.to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("ratio", [1, 2])
def test_append_matches_bulk_encoding(csa2, ratio):
    dev = "cuda"
    prefix = [0, 26, 80]            # tokens already in the cache (even at ratio 2)
    steps = 37                      # appended tokens: crosses block and ring boundaries
    batch = len(prefix)
    n_tok = [p + steps for p in prefix]
    stride = max(n_tok) // ratio + 8
    bst = (stride + 7) // 8
    ring = 128
    seed = 41 + ratio
    xs = [gen.latent(n, seed, seq=b, device=dev) for b, n in enumerate(n_tok)]
    ks = [gen.index_key(n, seed, seq=b, device=dev) for b, n in enumerate(n_tok)]
    nib = torch.zeros((batch * stride, 256), dtype=torch.uint8, device=dev)
    sc = torch.zeros((batch * stride, 32), dtype=torch.uint8, device=dev)
    k8 = torch.zeros((batch * stride, 64), dtype=torch.uint8, device=dev)
    kscale = torch.zeros((batch * stride,), dtype=torch.float32, device=dev)
    bk8 = torch.zeros((batch * bst, 64), dtype=torch.uint8, device=dev)
    bks = torch.zeros((batch * bst,), dtype=torch.float32, device=dev)
    swa = torch.zeros((batch, ring, 512), dtype=torch.bfloat16, device=dev)
    pending = torch.zeros((batch, 576), dtype=torch.float32, device=dev)
    # the prefix through the bulk encoders
    for b, p in enumerate(prefix):
        if p == 0:
            continue
        e0, e1 = b * stride, b * stride + p // ratio
        csa2.csa2_quantize_kv(xs[b][:p].contiguous(), ratio=ratio, k_in=ks[b][:p].contiguous(),
                              out=[nib[e0:e1], sc[e0:e1], k8[e0:e1], kscale[e0:e1]])
    csa2.csa2_build_block_keys(k8, kscale, [p // ratio for p in prefix], stride, bk8, bks, bst)
    # then one token per sequence per step
    for t in range(steps):
        pos = [p + t for p in prefix]
        x = torch.stack([xs[b][pos[b]] for b in range(batch)]).contiguous()
        k = torch.stack([ks[b][pos[b]] for b in range(batch)]).contiguous()
        csa2.csa2_append(x, k, pos, nib, sc, k8, kscale, stride, ratio=ratio, bk8=bk8, bkscale=bks,
                         bk_stride=bst, pending=pending, swa=swa, swa_ring=ring)
    torch.cuda.synchronize()
    for b, n in enumerate(n_tok):
        ne = n // ratio             # at ratio 2 an odd count leaves the last token pending
        xh, kh = xs[b][:ratio * ne].cpu().numpy(), ks[b][:ratio * ne].cpu().numpy()
        rn, rs, rk, rks = oracle.quantize_kv(xh, ratio, kh)
        e0 = b * stride
        assert np.array_equal(nib[e0:e0 + ne].cpu().numpy(), rn), f"seq {b}: nibbles"
        assert np.array_equal(sc[e0:e0 + ne].cpu().numpy(), rs), f"seq {b}: scales"
        assert np.array_equal(k8[e0:e0 + ne].cpu().numpy(), rk), f"seq {b}: key codes"
        assert np.array_equal(kscale[e0:e0 + ne].cpu().numpy().view(np.uint32), rks.view(np.uint32))
        rbk, rbks = oracle.block_keys(rk, rks)
        nb = (ne + 7) // 8
        assert np.array_equal(bk8[b * bst: b * bst + nb].cpu().numpy(), rbk), f"seq {b}: block keys"
        assert np.array_equal(bks[b * bst: b * bst + nb].cpu().numpy().view(np.uint32), rbks.view(np.uint32))
        # the ring holds the last appended tokens, token t at row t % ring
        ring_bits = swa[b].view(torch.int16).cpu().numpy().view(np.uint16)
        for tok in range(max(prefix[b], n - ring), n):
            assert np.array_equal(ring_bits[tok % ring], _bf16_bits(xs[b][tok])), f"seq {b}: window row of {tok}"


def test_ring_window_attention_matches_linear(csa2):
    """The same window rows laid out linearly and as a ring (wrapping inside
    the window) give bit-identical attention, which also matches the oracle."""
    dev = "cuda"
    batch, ctx, n_q, ring, seed = 2, 3000, 3, 160, 8
    q_pos0 = [1000, 2995]                        # window 873..1002 and 2868..2997
    x = gen.latent(batch * ctx, seed, device=dev)
    nib, sc = csa2.csa2_quantize_kv(x)
    rng = np.random.default_rng(seed)
    idx = np.stack([np.stack([np.sort(rng.choice(ctx, 512, replace=False)) for _ in range(n_q)])
                    for _ in range(batch)]).astype(np.int32)
    idx_d = torch.from_numpy(idx).to(dev)
    q = gen.attn_query((batch, n_q), seed, device=dev)
    rows = 128 + n_q - 1
    swa_pos0 = [p - 127 for p in q_pos0]
    lin = gen.window_rows(batch, rows, seed, device=dev)
    rg = torch.zeros((batch, ring, 512), dtype=torch.bfloat16, device=dev)
    for b in range(batch):
        for r in range(rows):
            rg[b, (swa_pos0[b] + r) % ring] = lin[b, r]
    ws = csa2.Workspace(batch, n_q, ctx)
    out_lin = csa2.csa2_sparse_swa_attn(ws, q, nib, sc, idx_d, lin, q_pos0, swa_pos0, ctx)
    out_ring = csa2.csa2_sparse_swa_attn(ws, q, nib, sc, idx_d, rg, q_pos0, None, ctx, swa_ring=ring)
    torch.cuda.synchronize()
    assert torch.equal(out_lin, out_ring)
    nh, sh = oracle_side.fp4(x, nib, sc)
    for b in range(batch):
        for i in range(n_q):
            ref = oracle.sparse_swa_attention(gen.bf16_bits(q[b, i]), nh[b * ctx:(b + 1) * ctx],
                                              sh[b * ctx:(b + 1) * ctx], idx[b, i],
                                              gen.bf16_bits(lin[b]), swa_pos0[b], q_pos0[b] + i)
            check_close(out_ring[b, i].cpu().numpy(), ref, f"b{b} q{i}")


def test_decode_steps_self_contained(csa2):
    """Three decode steps, each: append the new token (cache, block keys,
    window ring), then a Full + Reuse group on it.  The last step's indices
    and outputs match the oracle run on the whole token history."""
    dev = "cuda"
    batch, prefix, steps, ring, seed = 2, 3000, 3, 128, 19
    n_tok = prefix + steps
    stride = n_tok
    xs = [gen.latent(n_tok, seed, seq=b, device=dev) for b in range(batch)]
    ks = [gen.index_key(n_tok, seed, seq=b, device=dev) for b in range(batch)]
    nib = torch.zeros((batch * stride, 256), dtype=torch.uint8, device=dev)
    sc = torch.zeros((batch * stride, 32), dtype=torch.uint8, device=dev)
    k8 = torch.zeros((batch * stride, 64), dtype=torch.uint8, device=dev)
    kscale = torch.zeros((batch * stride,), dtype=torch.float32, device=dev)
    swa = [torch.zeros((batch, ring, 512), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    for b in range(batch):
        e0 = b * stride
        csa2.csa2_quantize_kv(xs[b][:prefix].contiguous(), k_in=ks[b][:prefix].contiguous(),
                              out=[nib[e0:e0 + prefix], sc[e0:e0 + prefix], k8[e0:e0 + prefix],
                                   kscale[e0:e0 + prefix]])
        # the window rows of the prefix (each layer keeps its own window of
        # raw rows; here both layers window the latent stream)
        for L in range(2):
            for tok in range(prefix - ring, prefix):
                swa[L][b, tok % ring] = xs[b][tok].to(torch.bfloat16)
    kv = csa2.make_kv(nib, sc, k8, kscale, stride)
    ws = csa2.Workspace(batch, 1, stride)
    st = csa2.State(batch, 1)
    for t in range(steps):
        pos = prefix + t
        x = torch.stack([xs[b][pos] for b in range(batch)]).contiguous()
        k = torch.stack([ks[b][pos] for b in range(batch)]).contiguous()
        csa2.csa2_append(x, k, [pos] * batch, nib, sc, k8, kscale, stride, swa=swa[0], swa_ring=ring)
        csa2.csa2_append(x, k, [pos] * batch, nib, sc, k8, kscale, stride, swa=swa[1], swa_ring=ring)
        layers = [dict(mode=csa2.MODE_FULL, q=gen.attn_query((batch, 1), seed + t, 0, device=dev), swa=swa[0],
                       idx_q=gen.index_query((batch, 1), seed + t, 0, device=dev), kv=kv),
                  dict(mode=csa2.MODE_REUSE, q=gen.attn_query((batch, 1), seed + t, 1, device=dev), swa=swa[1])]
        outs = csa2.csa2_run_group(ws, st, layers, [pos] * batch, [pos + 1] * batch, None, swa_ring=ring)
    torch.cuda.synchronize()
    pos = prefix + steps - 1
    idx = st.indices.cpu().numpy()
    for b in range(batch):
        xh, kh = xs[b].cpu().numpy(), ks[b].cpu().numpy()
        rn, rs, rk, rks = oracle.quantize_kv(xh, 1, kh)
        iq = layers[0]["idx_q"][b, 0].cpu().numpy()
        ref_idx = oracle.index_flat(iq, None, rk, rks, pos + 1)
        check_topk(idx[b, 0], ref_idx, oracle.scores(iq, None, rk, rks), 512, pos + 1, f"seq {b}")
        win = _bf16_bits(xs[b][pos - 127: pos + 1])
        for j, L in enumerate(layers):  # on the GPU's own index set
            ref = oracle.sparse_swa_attention(gen.bf16_bits(L["q"][b, 0]), rn, rs, idx[b, 0], win, pos - 127, pos)
            check_close(outs[j][b, 0].cpu().numpy(), ref, f"seq {b} layer {j}")
    assert ws.fallbacks() == 0
