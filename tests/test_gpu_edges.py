"""GPU edge cases against the oracle: a batch larger than one launch covers
(64 sequences), sequences with no cache entries inside a batch, and
attention over the largest index list (2,048 entries per query)."""

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


def test_batch_over_one_launch_with_empty_sequences(csa2):
    """70 sequences (two launches of every kernel), ragged lengths, two of
    them with no cache entries: a Full + Reuse group, checked on sequences on
    both sides of the launch boundary."""
    dev = "cuda"
    B, stride, seed = 70, 1500, 31
    rng = np.random.default_rng(seed)
    n_entries = rng.integers(200, stride + 1, size=B).tolist()
    n_entries[5] = 0
    n_entries[66] = 0
    x = gen.latent(B * stride, seed, device=dev)
    k = gen.index_key(B * stride, seed, device=dev)
    nib, sc, k8, ks = csa2.csa2_quantize_kv(x, k_in=k)
    kv = csa2.make_kv(nib, sc, k8, ks, stride)
    q_pos0 = [max(n - 1, 0) for n in n_entries]
    swa_pos0 = [max(p - 127, 0) for p in q_pos0]
    layers = [dict(mode=csa2.MODE_FULL, q=gen.attn_query((B, 1), seed, 0, device=dev),
                   swa=gen.window_rows(B, 128, seed, 0, device=dev),
                   idx_q=gen.index_query((B, 1), seed, 0, device=dev), kv=kv),
              dict(mode=csa2.MODE_REUSE, q=gen.attn_query((B, 1), seed, 1, device=dev),
                   swa=gen.window_rows(B, 128, seed, 1, device=dev))]
    ws = csa2.Workspace(B, 1, stride)
    st = csa2.State(B, 1)
    outs = csa2.csa2_run_group(ws, st, layers, q_pos0, n_entries, swa_pos0)
    torch.cuda.synchronize()
    idx = st.indices.cpu().numpy()
    k8h, ksh = oracle_side.keys(k, k8, ks)
    nibh, sch = oracle_side.fp4(x, nib, sc)
    iq = layers[0]["idx_q"].cpu().numpy()
    for b in range(B):
        n = n_entries[b]
        e0 = b * stride
        ref = oracle.index_flat(iq[b, 0], None, k8h[e0:e0 + n], ksh[e0:e0 + n], n)
        check_topk(idx[b, 0], ref, oracle.scores(iq[b, 0], None, k8h[e0:e0 + n], ksh[e0:e0 + n]), 512, n,
                   f"seq {b}")
        if n == 0:
            assert np.all(idx[b, 0] == -1)
        for j, L in enumerate(layers):  # on the GPU's own index set
            r = oracle.sparse_swa_attention(gen.bf16_bits(L["q"][b, 0]), nibh[e0:e0 + max(n, 1)],
                                            sch[e0:e0 + max(n, 1)], idx[b, 0], gen.bf16_bits(L["swa"][b]),
                                            swa_pos0[b], q_pos0[b])
            check_close(outs[j][b, 0].cpu().numpy(), r, f"seq {b} layer {j}")
    assert ws.fallbacks() == 0


def test_attention_over_the_largest_index_list(csa2):
    """2,048 selected entries per query (34 tiles with the window), two
    sequences with two queries each."""
    dev = "cuda"
    B, ctx, n_q, n_idx, seed = 2, 6000, 2, 2048, 12
    x = gen.latent(B * ctx, seed, device=dev)
    nib, sc = csa2.csa2_quantize_kv(x)
    rng = np.random.default_rng(seed)
    idx = np.stack([np.stack([np.sort(rng.choice(ctx, n_idx, replace=False)) for _ in range(n_q)])
                    for _ in range(B)]).astype(np.int32)
    q_pos0 = [ctx - n_q] * B
    swa_pos0 = [ctx - n_q - 127] * B
    q = gen.attn_query((B, n_q), seed, device=dev)
    swa = gen.window_rows(B, 127 + n_q, seed, device=dev)
    ws = csa2.Workspace(B, n_q, ctx)
    out = csa2.csa2_sparse_swa_attn(ws, q, nib, sc, torch.from_numpy(idx).to(dev), swa, q_pos0, swa_pos0, ctx)
    torch.cuda.synchronize()
    nh, sh = oracle_side.fp4(x, nib, sc)
    for b in range(B):
        for i in range(n_q):
            r = oracle.sparse_swa_attention(gen.bf16_bits(q[b, i]), nh[b * ctx:(b + 1) * ctx], sh[b * ctx:(b + 1) * ctx],
                                            idx[b, i], gen.bf16_bits(swa[b]), swa_pos0[b], q_pos0[b] + i)
            check_close(out[b, i].cpu().numpy(), r, f"b{b} q{i}")
