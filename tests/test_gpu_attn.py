"""GPU parity of sparse + sliding-window attention against the oracle, on the
oracle's own index lists (so attention is checked apart from top-k)."""

import numpy as np
import pytest
import torch

import csa2_inputs as gen
import oracle
import oracle_side
from parity import check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_decode_fp4_amd as m
    return m


def _case(csa2, seed, batch, ctx, n_q, q_pos0, n_idx, lognormal=False, pad=0):
    dev = "cuda"
    x = gen.latent(batch * ctx, seed, lognormal=lognormal, device=dev)
    nib, sc = csa2.csa2_quantize_kv(x)
    _case.oracle_codes = oracle_side.fp4(x, nib, sc)
    rng = np.random.default_rng(seed)
    idx = np.full((batch, n_q, n_idx), -1, np.int32)
    for b in range(batch):
        for i in range(n_q):
            m = min(ctx, n_idx - pad)
            idx[b, i, :m] = np.sort(rng.choice(ctx, size=m, replace=False))
    swa_pos0 = [max(0, p - 127) for p in q_pos0]
    rows = max(q_pos0) + n_q - min(swa_pos0)
    rows = max(rows, 128 + n_q)
    q = gen.attn_query((batch, n_q), seed, device=dev)
    swa = gen.window_rows(batch, rows, seed, lognormal=lognormal, device=dev)
    return nib, sc, torch.from_numpy(idx).to(dev), q, swa, swa_pos0


@pytest.mark.parametrize("batch,ctx,n_q,n_idx,q_pos,pad,lognormal", [
    (1, 4096, 1, 512, 4095, 0, False),      # decode-shaped, 10 tiles split over workgroups
    (3, 2000, 1, 512, 1999, 37, True),      # -1 padding, lognormal channel scales
    (2, 700, 1, 100, 60, 0, False),          # short window (query before token 127), ragged tile
    (1, 600, 5, 512, 300, 0, False),         # several queries per sequence
    (2, 300, 1, 0, 299, 0, False),           # window only
])
def test_attention_matches_oracle(csa2, batch, ctx, n_q, n_idx, q_pos, pad, lognormal):
    nib, sc, idx, q, swa, swa_pos0 = _case(csa2, 7 + n_idx, batch, ctx, n_q, [q_pos] * batch, n_idx,
                                           lognormal, pad)
    ws = csa2.Workspace(batch, n_q, ctx)
    out = csa2.csa2_sparse_swa_attn(ws, q, nib, sc, idx, swa, [q_pos] * batch, swa_pos0, ctx,
                                    softmax_scale=1.0)
    torch.cuda.synchronize()
    (nh, sh), ih = _case.oracle_codes, idx.cpu().numpy()
    qb, sb = gen.bf16_bits(q), gen.bf16_bits(swa)
    for b in range(batch):
        for i in range(n_q):
            ref = oracle.sparse_swa_attention(qb[b, i], nh[b * ctx:(b + 1) * ctx], sh[b * ctx:(b + 1) * ctx],
                                              ih[b, i], sb[b], swa_pos0[b], q_pos + i, 1.0)
            check_close(out[b, i].cpu().numpy(), ref, f"b{b} q{i}")
    # a second call on the same workspace gives identical bits (deterministic merge)
    out2 = csa2.csa2_sparse_swa_attn(ws, q, nib, sc, idx, swa, [q_pos] * batch, swa_pos0, ctx)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("big", [1e5, 1e30])
def test_attention_with_window_values_past_fp16(csa2, big):
    """Window rows of magnitude 1e5 or 1e30 (bf16 holds them, fp16 does not):
    the split partials keep them in range, so the merged output matches."""
    batch, ctx, q_pos, n_idx = 2, 2000, 1999, 512
    nib, sc, idx, q, swa, swa_pos0 = _case(csa2, 29, batch, ctx, 1, [q_pos] * batch, n_idx)
    swa = (swa.float() * big).to(torch.bfloat16)
    ws = csa2.Workspace(batch, 1, ctx)
    out = csa2.csa2_sparse_swa_attn(ws, q, nib, sc, idx, swa, [q_pos] * batch, swa_pos0, ctx,
                                    softmax_scale=1.0 / big)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    (nh, sh), ih = _case.oracle_codes, idx.cpu().numpy()
    qb, sb = gen.bf16_bits(q), gen.bf16_bits(swa)
    for b in range(batch):
        ref = oracle.sparse_swa_attention(qb[b, 0], nh[b * ctx:(b + 1) * ctx], sh[b * ctx:(b + 1) * ctx],
                                          ih[b, 0], sb[b], swa_pos0[b], q_pos, 1.0 / big)
        assert np.abs(ref).max() > big / 100  # the window rows do carry weight
        # the tolerance holds in units of the window rows' scale
        check_close(out[b, 0].cpu().numpy().astype(np.float64) / big, ref / big, f"b{b} x{big:g}")
