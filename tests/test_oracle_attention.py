"""Pins of the oracle's attention: a library attention routine when the
selection covers everything, and closed-form special cases."""

import numpy as np
import torch

import oracle


def _case(rng, ctx, rows=128):
    x = rng.standard_normal((ctx, 512)).astype(np.float32)
    nib, scale = oracle.fp4_encode_rows(x)
    q = torch.from_numpy(rng.standard_normal((16, 512)).astype(np.float32) / 8).to(torch.bfloat16)
    swa = torch.from_numpy(rng.standard_normal((rows, 512)).astype(np.float32)).to(torch.bfloat16)
    qb = q.view(torch.int16).numpy().view(np.uint16)
    sb = swa.view(torch.int16).numpy().view(np.uint16)
    return nib, scale, qb, sb


def test_full_coverage_equals_library_attention():
    rng = np.random.default_rng(0)
    ctx = 300
    nib, scale, qb, sb = _case(rng, ctx)
    q_pos = 1000
    idx = np.arange(ctx, dtype=np.int32)
    got = oracle.sparse_swa_attention(qb, nib, scale, idx, sb, q_pos - 127, q_pos, 0.7)
    rows = np.concatenate([oracle.fp4_decode_rows(nib, scale), oracle.bf16_value(sb)])
    q = torch.from_numpy(oracle.bf16_value(qb))[None, :, None, :]          # [1,16,1,512]
    kv = torch.from_numpy(rows)[None, None].expand(1, 16, -1, -1)
    want = torch.nn.functional.scaled_dot_product_attention(q, kv, kv, scale=0.7)
    assert np.allclose(got, want[0, :, 0].numpy(), rtol=1e-6, atol=1e-7)


def test_special_cases():
    rng = np.random.default_rng(1)
    nib, scale, qb, sb = _case(rng, 50)
    none = np.full(512, -1, np.int32)
    # query at token 0 with no selected entries: its window is its own row
    out = oracle.sparse_swa_attention(qb, nib, scale, none, sb, 0, 0)
    assert np.array_equal(out, np.repeat(oracle.bf16_value(sb[:1]).astype(np.float32), 16, 0))
    # equal logits (zero query) average the candidates
    zq = np.zeros_like(qb)
    idx = np.array([3, 7, 9] + [-1] * 509, np.int32)
    out = oracle.sparse_swa_attention(zq, nib, scale, idx, sb, 0, 1)
    rows = np.concatenate([oracle.fp4_decode_rows(nib[[3, 7, 9]], scale[[3, 7, 9]]),
                           oracle.bf16_value(sb[:2])])
    assert np.allclose(out, rows.mean(0)[None].repeat(16, 0), rtol=1e-6, atol=1e-7)
    # order of the index list does not matter
    idx = np.array(list(rng.permutation(50)[:40]) + [-1] * 472, np.int32)
    a = oracle.sparse_swa_attention(qb, nib, scale, idx, sb, 0, 127)
    b = oracle.sparse_swa_attention(qb, nib, scale, idx[::-1].copy(), sb, 0, 127)
    assert np.allclose(a, b, rtol=1e-6, atol=1e-7)
    # the window holds 128 tokens: a query at 200 with rows from token 73 on is served
    out = oracle.sparse_swa_attention(qb, nib, scale, idx, sb, 73, 200)
    assert out.shape == (16, 512)


def test_window_bounds_checked():
    rng = np.random.default_rng(2)
    nib, scale, qb, sb = _case(rng, 10)
    try:
        oracle.sparse_swa_attention(qb, nib, scale, np.full(512, -1, np.int32), sb, 100, 300)
    except ValueError:
        return
    raise AssertionError("missing window rows were not reported")
