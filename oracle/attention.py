"""Sparse + sliding-window attention of the CSA2 step.

TEST INFRASTRUCTURE: see oracle/__init__.py for who may use this package.

What the pages fix: attention runs over the selected entries of the shared
FP4 cache (news.hamidun.com "In DeepSeek-V4.1-Flash the HBM KV cache was cut
to 890 bytes per token ...", section "Three memory-saving mechanisms"), and
every layer keeps sliding-window attention over the last 128 tokens
(ai-wave.ru "DeepSeek V4.1-Flash: 1M context, FP4 KV cache ...", second
paragraph; agentnet.co.il "DeepSeek launches V4.1-Flash ...", section
"Architecture that halves prefill").

Readings (the pages give no formula):
  * one latent per entry serves as both key and value;
  * the window is a separate bfloat16 buffer of raw token rows; a query at
    token position p sees the rows of tokens max(0, p-127) .. p, itself
    included, and these join the selected entries in one softmax, without
    removing overlaps;
  * per head h: l_i = scale * q_h . e_i over the candidate rows e_i,
    out_h = sum_i softmax(l)_i e_i, in float64, reported as float32;
  * the softmax scale is an explicit argument.
"""

import numpy as np

from .formats import bf16_value
from .kv import fp4_decode_rows

SWA_WINDOW = 128


def swa_token_range(q_pos, window=SWA_WINDOW):
    """Tokens [first, last] of the sliding window of a query at token q_pos."""
    return max(0, q_pos - window + 1), q_pos


def attend(q_bits, rows, softmax_scale):
    """Softmax attention of heads q (bf16 bits [16, 512]) over rows float64 [n, 512]."""
    q = bf16_value(q_bits)                                     # [16, 512]
    logits = softmax_scale * (q @ rows.T)                      # [16, n]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=1, keepdims=True)
    return (p @ rows).astype(np.float32)


def sparse_swa_attention(q_bits, nib, scale, indices, swa_bits, swa_pos0, q_pos,
                         softmax_scale=1.0):
    """One query: attention over the selected FP4 entries plus its window.

    q_bits u16[16, 512]; nib u8[n, 256], scale u8[n, 32] (the sequence's
    cache); indices i32[k] (-1 ignored); swa_bits u16[rows, 512] holding
    tokens swa_pos0 .. swa_pos0 + rows - 1; q_pos the query's token position."""
    idx = np.asarray(indices, dtype=np.int64)
    idx = idx[idx >= 0]
    selected = fp4_decode_rows(nib[idx], scale[idx])
    first, last = swa_token_range(q_pos)
    lo, hi = first - swa_pos0, last - swa_pos0
    if lo < 0 or hi >= swa_bits.shape[0]:
        raise ValueError("window rows not present in the sliding-window buffer")
    window = bf16_value(swa_bits[lo: hi + 1])
    return attend(q_bits, np.concatenate([selected, window], axis=0), softmax_scale)
