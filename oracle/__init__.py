"""Plain CPU oracle of the CSA2 sparse-attention decode step with an FP4 KV cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only tests/, __graft_entry__.smoke()
and the cpu_baseline leg of bench.py may import or run anything in this
package.  The GPU library and its Python binding never import it and share no
code with it.

It is written from five public news pages about DeepSeek-V4.1-Flash (ai-wave.ru,
news.hamidun.com, globalfeed.ai, tgviewer.app sof_news24, agentnet.co.il) and
from the public OCP MX definitions of E2M1 and E4M3.  Where the pages are
silent the reading taken is stated in each module's docstring.  Floating point
is float64 unless a reading fixes binary32 (the fp8 key quantiser, the pair
mean and the block-key mean, whose roundings decide stored codes).

Parity status: every function is pinned by tests under tests/ against values
fixed by the format definitions, closed forms, invariants, brute force on tiny
inputs or an independent library routine; the score formula itself is a
reading (the pages print none), pinned only through invariants.
"""

from . import attention, formats, group, indexer, kv, storage  # noqa: F401
from .attention import sparse_swa_attention, swa_token_range  # noqa: F401
from .formats import bf16_value, e2m1_encode, e2m1_value, e4m3_encode, e4m3_value  # noqa: F401
from .group import FULL, REINDEX, REUSE, new_state, run_group  # noqa: F401
from .indexer import (index_flat, index_flat_pool, index_hier, index_pool, scores,  # noqa: F401
                      scores_many, top_k, visible_entries)
from .kv import (block_keys, compress_pairs, fp4_decode_rows, fp4_encode_rows,  # noqa: F401
                 index_key_decode, index_key_encode, index_key_encode_heads, quantize_kv)
