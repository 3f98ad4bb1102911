"""Global-KV storage per token implied by the layer plans and the entry layout.

TEST INFRASTRUCTURE: see oracle/__init__.py for who may use this package.

The pages put the global KV in HBM at 890 bytes per token (news.hamidun.com
"In DeepSeek-V4.1-Flash the HBM KV cache was cut to 890 bytes per token ...",
opening paragraph) and credit most of the saving to layers sharing one FP4
cache (same page, section "Three memory-saving mechanisms").  The plans
(agentnet.co.il "DeepSeek launches V4.1-Flash ...", section "CSA2: compression
along the layer axis"; globalfeed.ai "DeepSeek-V4.1-Flash released ...",
section "What changed in the architecture"): 18 encoder layers at ratio 2 in
three groups of one Full and five Reuse; 20 decoder layers at ratio 1 in five
groups of four, Full + 3 Reuse first, then Reindex + 3 Reuse.  Only Full
layers store an entry.
"""

import numpy as np

from .group import FULL, REINDEX, REUSE
from .kv import fp4_encode_rows, index_key_encode, index_key_encode_heads

ENCODER_PLAN = [FULL] + [REUSE] * 5
ENCODER_GROUPS, ENCODER_RATIO = 3, 2
DECODER_FIRST = [FULL] + [REUSE] * 3
DECODER_LATER = [REINDEX] + [REUSE] * 3
DECODER_GROUPS, DECODER_RATIO = 5, 1


def layer_plans():
    """[(mode, ratio)] for every layer: encoder then decoder."""
    enc = [(m, ENCODER_RATIO) for _ in range(ENCODER_GROUPS) for m in ENCODER_PLAN]
    dec = [(m, DECODER_RATIO) for m in DECODER_FIRST]
    dec += [(m, DECODER_RATIO) for _ in range(DECODER_GROUPS - 1) for m in DECODER_LATER]
    return enc + dec


def bytes_per_entry(key_heads=1):
    """Bytes one stored entry takes, measured on the encoders' own outputs
    (key_heads 4: the per-head indexer-key layout)."""
    nib, scale = fp4_encode_rows(np.zeros((1, 512), dtype=np.float32))
    if key_heads == 4:
        k8, ks = index_key_encode_heads(np.zeros((1, 4, 64), dtype=np.float32))
    else:
        k8, ks = index_key_encode(np.zeros((1, 64), dtype=np.float32))
    return nib.nbytes + scale.nbytes + k8.nbytes + ks.nbytes


def main_kv_bytes_per_entry():
    nib, scale = fp4_encode_rows(np.zeros((1, 512), dtype=np.float32))
    return nib.nbytes + scale.nbytes


def kv_bytes_per_token(key_heads=1):
    """Global-KV bytes per context token summed over the Full layers."""
    per_entry = bytes_per_entry(key_heads)
    return sum(per_entry / ratio for mode, ratio in layer_plans() if mode == FULL)
