"""Encoders of the CSA2 caches: FP4 main KV, fp8 indexer key, block keys.

TEST INFRASTRUCTURE: see oracle/__init__.py for who may use this package.

Main KV (ai-wave.ru "DeepSeek V4.1-Flash: 1M context, FP4 KV cache ...",
fourth paragraph; globalfeed.ai "DeepSeek-V4.1-Flash released ...", section
"What changed in the architecture"; agentnet.co.il "DeepSeek launches
V4.1-Flash ...", section "Quantization and deployment"): every position keeps
one latent row of 512 channels (a reading: the pages give no width), stored
as 4-bit E2M1 values with one E4M3 scale per 16 consecutive channels and no
global scale.

Readings where the pages are silent:
  * the block scale S is the E4M3 value nearest to amax/6 (6 = largest E2M1
    magnitude), from the real quotient, ties to even, saturating at 448;
  * every element code is the E2M1 value nearest to x/S (real quotient), ties
    to even, sign bit = sign of x; when S == 0 every code is 0;
  * byte i of a row holds channel 2i in its low nibble and channel 2i+1 in its
    high nibble; scale j covers channels 16j .. 16j+15;
  * the indexer key is 64 fp8 channels with one float32 scale:
    ks = fp32(amax / 448), code = E4M3(fp32(k / ks)), both IEEE binary32
    divisions; amax == 0 gives ks = 0 and all-zero codes;
  * at compression ratio 2 an entry is the float32 mean of a token pair,
    fp32(fp32(x_2j + x_2j+1) * 0.5), taken before encoding (globalfeed.ai,
    section "What changed in the architecture", and agentnet.co.il, section
    "CSA2: compression along the layer axis", give ratio 2 for the encoder);
  * a block key (agentnet.co.il, section "CSA2: compression along the layer
    axis": blocks of 8 positions) is the float32 mean of the dequantised
    keys of the block, summed in position order and divided by the number of
    keys present, then encoded like any indexer key;
  * per-head keys (the other layout reading: each of the 4 indexer heads
    has its own 64-channel key) are quantised as one
    256-value vector: one float32 scale ks = fp32(amax / 448) over all four
    heads, codes as above.
"""

import numpy as np

from .formats import e2m1_encode, e2m1_value, e4m3_encode, e4m3_value

D_LATENT = 512
SCALE_GROUP = 16
D_INDEX = 64
BLOCK = 8


def compress_pairs(x, ratio):
    """Entries from tokens at the given compression ratio (1 or 2), float32."""
    x = np.asarray(x, dtype=np.float32)
    if ratio == 1:
        return x.copy()
    if ratio != 2 or x.shape[0] % 2:
        raise ValueError("ratio must be 1, or 2 with an even token count")
    pair_sum = (x[0::2] + x[1::2]).astype(np.float32)
    return (pair_sum * np.float32(0.5)).astype(np.float32)


def fp4_encode_rows(x):
    """FP4-encode float32 rows [n, 512] -> (nibbles u8[n, 256], scales u8[n, 32])."""
    x = np.asarray(x, dtype=np.float32)
    n, d = x.shape
    if d != D_LATENT:
        raise ValueError("latent rows have 512 channels")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the contract")
    blocks = x.astype(np.float64).reshape(n, d // SCALE_GROUP, SCALE_GROUP)
    amax = np.abs(blocks).max(axis=2)
    scale_code = e4m3_encode(amax / 6.0)                      # [n, 32]
    s = e4m3_value(scale_code)[:, :, None]                    # [n, 32, 1]
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(s > 0, blocks / np.where(s > 0, s, 1.0), 0.0)
    codes = e2m1_encode(ratio).astype(np.int64)
    codes = np.where(s > 0, codes, 0)                          # S == 0 -> code 0
    codes = codes.reshape(n, d)
    nib = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return nib, scale_code.astype(np.uint8)


def fp4_decode_rows(nib, scale):
    """Dequantised float64 rows [n, 512] from (nibbles, scales)."""
    nib = np.asarray(nib, dtype=np.int64)
    n = nib.shape[0]
    codes = np.empty((n, D_LATENT), dtype=np.int64)
    codes[:, 0::2] = nib & 15
    codes[:, 1::2] = nib >> 4
    s = np.repeat(e4m3_value(np.asarray(scale)), SCALE_GROUP, axis=1)
    return e2m1_value(codes) * s


def index_key_encode(k):
    """Indexer keys float32 [n, 64] -> (codes u8[n, 64], scales f32[n])."""
    k = np.asarray(k, dtype=np.float32)
    if k.shape[1] != D_INDEX:
        raise ValueError("indexer keys have 64 channels")
    return _key_encode(k)


def index_key_encode_heads(k):
    """Per-head indexer keys float32 [n, 4, 64] -> (codes u8[n, 4, 64],
    scales f32[n]): one scale per position over its four heads."""
    k = np.asarray(k, dtype=np.float32)
    if k.ndim != 3 or k.shape[1:] != (4, D_INDEX):
        raise ValueError("per-head indexer keys are [n, 4, 64]")
    codes, ks = _key_encode(k.reshape(k.shape[0], 4 * D_INDEX))
    return codes.reshape(k.shape), ks


def _key_encode(k):
    """Rows of float32 key values -> (codes, one float32 scale per row)."""
    if not np.all(np.isfinite(k)):
        raise ValueError("non-finite input is outside the contract")
    amax = np.abs(k).max(axis=1)
    ks = (amax / np.float32(448.0)).astype(np.float32)         # IEEE binary32 divide
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(ks[:, None] > 0, k / np.where(ks > 0, ks, np.float32(1))[:, None],
                     np.float32(0)).astype(np.float32)
    codes = e4m3_encode(r.astype(np.float64))
    codes = np.where(ks[:, None] > 0, codes, 0).astype(np.uint8)
    return codes, ks


def index_key_decode(codes, ks):
    """Dequantised indexer keys as float32 (code value times scale, one binary32
    rounding), the values the block-key mean is taken over."""
    v = e4m3_value(np.asarray(codes)).astype(np.float32)
    return (v * np.asarray(ks, dtype=np.float32)[:, None]).astype(np.float32)


def block_keys(codes, ks):
    """Block keys over blocks of 8 consecutive entries: (codes u8[nb, 64], f32[nb])."""
    kd = index_key_decode(codes, ks)
    n = kd.shape[0]
    nb = -(-n // BLOCK)
    acc = np.zeros((nb, D_INDEX), dtype=np.float32)
    count = np.zeros(nb, dtype=np.float32)
    for j in range(BLOCK):                 # position order inside every block
        rows = kd[j::BLOCK]                # entry 8b + j of every block b holding one
        acc[: len(rows)] = (acc[: len(rows)] + rows).astype(np.float32)
        count[: len(rows)] += 1
    means = (acc / count[:, None]).astype(np.float32)
    return index_key_encode(means)


def quantize_kv(x, ratio=1, k=None):
    """Whole encoder step: tokens -> entries -> FP4 main KV (+ fp8 indexer keys).

    Returns (nib, scale) or (nib, scale, k8, ks) when indexer keys are given."""
    e = compress_pairs(x, ratio)
    nib, scale = fp4_encode_rows(e)
    if k is None:
        return nib, scale
    k = np.asarray(k, dtype=np.float32)
    if k.ndim == 3:  # per-head keys [n, 4, 64]
        e = compress_pairs(k.reshape(k.shape[0], -1), ratio)
        k8, ks = index_key_encode_heads(e.reshape(e.shape[0], 4, D_INDEX))
    else:
        k8, ks = index_key_encode(compress_pairs(k, ratio))
    return nib, scale, k8, ks
