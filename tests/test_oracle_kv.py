"""Pins of the oracle's cache encoders and of the storage arithmetic."""

import numpy as np

import oracle
from oracle import storage


def test_storage_reproduces_890_bytes_per_token():
    # news.hamidun.com "... KV cache was cut to 890 bytes per token instead of 3514",
    # opening paragraph: 890 B/token; layer plans from agentnet.co.il, section
    # "CSA2: compression along the layer axis"
    assert storage.main_kv_bytes_per_entry() == 256 + 32
    assert storage.bytes_per_entry() == 288 + 64 + 4
    assert storage.kv_bytes_per_token() == 890
    plans = storage.layer_plans()
    assert len(plans) == 38                       # 18 encoder + 20 decoder CSA2 layers
    assert sum(1 for m, r in plans if m == oracle.FULL) == 4
    # FP4 nearly halves the FP8 cache (ai-wave.ru, fourth paragraph): 288 of 512 bytes
    assert 0.5 < storage.main_kv_bytes_per_entry() / 512 < 0.6
    # about four times below the predecessor's 3,514 B/token (ai-wave.ru, first paragraph)
    assert round(3514 / storage.kv_bytes_per_token()) == 4


def test_index_key_quantiser():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((500, 64)).astype(np.float32)
    k[3] = 0.0
    codes, ks = oracle.index_key_encode(k)
    amax = np.abs(k).max(axis=1)
    assert ks.dtype == np.float32
    assert np.array_equal(ks, (amax / np.float32(448)).astype(np.float32))
    assert ks[3] == 0 and not codes[3].any()
    # the amax element lands on the top code 448
    arg = np.abs(k).argmax(axis=1)
    top = codes[np.arange(500), arg] & 0x7F
    assert np.all(top[np.arange(500) != 3] == 0x7E)
    # dequantised key within half an E4M3 step (relative 2^-4) or half the
    # subnormal step of the key's own scale
    deq = oracle.e4m3_value(codes) * ks[:, None]
    err = np.abs(deq - k)
    assert np.all(err <= np.maximum(np.abs(k) * 2.0 ** -4, 2.0 ** -10 * ks[:, None]) * 1.0001)


def test_pair_mean_closed_form():
    x = np.arange(8 * 512, dtype=np.float32).reshape(8, 512)
    e = oracle.compress_pairs(x, 2)
    assert e.shape == (4, 512)
    assert np.array_equal(e, (x[0::2] + 0.5 * 512).astype(np.float32))
    assert np.array_equal(oracle.compress_pairs(np.ones((2, 64), np.float32) * 3, 2),
                          np.full((1, 64), 3, np.float32))


def test_block_key_of_identical_keys_is_the_key():
    # a key whose scale is a power of two dequantises exactly, so the mean of
    # eight copies re-encodes to the same codes and scale
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 0x7E, size=(1, 64)).astype(np.uint8)
    codes[0, 0] = 0x7E
    codes[0, 1] = 0x80 | 0x33
    k8 = np.repeat(codes, 8, axis=0)
    ks = np.full(8, 0.125, np.float32)
    bk, bks = oracle.block_keys(k8, ks)
    assert bk.shape == (1, 64) and bks[0] == np.float32(0.125)
    assert np.array_equal(bk[0], codes[0])
    # token score equals block score for such a block
    q = rng.integers(0, 0x7E, size=(4, 64)).astype(np.uint8)
    assert oracle.scores(q, None, bk, bks)[0] == oracle.scores(q, None, k8[:1], ks[:1])[0]


def test_block_keys_partial_tail_and_order():
    rng = np.random.default_rng(9)
    k = rng.standard_normal((11, 64)).astype(np.float32)
    k8, ks = oracle.index_key_encode(k)
    bk, bks = oracle.block_keys(k8, ks)
    assert bk.shape == (2, 64)
    kd = oracle.index_key_decode(k8, ks)
    acc = np.zeros(64, np.float32)
    for r in kd[8:11]:
        acc = (acc + r).astype(np.float32)
    want = oracle.index_key_encode((acc / np.float32(3)).astype(np.float32)[None])
    assert np.array_equal(bk[1], want[0][0]) and bks[1] == want[1][0]


def test_quantize_kv_ratio2_is_pair_mean_then_encode():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((6, 512)).astype(np.float32)
    k = rng.standard_normal((6, 64)).astype(np.float32)
    nib, sc, k8, ks = oracle.quantize_kv(x, 2, k)
    m = ((x[0::2] + x[1::2]).astype(np.float32) * np.float32(0.5)).astype(np.float32)
    n2, s2 = oracle.fp4_encode_rows(m)
    assert np.array_equal(nib, n2) and np.array_equal(sc, s2)
    assert k8.shape == (3, 64) and ks.shape == (3,)


def test_per_head_key_quantiser_and_its_storage():
    import torch
    rng = np.random.default_rng(3)
    k = rng.standard_normal((300, 4, 64)).astype(np.float32)
    k[7] = 0.0
    k[9, 2] *= 50.0                       # one head dominates the shared scale
    codes, ks = oracle.index_key_encode_heads(k)
    assert codes.shape == (300, 4, 64) and ks.dtype == np.float32
    # one scale over all four heads: fp32(amax / 448)
    amax = np.abs(k.reshape(300, -1)).max(axis=1)
    assert np.array_equal(ks, (amax / np.float32(448)).astype(np.float32))
    assert ks[7] == 0 and not codes[7].any()
    # codes: E4M3 (torch's round-to-nearest-even float8 cast) of fp32(k / ks)
    r = (k[ks > 0] / ks[ks > 0][:, None, None]).astype(np.float32)
    want = torch.from_numpy(np.clip(r, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[ks > 0], want)
    # a position whose four heads are equal keeps the shared key's codes
    same = np.repeat(k[:1, :1], 4, axis=1)
    c1, s1 = oracle.index_key_encode(k[0, :1])
    c4, s4 = oracle.index_key_encode_heads(same)
    assert np.array_equal(s1, s4) and all(np.array_equal(c4[0, h], c1[0]) for h in range(4))
    # the per-head layout costs 2.5 x (288 + 256 + 4) = 1,370 B/token
    assert storage.bytes_per_entry(4) == 288 + 256 + 4
    assert storage.kv_bytes_per_token(4) == 1370
