"""GPU parity of the cache encoders: bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import csa2_inputs as gen
import oracle
import oracle_side

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_decode_fp4_amd as m
    return m


def _edge_rows():
    """Rows with hand-picked blocks: golden cases, every E2M1 tie at several
    scales, zeros, subnormal scales, saturation, negative zeros."""
    rows = np.zeros((4, 512), np.float32)
    ties = np.array([6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, -.25, -.75, -1.25, -1.75, -2.5, -3.5, -5, 0],
                    np.float32)
    for b in range(32):
        rows[0, 16 * b:16 * b + 16] = ties * np.float32(2.0 ** (b - 16))
    rows[1, :16] = [6.375, 1] + [0] * 14
    rows[1, 16:32] = [7.125, 2.5] + [0] * 14
    rows[1, 32:48] = [10000, 1000, -1000] + [0] * 13
    rows[1, 48:64] = [2688, -1344, 672] + [0] * 13
    rows[1, 64:80] = [0.01171875, 0.005859375] + [0] * 14
    rows[1, 80:96] = -0.0
    rows[1, 96:112] = [1e-30, -1e-30] + [0] * 14
    rows[1, 112:128] = np.linspace(-3e-3, 3e-3, 16)
    rng = np.random.default_rng(0)
    rows[2] = rng.standard_normal(512) * np.exp(rng.uniform(-12, 10, 512))
    rows[3] = rng.standard_normal(512).astype(np.float32) * np.float32(1e-3)
    return rows


@pytest.mark.parametrize("ratio", [1, 2])
def test_quantize_bit_exact(csa2, ratio):
    dev = "cuda"
    n_tok = 2 * 3001
    x = gen.latent(n_tok, 11, lognormal=True, device=dev)
    x[:4] = torch.from_numpy(_edge_rows()).to(dev)
    k = gen.index_key(n_tok, 11, device=dev)
    k[5] = 0.0
    k[6, :10] = torch.tensor([448.0, -1e-30, 3e-38, 1.0, 0.5, 1e5, -1e5, 2.0 ** -9, 7.0, 1e-9])
    nib, sc, k8, ks = csa2.csa2_quantize_kv(x, ratio=ratio, k_in=k)
    torch.cuda.synchronize()
    rn, rs, rk, rks = oracle.quantize_kv(x.cpu().numpy(), ratio, k.cpu().numpy())
    assert np.array_equal(sc.cpu().numpy(), rs), "E4M3 scales differ"
    assert np.array_equal(nib.cpu().numpy(), rn), "E2M1 nibbles differ"
    assert np.array_equal(k8.cpu().numpy(), rk), "indexer key codes differ"
    assert np.array_equal(ks.cpu().numpy().view(np.uint32), rks.view(np.uint32)), "key scales differ"


def test_quantize_strided_input_and_empty(csa2):
    dev = "cuda"
    big = gen.latent(300, 3, device=dev)
    wide = torch.zeros((300, 520), dtype=torch.float32, device=dev)
    wide[:, :512] = big
    nib, sc = csa2.csa2_quantize_kv(wide)
    rn, rs = oracle.quantize_kv(big.cpu().numpy(), 1)
    assert np.array_equal(nib.cpu().numpy(), rn) and np.array_equal(sc.cpu().numpy(), rs)
    empty = torch.zeros((0, 512), dtype=torch.float32, device=dev)
    n0, s0 = csa2.csa2_quantize_kv(empty)
    assert n0.shape == (0, 256)


def test_block_keys_bit_exact(csa2):
    dev = "cuda"
    n_entries = [8 * 700, 8 * 311 + 5, 3]
    stride = 8 * 700
    k = gen.index_key(3 * stride, 21, device=dev)
    _, _, k8, ks = csa2.csa2_quantize_kv(gen.latent(3 * stride, 21, device=dev), k_in=k)
    bk8, bks = csa2.csa2_build_block_keys(k8, ks, n_entries, stride)
    torch.cuda.synchronize()
    k8h, ksh = oracle_side.keys(k, k8, ks)  # the oracle's own codes of the same draws
    bst = (stride + 7) // 8
    for s, n in enumerate(n_entries):
        rb, rbs = oracle.block_keys(k8h[s * stride: s * stride + n], ksh[s * stride: s * stride + n])
        nb = len(rbs)
        assert np.array_equal(bk8[s * bst: s * bst + nb].cpu().numpy(), rb), s
        assert np.array_equal(bks[s * bst: s * bst + nb].cpu().numpy().view(np.uint32), rbs.view(np.uint32)), s
