"""The oracle's own encodings of the fp32 draws a GPU test started from.

Every GPU test hands the oracle inputs the oracle made itself: the caches
are encoded here from the same fp32 draws the GPU encoded, and checked equal
to the GPU's bytes on the way (the encoders are bit-exact), so no oracle
input is a GPU result."""

import numpy as np

import oracle


def keys(k_fp32, k8_gpu=None, ks_gpu=None, ratio=1):
    """Oracle indexer codes / scales of fp32 keys [n_tok, 64] (a torch tensor
    on any device), ratio-2 pairs averaged first; checked against the GPU's."""
    kh = k_fp32.detach().cpu().numpy()
    if ratio == 2:
        kh = oracle.compress_pairs(kh, 2)
    rk, rks = oracle.index_key_encode(kh)
    if k8_gpu is not None:
        assert np.array_equal(k8_gpu.cpu().numpy(), rk), "indexer codes differ from the oracle's"
        assert np.array_equal(ks_gpu.cpu().numpy().view(np.uint32), rks.view(np.uint32)), "key scales differ"
    return rk, rks


def fp4(x_fp32, nib_gpu=None, sc_gpu=None, ratio=1):
    """Oracle FP4 codes / scales of fp32 latents [n_tok, 512]; checked
    against the GPU's."""
    xh = x_fp32.detach().cpu().numpy()
    if ratio == 2:
        xh = oracle.compress_pairs(xh, 2)
    rn, rs = oracle.fp4_encode_rows(xh)
    if nib_gpu is not None:
        assert np.array_equal(nib_gpu.cpu().numpy(), rn), "FP4 nibbles differ from the oracle's"
        assert np.array_equal(sc_gpu.cpu().numpy(), rs), "FP4 scales differ from the oracle's"
    return rn, rs


def block_keys(rk, rks, n_entries, stride, bk8_gpu=None, bks_gpu=None):
    """Oracle block keys of each sequence (stored stride entries apart),
    concatenated ceil(stride / 8) blocks apart; checked against the GPU's."""
    bst = (stride + 7) // 8
    bk = np.zeros((len(n_entries) * bst, 64), np.uint8)
    bs = np.zeros(len(n_entries) * bst, np.float32)
    for b, n in enumerate(n_entries):
        a, s = oracle.block_keys(rk[b * stride: b * stride + n], rks[b * stride: b * stride + n])
        bk[b * bst: b * bst + len(a)] = a
        bs[b * bst: b * bst + len(s)] = s
        if bk8_gpu is not None:
            nb = len(a)
            assert np.array_equal(bk8_gpu[b * bst: b * bst + nb].cpu().numpy(), a), f"seq {b}: block keys"
            assert np.array_equal(bks_gpu[b * bst: b * bst + nb].cpu().numpy().view(np.uint32), s.view(np.uint32))
    return bk, bs
