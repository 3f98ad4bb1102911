"""Pins of the oracle's layer plan: Reuse keeps indices bit for bit, Reindex
with the Full layer's own query reproduces it, a Full + 3 Reuse group equals
four single attention calls, and illegal orders are refused."""

import numpy as np
import pytest

import csa2_inputs as gen
import oracle

B, CTX = 2, 1500


def _kv(seed):
    nib, sc, k8, ks = [], [], [], []
    for b in range(B):
        x = gen.latent(CTX, seed, seq=b).numpy()
        k = gen.index_key(CTX, seed, seq=b).numpy()
        n_, s_, k_, ks_ = oracle.quantize_kv(x, 1, k)
        nib.append(n_); sc.append(s_); k8.append(k_); ks.append(ks_)
    bk = [oracle.block_keys(k8[b], ks[b]) for b in range(B)]
    return dict(nib=nib, scale=sc, k8=k8, ks=ks, bk8=[b[0] for b in bk], bks=[b[1] for b in bk])


def _layer(mode, seed, layer, kv=None):
    d = dict(mode=mode,
             q=gen.bf16_bits(gen.attn_query((B, 1), seed, layer)),
             swa=gen.bf16_bits(gen.window_rows(B, 128, seed, layer)))
    if mode != oracle.REUSE:
        d["idx_q"] = gen.index_query((B, 1), seed, layer).numpy()
        d["idx_w"] = None
    if kv is not None:
        d["kv"] = kv
    return d


def _run(plan_layers, state):
    q_pos0 = [CTX - 1] * B
    return oracle.run_group(plan_layers, state, q_pos0, [CTX] * B, [CTX - 128] * B)


def test_reuse_keeps_indices_and_equals_single_calls():
    kv = _kv(1)
    st = oracle.new_state()
    layers = [_layer(oracle.FULL, 1, 0, kv)] + [_layer(oracle.REUSE, 1, l) for l in (1, 2, 3)]
    outs = _run(layers, st)
    full_idx = st["indices"].copy()
    for b in range(B):
        want_idx = oracle.index_flat(layers[0]["idx_q"][b, 0], None, kv["k8"][b], kv["ks"][b], CTX)
        assert np.array_equal(full_idx[b, 0], want_idx)
    for l, out in enumerate(outs):
        for b in range(B):
            one = oracle.sparse_swa_attention(layers[l]["q"][b, 0], kv["nib"][b], kv["scale"][b],
                                              full_idx[b, 0], layers[l]["swa"][b], CTX - 128, CTX - 1)
            assert np.array_equal(out[b, 0], one)
    # a second call with Reuse only keeps the same indices bit for bit
    _run([_layer(oracle.REUSE, 1, 9)], st)
    assert np.array_equal(st["indices"], full_idx)


def test_reindex_with_full_query_reproduces_full():
    kv = _kv(2)
    st = oracle.new_state()
    full = _layer(oracle.FULL, 2, 0, kv)
    _run([full], st)
    full_idx = st["indices"].copy()
    re = _layer(oracle.REINDEX, 2, 5)
    re["idx_q"] = full["idx_q"]
    _run([re], st)
    assert np.array_equal(st["indices"], full_idx)
    re2 = _layer(oracle.REINDEX, 2, 6)
    _run([re2], st)
    assert not np.array_equal(st["indices"], full_idx)       # a fresh query ranks anew
    assert st["kv"] is kv                                     # and keeps the Full KV


def test_illegal_orders_refused():
    with pytest.raises(RuntimeError):
        _run([_layer(oracle.REUSE, 3, 0)], oracle.new_state())
    with pytest.raises(RuntimeError):
        _run([_layer(oracle.REINDEX, 3, 0)], oracle.new_state())


def test_prefill_rows_match_single_queries_and_short_prefixes_take_all():
    # ratio 2, queries at tokens 0..n_q-1 of a fresh sequence: query p sees (p+1)//2
    # entries; below 512 visible entries it selects all of them
    rng_seed = 4
    n_tok = 64
    x = gen.latent(n_tok, rng_seed).numpy()
    k = gen.index_key(n_tok, rng_seed).numpy()
    nib, sc, k8, ks = oracle.quantize_kv(x, 2, k)
    kv = dict(nib=[nib], scale=[sc], k8=[k8], ks=[ks])
    n_q = n_tok
    layer = dict(mode=oracle.FULL, kv=kv,
                 q=gen.bf16_bits(gen.attn_query((1, n_q), rng_seed)),
                 swa=gen.bf16_bits(gen.window_rows(1, n_tok, rng_seed)),
                 idx_q=gen.index_query((1, n_q), rng_seed).numpy(), idx_w=None)
    st = oracle.new_state()
    out = oracle.run_group([layer], st, [0], [n_tok // 2], [0], ratio=2)[0]
    for p in range(n_q):
        nv = (p + 1) // 2
        assert np.array_equal(st["indices"][0, p, :nv], np.arange(nv))
        assert np.all(st["indices"][0, p, nv:] == -1)
    # the last row equals a one-query call at that position
    last = dict(layer, q=layer["q"][:, -1:], idx_q=layer["idx_q"][:, -1:])
    st1 = oracle.new_state()
    out1 = oracle.run_group([last], st1, [n_q - 1], [n_tok // 2], [0], ratio=2)[0]
    assert np.array_equal(out1[0, 0], out[0, -1])
