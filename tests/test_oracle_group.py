"""Pins of the oracle's layer plan: Reuse keeps indices bit for bit, Reindex
with the Full layer's own query reproduces it, a Full + 3 Reuse group equals
four single attention calls, and illegal orders are refused."""

import numpy as np
import pytest
import torch

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


# --- hierarchical Full layer, and Reindex over its pool ----------------------
# A context of 20,000 entries has 2,500 blocks of 8, so the 2,048 kept blocks
# are a strict subset and the pool is not the whole context.  The checks below
# rank by brute force, with torch's float8 decoder and Python sorting, and so
# share no arithmetic with the oracle's indexer.
HCTX = 20000


def _brute_scores(idx_q, k8, ks):
    q = torch.from_numpy(np.ascontiguousarray(idx_q)).view(torch.float8_e4m3fn).to(torch.float64)
    k = torch.from_numpy(np.ascontiguousarray(k8)).view(torch.float8_e4m3fn).to(torch.float64)
    dots = torch.clamp(k @ q.T, min=0.0).sum(dim=1)
    return (torch.from_numpy(np.asarray(ks, dtype=np.float64)) * dots).numpy()


def _brute_top(score, positions, k):
    order = sorted(range(len(positions)), key=lambda i: (-score[i], positions[i]))
    return sorted(int(positions[i]) for i in order[:k])


def _hier_kv(seed):
    x = gen.latent(HCTX, seed).numpy()
    k = gen.index_key(HCTX, seed).numpy()
    nib, sc, k8, ks = oracle.quantize_kv(x, 1, k)
    bk8, bks = oracle.block_keys(k8, ks)
    return dict(nib=[nib], scale=[sc], k8=[k8], ks=[ks], bk8=[bk8], bks=[bks])


def _hier_layer(mode, seed, layer, kv=None):
    d = dict(mode=mode, q=gen.bf16_bits(gen.attn_query((1, 1), seed, layer)),
             swa=gen.bf16_bits(gen.window_rows(1, 128, seed, layer)))
    if mode != oracle.REUSE:
        d["idx_q"] = gen.index_query((1, 1), seed, layer).numpy()
        d["idx_w"] = None
    if kv is not None:
        d["kv"] = kv
    return d


def _hier_run(layers, st, reindex_kind="flat"):
    return oracle.run_group(layers, st, [HCTX - 1], [HCTX], [HCTX - 128], kind="hier",
                            reindex_kind=reindex_kind)


def test_hier_full_stores_the_pool_of_the_best_blocks():
    kv = _hier_kv(11)
    st = oracle.new_state()
    full = _hier_layer(oracle.FULL, 11, 0, kv)
    _hier_run([full, _hier_layer(oracle.REUSE, 11, 1)], st)
    iq = full["idx_q"][0, 0]
    bsc = _brute_scores(iq, kv["bk8"][0], kv["bks"][0])
    n_blk = len(bsc)
    assert n_blk == HCTX // 8
    blocks = _brute_top(bsc, np.arange(n_blk), 2048)
    want_pool = sorted(p for b in blocks for p in range(8 * b, 8 * b + 8) if p < HCTX)
    pool = np.asarray(st["pool"][0][0])
    assert len(want_pool) == 2048 * 8
    assert np.array_equal(pool[pool >= 0], want_pool) and np.all(pool[len(want_pool):] == -1)
    # the Full layer's indices: the top 512 positions inside that pool
    tsc = _brute_scores(iq, kv["k8"][0][want_pool], kv["ks"][0][want_pool])
    assert np.array_equal(st["indices"][0, 0], _brute_top(tsc, np.asarray(want_pool), 512))
    # and they differ from the flat top-512 over the whole context (the pool
    # is a real restriction on this input)
    flat = _brute_top(_brute_scores(iq, kv["k8"][0], kv["ks"][0]), np.arange(HCTX), 512)
    assert not np.array_equal(st["indices"][0, 0], flat)


def test_pool_reindex_ranks_only_the_stored_pool():
    kv = _hier_kv(12)
    st = oracle.new_state()
    full = _hier_layer(oracle.FULL, 12, 0, kv)
    _hier_run([full], st, "pool")
    full_idx = st["indices"].copy()
    pool = np.asarray(st["pool"][0][0])
    pool = pool[pool >= 0]
    # with the Full layer's own indexer query the pool Reindex gives the Full
    # layer's indices back
    re = _hier_layer(oracle.REINDEX, 12, 1)
    re["idx_q"] = full["idx_q"]
    _hier_run([re], st, "pool")
    assert np.array_equal(st["indices"], full_idx)
    # with a fresh query: the top 512 of the pool, not of the whole context
    re2 = _hier_layer(oracle.REINDEX, 12, 2)
    reuse = _hier_layer(oracle.REUSE, 12, 3)
    outs = _hier_run([re2, reuse], st, "pool")
    iq = re2["idx_q"][0, 0]
    want = _brute_top(_brute_scores(iq, kv["k8"][0][pool], kv["ks"][0][pool]), pool, 512)
    assert np.array_equal(st["indices"][0, 0], want)
    flat = _brute_top(_brute_scores(iq, kv["k8"][0], kv["ks"][0]), np.arange(HCTX), 512)
    assert not np.array_equal(want, flat)
    # the Reuse layer attends over those indices
    one = oracle.sparse_swa_attention(reuse["q"][0, 0], kv["nib"][0], kv["scale"][0], np.asarray(want),
                                      reuse["swa"][0], HCTX - 128, HCTX - 1)
    assert np.array_equal(outs[1][0, 0], one)
    # a flat reindex of the same query ranks the whole context instead
    st2 = oracle.new_state()
    _hier_run([full, re2], st2, "flat")
    assert np.array_equal(st2["indices"][0, 0], flat)


def test_pool_reindex_needs_a_hierarchical_pool():
    st = oracle.new_state()
    kv = _hier_kv(13)
    oracle.run_group([_hier_layer(oracle.FULL, 13, 0, kv)], st, [HCTX - 1], [HCTX], [HCTX - 128], kind="flat")
    with pytest.raises(RuntimeError):
        _hier_run([_hier_layer(oracle.REINDEX, 13, 1)], st, "pool")


# --- flat Full layer that keeps a pool from its own token scores -------------
def test_flat_pool_keeps_the_blocks_of_the_best_token_scores():
    kv = _hier_kv(14)
    st = oracle.new_state()
    full = _hier_layer(oracle.FULL, 14, 0, kv)
    oracle.run_group([full], st, [HCTX - 1], [HCTX], [HCTX - 128], kind="flatpool")
    iq = full["idx_q"][0, 0]
    tsc = _brute_scores(iq, kv["k8"][0], kv["ks"][0])
    # the indices are the flat top 512 over the whole context
    flat = _brute_top(tsc, np.arange(HCTX), 512)
    assert np.array_equal(st["indices"][0, 0], flat)
    # block b scores the largest of its 8 token scores
    bmax = [max(tsc[p] for p in range(8 * b, min(8 * b + 8, HCTX))) for b in range(-(-HCTX // 8))]
    blocks = _brute_top(np.asarray(bmax), np.arange(len(bmax)), 2048)
    want_pool = sorted(p for b in blocks for p in range(8 * b, 8 * b + 8) if p < HCTX)
    pool = np.asarray(st["pool"][0][0])
    assert np.array_equal(pool[pool >= 0], want_pool) and np.all(pool[len(want_pool):] == -1)
    assert set(flat) <= set(want_pool)      # the indices' blocks are always kept
    # a different pool from the block-key reading on the same input
    _, hpool = oracle.index_hier(iq, None, kv["k8"][0], kv["ks"][0], kv["bk8"][0], kv["bks"][0], HCTX)
    assert not np.array_equal(hpool, pool)
    # a pool Reindex with a fresh query ranks that pool
    re = _hier_layer(oracle.REINDEX, 14, 1)
    oracle.run_group([re], st, [HCTX - 1], [HCTX], [HCTX - 128], kind="flatpool", reindex_kind="pool")
    iq2 = re["idx_q"][0, 0]
    wp = np.asarray(want_pool)
    assert np.array_equal(st["indices"][0, 0], _brute_top(_brute_scores(iq2, kv["k8"][0][wp], kv["ks"][0][wp]), wp, 512))


def test_flat_pool_block_ties_and_partial_blocks():
    iq = np.full((4, 64), 0x38, np.uint8)            # every code 1.0
    k8 = np.full((37, 64), 0x38, np.uint8)
    ks = np.ones(37, np.float32)
    # equal scores everywhere: the lower blocks win, the partial block 4 keeps
    # its 5 positions
    idx, pool = oracle.index_flat_pool(iq, None, k8, ks, 37, k=3, n_blocks=5)
    assert list(idx) == [0, 1, 2]
    assert list(pool[:37]) == list(range(37)) and np.all(pool[37:] == -1)
    idx, pool = oracle.index_flat_pool(iq, None, k8, ks, 37, k=3, n_blocks=2)
    assert list(pool[:16]) == list(range(16)) and np.all(pool[16:] == -1)
    # one larger key in the partial block and one in block 1: those two blocks
    ks2 = ks.copy()
    ks2[35], ks2[9] = 2.0, 1.5
    idx, pool = oracle.index_flat_pool(iq, None, k8, ks2, 37, k=2, n_blocks=2)
    assert list(idx) == [9, 35]
    assert list(pool[:13]) == list(range(8, 16)) + list(range(32, 37)) and np.all(pool[13:] == -1)
    # a position past n_visible never counts for its block
    idx, pool = oracle.index_flat_pool(iq, None, k8, ks2, 34, k=2, n_blocks=1)
    assert list(pool[:8]) == list(range(8, 16)) and np.all(pool[8:] == -1)


def test_flat_full_drops_an_earlier_pool():
    st = oracle.new_state()
    kv = _hier_kv(15)
    _hier_run([_hier_layer(oracle.FULL, 15, 0, kv)], st)
    assert st["pool"] is not None
    oracle.run_group([_hier_layer(oracle.FULL, 15, 1, kv)], st, [HCTX - 1], [HCTX], [HCTX - 128], kind="flat")
    assert st["pool"] is None
    with pytest.raises(RuntimeError):
        _hier_run([_hier_layer(oracle.REINDEX, 15, 2)], st, "pool")
