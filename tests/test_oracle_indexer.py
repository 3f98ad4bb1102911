"""Pins of the oracle's indexer: exact integer dots, invariants of the score,
brute-force top-k, and hierarchical == flat where the pool covers everything."""

import itertools

import numpy as np

import oracle
from oracle.formats import e4m3_value


def _codes(rng, shape, hi=0x7E):
    c = rng.integers(0, hi + 1, size=shape).astype(np.uint8)
    return c | (rng.integers(0, 2, size=shape).astype(np.uint8) << 7)


def test_dot_is_exact_integer_arithmetic():
    rng = np.random.default_rng(0)
    q = _codes(rng, (4, 64))
    k = _codes(rng, (50, 64))
    ks = np.ones(50, np.float32)
    s = oracle.scores(q, None, k, ks)
    # the same scores from Python integers: every E4M3 value is n * 2^-9
    qi = [[int(v * 512) for v in e4m3_value(q[h])] for h in range(4)]
    for p in range(50):
        ki = [int(v * 512) for v in e4m3_value(k[p])]
        tot = 0
        for h in range(4):
            d = sum(a * b for a, b in zip(qi[h], ki))
            tot += max(d, 0)
        assert s[p] == tot / 2 ** 18


def test_score_invariants():
    rng = np.random.default_rng(1)
    q = _codes(rng, (4, 64), hi=0x50)
    k = _codes(rng, (300, 64), hi=0x70)
    ks = rng.uniform(0.01, 2, 300).astype(np.float32)
    s = oracle.scores(q, None, k, ks)
    # heads add up: one-hot weights give single-head scores that sum to the total
    single = [oracle.scores(q, np.eye(4)[h], k, ks) for h in range(4)]
    assert np.allclose(sum(single), s, rtol=1e-15, atol=0)
    # ReLU: a head whose query is negated contributes only where the dot was negative
    qn = q.copy()
    qn[0] ^= 0x80
    s0 = single[0]
    s0n = oracle.scores(qn, np.eye(4)[0], k, ks)
    assert np.all((s0 == 0) | (s0n == 0))
    # the key scale multiplies
    assert np.array_equal(oracle.scores(q, None, k, ks * np.float32(2)), 2 * s)
    # joint channel permutation of q and k leaves scores unchanged
    perm = rng.permutation(64)
    assert np.array_equal(oracle.scores(q[:, perm], None, k[:, perm], ks), s)
    # closed form: a key equal to a one-head query scores ks * |q|^2
    kk = q[2:3].copy()
    qv = e4m3_value(q[2])
    assert oracle.scores(q, np.eye(4)[2], kk, np.ones(1, np.float32))[0] == np.dot(qv, qv)
    # zero query: every score is 0
    assert not oracle.scores(np.zeros((4, 64), np.uint8), None, k, ks).any()


def _brute_top_k(score, k):
    """The unique k-subset whose every member beats every non-member under
    (score descending, position ascending)."""
    n = len(score)
    k = min(k, n)

    def beats(a, b):
        return score[a] > score[b] or (score[a] == score[b] and a < b)

    for sub in itertools.combinations(range(n), k):
        rest = set(range(n)) - set(sub)
        if all(beats(a, b) for a in sub for b in rest):
            return sorted(sub)
    raise AssertionError("no dominant subset")


def test_top_k_brute_force_with_ties():
    rng = np.random.default_rng(2)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        k = int(rng.integers(1, 6))
        score = rng.integers(0, 4, n).astype(np.float64)      # many ties
        got = oracle.top_k(score, np.arange(n), k)
        want = _brute_top_k(score, k)
        assert list(got[: len(want)]) == want
        assert np.all(got[len(want):] == -1)


def test_zero_query_selects_first_positions():
    rng = np.random.default_rng(3)
    k8 = _codes(rng, (2000, 64))
    ks = np.ones(2000, np.float32)
    idx = oracle.index_flat(np.zeros((4, 64), np.uint8), None, k8, ks, 2000)
    assert np.array_equal(idx, np.arange(512))
    short = oracle.index_flat(np.zeros((4, 64), np.uint8), None, k8, ks, 100)
    assert np.array_equal(short[:100], np.arange(100)) and np.all(short[100:] == -1)


def test_hierarchical_equals_flat_when_pool_covers_context():
    rng = np.random.default_rng(4)
    for ctx in (5, 700, 4096, 4099):
        k = rng.standard_normal((ctx, 64)).astype(np.float32)
        k8, ks = oracle.index_key_encode(k)
        bk8, bks = oracle.block_keys(k8, ks)
        q = _codes(rng, (4, 64), hi=0x48)
        flat = oracle.index_flat(q, None, k8, ks, ctx)
        hier, pool = oracle.index_hier(q, None, k8, ks, bk8, bks, ctx, n_blocks=2048)
        assert np.array_equal(flat, hier)
        assert np.array_equal(pool[:ctx], np.arange(ctx)) and np.all(pool[ctx:] == -1)


def test_hierarchical_pool_is_top_blocks():
    rng = np.random.default_rng(5)
    ctx = 8 * 64
    k8, ks = oracle.index_key_encode(rng.standard_normal((ctx, 64)).astype(np.float32))
    bk8, bks = oracle.block_keys(k8, ks)
    q = _codes(rng, (4, 64), hi=0x48)
    idx, pool = oracle.index_hier(q, None, k8, ks, bk8, bks, ctx, k=16, n_blocks=4)
    bs = oracle.scores(q, None, bk8, bks)
    best = sorted(np.argsort(-bs, kind="stable")[:4])
    want_pool = np.concatenate([np.arange(8 * b, 8 * b + 8) for b in best])
    assert np.array_equal(pool, want_pool)
    ts = oracle.scores(q, None, k8[want_pool], ks[want_pool])
    want = np.sort(want_pool[np.argsort(-ts, kind="stable")[:16]])
    assert np.array_equal(idx, want)


def test_visibility_rule():
    assert oracle.visible_entries(0, 1) == 1
    assert oracle.visible_entries(9, 1) == 10
    assert oracle.visible_entries(0, 2) == 0          # entry 0 needs tokens 0 and 1
    assert oracle.visible_entries(1, 2) == 1
    assert oracle.visible_entries(262144 + 4095, 2) == 131072 + 2048


def test_scores_many_rows_equal_single_query_scores():
    # the multi-query form is the single-query score row by row, bit for bit
    # (with and without head weights, negative weights included)
    rng = np.random.default_rng(7)
    k8 = rng.integers(0, 256, size=(300, 64)).astype(np.uint8)
    k8[(k8 & 0x7F) == 0x7F] = 0      # no NaN codes
    ks = rng.random(300).astype(np.float32)
    q = rng.integers(0, 256, size=(5, 4, 64)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 1
    w = rng.standard_normal((5, 4)).astype(np.float32)
    many = oracle.scores_many(q, None, k8, ks)
    many_w = oracle.scores_many(q, w, k8, ks)
    assert many.shape == (5, 300)
    for i in range(5):
        assert np.array_equal(many[i], oracle.scores(q[i], None, k8, ks))
        assert np.array_equal(many_w[i], oracle.scores(q[i], w[i], k8, ks))


def test_per_head_keys_dot_each_head_with_its_own_key():
    import torch
    rng = np.random.default_rng(9)
    q = _codes(rng, (4, 64), hi=0x60)
    k = _codes(rng, (120, 4, 64), hi=0x70)
    ks = rng.uniform(0.01, 2, 120).astype(np.float32)
    w = np.array([1.0, 0.5, 2.0, -1.0], np.float32)
    s = oracle.scores(q, w, k, ks)
    # brute force with torch's float8 decoder and Python sums
    qt = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    kt = torch.from_numpy(k).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for p in range(120):
        tot = 0.0
        for h in range(4):
            d = float(sum(float(a) * float(b) for a, b in zip(qt[h], kt[p, h])))
            tot += float(w[h]) * max(d, 0.0)
        assert s[p] == float(ks[p]) * tot
    # four equal heads reduce to the shared-key score
    k1 = k[:, 0]
    assert np.array_equal(oracle.scores(q, w, np.repeat(k1[:, None], 4, axis=1), ks), oracle.scores(q, w, k1, ks))
    # the many-query form agrees row by row
    qs = np.stack([q, _codes(rng, (4, 64), hi=0x60)])
    many = oracle.scores_many(qs, None, k, ks)
    for i in range(2):
        assert np.array_equal(many[i], oracle.scores(qs[i], None, k, ks))
    # flat top-k over per-head keys is the top-k of those scores
    idx = oracle.index_flat(q, w, k, ks, 120, k=10)
    order = sorted(range(120), key=lambda p: (-s[p], p))[:10]
    assert list(idx) == sorted(order)
