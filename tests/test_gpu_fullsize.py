"""GPU parity at the full workload sizes, every sequence checked.

The GPU runs the whole batch exactly as bench.py does; the oracle then
recomputes every sequence from the same fp32 draws: the indexer keys of the
whole sequence (bit-exact), the main-KV rows of a sample and of every
selected entry (bit-exact), the top-k (tie-aware; hierarchical rows against
the GPU's own pool, see parity.check_hier) and the attention output of every
layer of every run, evaluated by the oracle on the GPU's own index set, so
attention is checked whatever the selection did."""

import sys

import numpy as np
import pytest
import torch

import csa2_inputs as gen
import oracle
from parity import check_close, check_hier, check_topk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_decode_fp4_amd as m
    return m


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _caches(csa2, B, ctx, seed, lognormal, hier):
    dev = "cuda"
    nib = torch.empty((B * ctx, 256), dtype=torch.uint8, device=dev)
    sc = torch.empty((B * ctx, 32), dtype=torch.uint8, device=dev)
    k8 = torch.empty((B * ctx, 64), dtype=torch.uint8, device=dev)
    ks = torch.empty((B * ctx,), dtype=torch.float32, device=dev)
    for b in range(B):
        x = gen.latent(ctx, seed, seq=b, lognormal=lognormal, device=dev)
        k = gen.index_key(ctx, seed, seq=b, device=dev)
        sl = slice(b * ctx, (b + 1) * ctx)
        csa2.csa2_quantize_kv(x, k_in=k, out=[nib[sl], sc[sl], k8[sl], ks[sl]])
        del x, k
    bk8 = bks = None
    bst = 0
    if hier:
        bst = ctx // 8
        bk8, bks = csa2.csa2_build_block_keys(k8, ks, [ctx] * B, ctx)
    return csa2.make_kv(nib, sc, k8, ks, ctx, bk8, bks, bst), (nib, sc, k8, ks, bk8, bks)


class _Seq:
    """The oracle's view of one sequence: its indexer keys encoded from the
    fp32 draws (checked against the GPU's bit for bit), and FP4 rows encoded
    on demand from the fp32 latents."""

    def __init__(self, b, ctx, seed, lognormal, gpu_t, hier):
        nib, sc, k8, ks, bk8, bks = gpu_t
        self.b, self.ctx, self.seed, self.lognormal = b, ctx, seed, lognormal
        self.sl = slice(b * ctx, (b + 1) * ctx)
        kf = gen.index_key(ctx, seed, seq=b, device="cuda").cpu().numpy()
        self.k8, self.ks = oracle.index_key_encode(kf)
        assert np.array_equal(k8[self.sl].cpu().numpy(), self.k8), f"seq {b}: indexer codes"
        assert np.array_equal(ks[self.sl].cpu().numpy().view(np.uint32), self.ks.view(np.uint32)), \
            f"seq {b}: key scales"
        if hier:
            self.bk8, self.bks = oracle.block_keys(self.k8, self.ks)
            bst = ctx // 8
            assert np.array_equal(bk8[b * bst:(b + 1) * bst].cpu().numpy(), self.bk8), f"seq {b}: block keys"
            assert np.array_equal(bks[b * bst:(b + 1) * bst].cpu().numpy().view(np.uint32),
                                  self.bks.view(np.uint32)), f"seq {b}: block key scales"
        self.gnib, self.gsc = nib[self.sl], sc[self.sl]

    def fp4_rows(self, rows):
        """Oracle FP4 codes of the given rows, checked bit-exact against the GPU's."""
        rows_t = torch.from_numpy(np.asarray(rows, dtype=np.int64)).cuda()
        x = gen.latent(self.ctx, self.seed, seq=self.b, lognormal=self.lognormal, device="cuda")
        rn, rs = oracle.fp4_encode_rows(x[rows_t].cpu().numpy())
        del x
        assert np.array_equal(self.gnib[rows_t].cpu().numpy(), rn), f"seq {self.b}: nibbles"
        assert np.array_equal(self.gsc[rows_t].cpu().numpy(), rs), f"seq {self.b}: scales"
        return rn, rs


def _attention_all_layers(s, gpu_idx, layers, outs_h, q_pos, what):
    """Every layer's output against the oracle on the GPU's own index set."""
    sel = gpu_idx[gpu_idx >= 0]
    sn, ss = s.fp4_rows(sel)
    for j, L in enumerate(layers):
        ref = oracle.sparse_swa_attention(L["q_bits"][s.b, 0], sn, ss, np.arange(len(sel)),
                                          L["swa_bits"][s.b], q_pos - 127, q_pos)
        check_close(outs_h[j][s.b, 0], ref, f"{what} layer {j}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_config_full_size(csa2, cfg):
    c = gen.CONFIGS[cfg]
    B, ctx = c["batch"], c["ctx"]
    seed = 1000 + cfg
    hier = c["index"] == "hier"
    kv, gpu_t = _caches(csa2, B, ctx, seed, c["lognormal"], hier)
    ws = csa2.Workspace(B, 1, ctx)
    st = csa2.State(B, 1, with_pool=hier)
    q_pos0, n_entries, swa_pos0 = [ctx - 1] * B, [ctx] * B, [ctx - 128] * B
    seqs = {}
    kinds = []
    for run, plan in enumerate(c["plans"]):
        layers = []
        for j, m in enumerate(plan):
            li = 4 * run + j
            d = dict(mode={"F": csa2.MODE_FULL, "R": csa2.MODE_REINDEX, "U": csa2.MODE_REUSE}[m],
                     q=gen.attn_query((B, 1), seed, li, device="cuda"),
                     swa=gen.window_rows(B, 128, seed, li, lognormal=c["lognormal"], device="cuda"))
            if m in "FR":
                d["idx_q"] = gen.index_query((B, 1), seed, li, device="cuda")
            if m == "F":
                d["kv"] = kv
            layers.append(d)
        outs = csa2.csa2_run_group(ws, st, layers, q_pos0, n_entries, swa_pos0,
                                   index_kind=csa2.INDEX_HIER if hier else csa2.INDEX_FLAT)
        torch.cuda.synchronize()
        idx = st.indices.cpu().numpy()
        gpool = st.pool.cpu().numpy() if hier else None
        outs_h = [o.cpu().numpy() for o in outs]
        hl = [dict(q_bits=gen.bf16_bits(L["q"]), swa_bits=gen.bf16_bits(L["swa"])) for L in layers]
        iq = layers[0]["idx_q"].cpu().numpy()
        for b in range(B):
            if b not in seqs:
                seqs[b] = _Seq(b, ctx, seed, c["lognormal"], gpu_t, hier)
                if run == 0:  # a fixed sample of main-KV rows, bit-exact
                    rng = np.random.default_rng(b)
                    seqs[b].fp4_rows(np.sort(rng.choice(ctx, size=min(2048, ctx), replace=False)))
            s = seqs[b]
            if hier and plan[0] == "F":
                kinds.append(check_hier(idx[b, 0], gpool[b, 0], iq[b, 0], None, s.k8, s.ks, s.bk8, s.bks, ctx,
                                        what=f"run {run} seq {b}"))
            else:
                ref = oracle.index_flat(iq[b, 0], None, s.k8, s.ks, ctx)
                kinds.append(check_topk(idx[b, 0], ref, oracle.scores(iq[b, 0], None, s.k8, s.ks), 512, ctx,
                                        f"run {run} seq {b}"))
            _attention_all_layers(s, idx[b, 0], hl, outs_h, ctx - 1, f"run {run} seq {b}")
            _say(f"config {cfg} run {run} seq {b}: {kinds[-1]}")
    _say(f"config {cfg}: {kinds}")
    # the candidate pass held every row's answer: no exact recompute
    assert ws.fallbacks() == 0


@pytest.mark.timeout(900)
def test_prefill_full_size(csa2):
    """The full prefill chunk (262,144-token prefix + 4,096 queries, ratio 2):
    the chunk's encoding bit-exact, and 256 query rows (the first three, the
    last two and 251 drawn by a fixed seed) against the oracle: the top-k and
    every layer's attention on the GPU's own index set."""
    c = gen.CONFIGS[4]
    P, T = c["prefix_tokens"], c["chunk"]
    seed = 1004
    n_ent = (P + T) // 2
    dev = "cuda"
    x = gen.latent(P + T, seed, device=dev)
    kin = gen.index_key(P + T, seed, device=dev)
    nib, sc, k8, ks = csa2.csa2_quantize_kv(x, ratio=2, k_in=kin)
    kv = csa2.make_kv(nib, sc, k8, ks, n_ent)
    swa_pos0 = P - 127
    layers = []
    for j, m in enumerate(c["plans"][0]):
        d = dict(mode=csa2.MODE_FULL if m == "F" else csa2.MODE_REUSE,
                 q=gen.attn_query((1, T), seed, j, device=dev),
                 swa=gen.window_rows(1, P + T - swa_pos0, seed, j, device=dev))
        if m == "F":
            d["idx_q"], d["kv"] = gen.index_query((1, T), seed, j, device=dev), kv
        layers.append(d)
    ws = csa2.Workspace(1, T, n_ent)
    st = csa2.State(1, T)
    outs = csa2.csa2_run_group(ws, st, layers, [P], [n_ent], [swa_pos0], ratio=2)
    torch.cuda.synchronize()
    kh = kin.cpu().numpy()
    rk, rks = oracle.index_key_encode(oracle.compress_pairs(kh, 2))
    assert np.array_equal(k8.cpu().numpy(), rk) and np.array_equal(ks.cpu().numpy().view(np.uint32),
                                                                    rks.view(np.uint32))
    iq = layers[0]["idx_q"].cpu().numpy()
    idx = st.indices.cpu().numpy()
    gnib, gsc = nib.cpu().numpy(), sc.cpu().numpy()
    qb = [gen.bf16_bits(L["q"]) for L in layers]
    sb = [gen.bf16_bits(L["swa"]) for L in layers]
    outs_h = [o.cpu().numpy() for o in outs]
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, 1, 2, T - 2, T - 1], rng.choice(np.arange(3, T - 2), 251, replace=False)]))
    assert len(rows) == 256
    kinds = []
    for r0 in range(0, len(rows), 32):
        part = rows[r0:r0 + 32]
        sc_many = oracle.scores_many(iq[0, part], None, rk, rks)
        for i, s_row in zip(part, sc_many):
            nv = oracle.visible_entries(P + i, 2)
            ref = oracle.top_k(s_row[:nv], np.arange(nv), 512)
            kinds.append(check_topk(idx[0, i], ref, s_row[:nv], 512, nv, f"query {i}"))
            sel = idx[0, i][idx[0, i] >= 0]
            tok = np.concatenate([2 * sel[:, None], 2 * sel[:, None] + 1], axis=1).reshape(-1)
            xs = x[torch.from_numpy(tok.astype(np.int64)).cuda()].cpu().numpy()
            sn, ss = oracle.fp4_encode_rows(oracle.compress_pairs(xs, 2))
            assert np.array_equal(gnib[sel], sn) and np.array_equal(gsc[sel], ss), f"query {i}: FP4 rows"
            for j in range(len(layers)):
                r = oracle.sparse_swa_attention(qb[j][0, i], sn, ss, np.arange(len(sel)), sb[j][0], swa_pos0, P + i)
                check_close(outs_h[j][0, i], r, f"query {i} layer {j}")
        _say(f"prefill rows {r0}..{r0 + len(part) - 1}: {kinds[-len(part):].count('exact')} exact")
    nfb = ws.fallbacks()
    _say("prefill full size:", kinds.count("exact"), "exact,", kinds.count("tie"), "tie; exact recomputes:", nfb)
    assert nfb <= T // 100
