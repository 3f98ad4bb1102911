"""GPU parity of a ratio-2 prefill chunk: pair-mean encoding of the chunk,
causal per-query indexing over prefix + chunk entries, and a Full + 5 Reuse
group with many query rows."""

import numpy as np
import pytest
import torch

import csa2_inputs as gen
import oracle
from parity import check_close, check_topk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_decode_fp4_amd as m
    return m


@pytest.mark.parametrize("prefix_tok,chunk", [(6000, 256), (0, 200), (1500, 64)])
def test_prefill_chunk(csa2, prefix_tok, chunk):
    dev = "cuda"
    seed = 4
    n_tok = prefix_tok + chunk
    x = gen.latent(n_tok, seed, device=dev)
    k = gen.index_key(n_tok, seed, device=dev)
    n_ent = n_tok // 2
    nib = torch.empty((n_ent, 256), dtype=torch.uint8, device=dev)
    sc = torch.empty((n_ent, 32), dtype=torch.uint8, device=dev)
    k8 = torch.empty((n_ent, 64), dtype=torch.uint8, device=dev)
    ks = torch.empty((n_ent,), dtype=torch.float32, device=dev)
    pe = prefix_tok // 2
    # prefix and chunk encoded by separate calls, as a prefill appends a chunk
    csa2.csa2_quantize_kv(x[:prefix_tok], ratio=2, k_in=k[:prefix_tok], out=[nib[:pe], sc[:pe], k8[:pe], ks[:pe]])
    csa2.csa2_quantize_kv(x[prefix_tok:], ratio=2, k_in=k[prefix_tok:], out=[nib[pe:], sc[pe:], k8[pe:], ks[pe:]])
    kv = csa2.make_kv(nib, sc, k8, ks, n_ent)
    swa_pos0 = max(0, prefix_tok - 127)
    rows = n_tok - swa_pos0
    plan = "FUUUUU"
    layers, host = [], []
    for j, m in enumerate(plan):
        q = gen.attn_query((1, chunk), seed, j, device=dev)
        swa = gen.window_rows(1, rows, seed, j, device=dev)
        d = dict(mode=csa2.MODE_FULL if m == "F" else csa2.MODE_REUSE, q=q, swa=swa)
        h = dict(mode=oracle.FULL if m == "F" else oracle.REUSE, q=gen.bf16_bits(q), swa=gen.bf16_bits(swa))
        if m == "F":
            iq = gen.index_query((1, chunk), seed, j, device=dev)
            d["idx_q"], d["kv"] = iq, kv
            h["idx_q"], h["idx_w"] = iq.cpu().numpy(), None
        layers.append(d)
        host.append(h)
    ws = csa2.Workspace(1, chunk, n_ent)
    st = csa2.State(1, chunk)
    outs = csa2.csa2_run_group(ws, st, layers, [prefix_tok], [n_ent], [swa_pos0], ratio=2)
    torch.cuda.synchronize()
    rn, rs, rk, rks = oracle.quantize_kv(x.cpu().numpy(), 2, k.cpu().numpy())
    assert np.array_equal(nib.cpu().numpy(), rn) and np.array_equal(sc.cpu().numpy(), rs)
    assert np.array_equal(k8.cpu().numpy(), rk) and np.array_equal(ks.cpu().numpy(), rks)
    host[0]["kv"] = dict(nib=[rn], scale=[rs], k8=[rk], ks=[rks])
    ref_st = oracle.new_state()
    ref = oracle.run_group(host, ref_st, [prefix_tok], [n_ent], [swa_pos0], ratio=2)
    gi = st.indices.cpu().numpy()
    iq = host[0]["idx_q"]
    n_same = 0
    for i in range(chunk):
        nv = oracle.visible_entries(prefix_tok + i, 2)
        s = oracle.scores(iq[0, i], None, rk[:nv], rks[:nv])
        check_topk(gi[0, i], ref_st["indices"][0, i], s, 512, nv, f"query {i}")
        if np.array_equal(gi[0, i], ref_st["indices"][0, i]):
            n_same += 1
            for j in range(len(plan)):
                check_close(outs[j][0, i].cpu().numpy(), ref[j][0, i], f"layer {j} query {i}")
        else:  # a tie: the oracle's attention on the GPU's own index set
            for j in range(len(plan)):
                r = oracle.sparse_swa_attention(host[j]["q"][0, i], rn, rs, gi[0, i], host[j]["swa"][0], swa_pos0,
                                                prefix_tok + i)
                check_close(outs[j][0, i].cpu().numpy(), r, f"layer {j} query {i}")
    assert n_same >= chunk * 0.9
