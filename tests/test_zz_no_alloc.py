"""GPU test of csa2_run_group_noalloc (the allocation-free csa2_run_group):
through the C ABI, its outputs and index state equal those of
csa2_run_group with a workspace, bit for bit, on two calls in a row, the
second smaller than the first."""

import pytest
import torch

import csa2_inputs as gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_decode_fp4_amd as m
    return m


def _inputs(csa2, seed, batch, n_ent, plan):
    dev = "cuda"
    x = gen.latent(batch * n_ent, seed, device=dev)
    k = gen.index_key(batch * n_ent, seed, device=dev)
    nib, sc, k8, ks = csa2.csa2_quantize_kv(x, k_in=k)
    kv = csa2.make_kv(nib, sc, k8, ks, n_ent)
    rows = 129
    layers = []
    for j, mode in enumerate(plan):
        L = {"mode": {"F": csa2.MODE_FULL, "R": csa2.MODE_REINDEX, "U": csa2.MODE_REUSE}[mode],
             "q": gen.attn_query((batch, 1), seed, j, device=dev),
             "swa": gen.window_rows(batch, rows, seed, j, device=dev)}
        if mode != "U":
            L["idx_q"] = gen.index_query((batch, 1), seed, j, device=dev)
        if mode == "F":
            L["kv"] = kv
        layers.append(L)
    q_pos0 = [n_ent - 1] * batch
    swa_pos0 = [n_ent - 129] * batch
    return layers, q_pos0, [n_ent] * batch, swa_pos0, (nib, sc, k8, ks)


def _with_outs(layers, batch):
    return [dict(L, out=torch.full((batch, 1, 16, 512), float("nan"), device="cuda")) for L in layers]


@pytest.mark.parametrize("calls", [[(16, 131072, "FUUU"), (3, 5000, "FU")],
                                   [(4, 40000, "FRUU"), (1, 3000, "F")]])
def test_noalloc_equals_run_group(csa2, calls):
    for seed, (batch, n_ent, plan) in enumerate(calls):
        print(f"noalloc: batch {batch}, {n_ent} entries, plan {plan}", flush=True)
        layers, q_pos0, n_entries, swa_pos0, keep = _inputs(csa2, 100 + seed, batch, n_ent, plan)
        ws = csa2.Workspace(batch, 1, n_ent)
        st_ref, st = csa2.State(batch, 1), csa2.State(batch, 1)
        ref = csa2.csa2_run_group(ws, st_ref, _with_outs(layers, batch), q_pos0, n_entries, swa_pos0)
        torch.cuda.synchronize()
        outs = _with_outs(layers, batch)
        got = csa2.csa2_run_group_noalloc(st, outs, q_pos0, n_entries, swa_pos0)
        torch.cuda.synchronize()
        assert all(g.data_ptr() == o["out"].data_ptr() for g, o in zip(got, outs))  # written in place
        assert torch.equal(st.indices, st_ref.indices)
        for l, (a, b) in enumerate(zip(got, ref)):
            assert torch.isfinite(a).all(), f"layer {l}"
            assert torch.equal(a, b), f"layer {l}: max diff {(a - b).abs().max().item()}"
        del ws, keep
