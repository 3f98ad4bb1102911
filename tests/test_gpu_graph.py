"""A decode group step captured into a HIP graph (as bench.py times it):
every replay, with eager work and synchronisations between replays, gives
the eager call's outputs and indices bit for bit."""

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


def test_group_graph_replays_match_eager(csa2):
    dev = "cuda"
    n_entries = [6001, 4099, 20000]
    stride = 20000
    B = len(n_entries)
    x = gen.latent(B * stride, 51, device=dev)
    k = gen.index_key(B * stride, 51, device=dev)
    nib, sc, k8, ks = csa2.csa2_quantize_kv(x, k_in=k)
    kv = csa2.make_kv(nib, sc, k8, ks, stride)
    q_pos0 = [n - 1 for n in n_entries]
    swa_pos0 = [p - 127 for p in q_pos0]
    mode = {"F": csa2.MODE_FULL, "R": csa2.MODE_REINDEX, "U": csa2.MODE_REUSE}

    def layers(plan, layer0):
        ls = []
        for j, m in enumerate(plan):
            d = dict(mode=mode[m], q=gen.attn_query((B, 1), 51, layer0 + j, device=dev),
                     swa=gen.window_rows(B, 128, 51, layer0 + j, device=dev),
                     out=torch.empty((B, 1, 16, 512), dtype=torch.float32, device=dev))
            if m in "FR":
                d["idx_q"] = gen.index_query((B, 1), 51, layer0 + j, device=dev)
            if m == "F":
                d["kv"] = kv
            ls.append(d)
        return ls

    runs = [layers("FUUU", 0), layers("RUUU", 10)]
    ws = csa2.Workspace(B, 1, stride)
    st = csa2.State(B, 1)

    def step():
        for ls in runs:
            csa2.csa2_run_group(ws, st, ls, q_pos0, n_entries, swa_pos0)

    step()
    torch.cuda.synchronize()
    ref_out = [[L["out"].clone() for L in ls] for ls in runs]
    ref_idx = st.indices.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for ls in runs:  # eager work between replays: poison the outputs
            for L in ls:
                L["out"].fill_(float("nan"))
        st.indices.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.indices, ref_idx), f"replay {rep}: indices"
        for r, ls in enumerate(runs):
            for j, L in enumerate(ls):
                assert torch.equal(L["out"], ref_out[r][j]), f"replay {rep}: run {r} layer {j}"
    assert ws.fallbacks() == 0
