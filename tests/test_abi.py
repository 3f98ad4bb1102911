"""CPU tests of the C ABI: the library loads, exports every function the
header declares, its struct layouts match the binding, and every validation
error is reported before anything is enqueued (no GPU is touched: each call
below fails validation, which runs before the first HIP call)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def m():
    import sparse_attention_decode_fp4_amd as mod
    return mod


def _declared():
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_\w+)\s*\(", src)))


def test_exports_every_declared_function(m):
    names = _declared()
    assert len(names) >= 12
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_struct_layouts(m):
    assert m.lib.csa2_abi_version() == m.ABI_VERSION
    for i, st in enumerate(m._STRUCTS):
        assert m.lib.csa2_struct_size(i) == ctypes.sizeof(st)
    assert m.lib.csa2_struct_size(99) == 0


def test_workspace_sizes(m):
    assert m.lib.csa2_workspace_bytes(0, 1, 10) == 0
    small = m.lib.csa2_workspace_bytes(1, 1, 4096)
    big = m.lib.csa2_workspace_bytes(16, 1, 131072)
    assert 0 < small < big
    assert m.lib.csa2_workspace_init(None, 1024, None) == m.ERR_WORKSPACE
    assert m.lib.csa2_workspace_init(ctypes.c_void_p(0x1001), 1024, None) == m.ERR_WORKSPACE
    n = ctypes.c_uint32(7)
    assert m.lib.csa2_workspace_fallbacks(None, ctypes.byref(n), None) == m.ERR_ARG
    assert m.lib.csa2_workspace_fallbacks(ctypes.c_void_p(0x10000000), None, None) == m.ERR_ARG
    assert m.lib.csa2_workspace_fallbacks(ctypes.c_void_p(0x10000001), ctypes.byref(n), None) == m.ERR_WORKSPACE
    assert n.value == 7


FAKE = 0x10000000  # aligned, never dereferenced: every call here fails validation first


def _p(off=0):
    return ctypes.c_void_p(FAKE + off)


def test_quantize_errors(m):
    q = m.lib.csa2_quantize_kv
    assert q(_p(), 4, 512, 3, _p(), _p(), None, 0, None, None, None) == m.ERR_ARG       # ratio
    assert q(_p(), 3, 512, 2, _p(), _p(), None, 0, None, None, None) == m.ERR_ARG       # odd tokens
    assert q(_p(), 4, 500, 1, _p(), _p(), None, 0, None, None, None) == m.ERR_ARG       # ld < 512
    assert q(_p(4), 4, 512, 1, _p(), _p(), None, 0, None, None, None) == m.ERR_ARG      # misaligned x
    assert q(None, 4, 512, 1, _p(), _p(), None, 0, None, None, None) == m.ERR_ARG       # null x
    assert q(_p(), 4, 512, 1, _p(), _p(), _p(), 64, None, None, None) == m.ERR_ARG      # k_in without k8
    assert q(None, 0, 512, 1, None, None, None, 0, None, None, None) == m.OK            # empty: nothing to do
    q(_p(), 4, 512, 5, _p(), _p(), None, 0, None, None, None)
    assert b"ratio" in m.lib.csa2_last_error()


def _index_args(m, **kw):
    a = m.IndexArgs()
    qp = (ctypes.c_int64 * 2)(99, 99)
    ne = (ctypes.c_int64 * 2)(100, 100)
    a.kind, a.batch, a.n_q, a.ratio = m.INDEX_FLAT, 2, 1, 1
    a.q_pos0, a.n_entries = ctypes.cast(qp, ctypes.c_void_p), ctypes.cast(ne, ctypes.c_void_p)
    a.idx_q, a.k8, a.kscale, a.k_stride = _p(), _p(), _p(), 100
    a.k, a.n_blocks, a.out_idx = 512, 2048, _p()
    for k, v in kw.items():
        setattr(a, k, v)
    a._keep = (qp, ne)
    return a


def test_index_errors(m):
    f = m.lib.csa2_index_topk
    assert f(None, _p(), 1 << 30, None) == m.ERR_ARG
    assert f(ctypes.byref(_index_args(m, kind=7)), _p(), 1 << 30, None) == m.ERR_ARG
    assert f(ctypes.byref(_index_args(m, k=0)), _p(), 1 << 30, None) == m.ERR_UNSUPPORTED
    assert f(ctypes.byref(_index_args(m, k=4096)), _p(), 1 << 30, None) == m.ERR_UNSUPPORTED
    assert f(ctypes.byref(_index_args(m, ratio=3)), _p(), 1 << 30, None) == m.ERR_ARG
    assert f(ctypes.byref(_index_args(m, k_stride=50)), _p(), 1 << 30, None) == m.ERR_ARG
    assert f(ctypes.byref(_index_args(m, idx_q=_p(8))), _p(), 1 << 30, None) == m.ERR_ARG
    assert f(ctypes.byref(_index_args(m, kind=m.INDEX_HIER)), _p(), 1 << 30, None) == m.ERR_ARG
    assert f(ctypes.byref(_index_args(m, kind=m.INDEX_POOL)), _p(), 1 << 30, None) == m.ERR_ARG
    assert f(ctypes.byref(_index_args(m)), None, 0, None) == m.ERR_WORKSPACE
    assert f(ctypes.byref(_index_args(m)), _p(), 1024, None) == m.ERR_WORKSPACE
    assert f(ctypes.byref(_index_args(m)), _p(16), 1 << 30, None) == m.ERR_WORKSPACE


def test_attention_errors(m):
    f = m.lib.csa2_sparse_swa_attn
    a = m.AttnArgs()
    qp = (ctypes.c_int64 * 1)(300)
    sp = (ctypes.c_int64 * 1)(250)          # window of token 300 starts at 173: rows missing
    a.batch, a.n_q, a.n_idx = 1, 1, 512
    a.q_pos0, a.swa_pos0 = ctypes.cast(qp, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p)
    a.q, a.nib, a.scale, a.idx, a.swa, a.out = _p(), _p(), _p(), _p(), _p(), _p()
    a.swa_rows, a.swa_stride, a.kv_stride = 128, 128, 1000
    assert f(ctypes.byref(a), _p(), 1 << 30, None) == m.ERR_ARG
    assert b"window" in m.lib.csa2_last_error()
    sp[0] = 173
    a.n_idx = 4096
    assert f(ctypes.byref(a), _p(), 1 << 30, None) == m.ERR_UNSUPPORTED
    a.n_idx = 512
    a.q = _p(2)
    assert f(ctypes.byref(a), _p(), 1 << 30, None) == m.ERR_ARG


def test_append_errors(m):
    A = m.AppendArgs
    pos = (ctypes.c_int64 * 2)(5, 7)

    def args(**kw):
        a = A()
        a.batch, a.ratio, a.pos = 2, 1, ctypes.cast(pos, ctypes.c_void_p)
        a.x, a.k_in, a.nib, a.scale, a.k8, a.kscale = _p(), _p(0x1000), _p(0x2000), _p(0x3000), _p(0x4000), _p(0x5000)
        a.stride = 16
        for k, v in kw.items():
            setattr(a, k, v)
        return ctypes.byref(a)

    ap = m.lib.csa2_append
    assert ap(None, None) == m.ERR_ARG
    assert ap(args(ratio=3), None) == m.ERR_ARG
    assert ap(args(x=None), None) == m.ERR_ARG
    assert ap(args(ratio=2), None) == m.ERR_ARG                         # no pending buffer
    assert ap(args(bk8=_p(0x6000)), None) == m.ERR_ARG                 # bk8 without bkscale
    assert ap(args(x=_p(4)), None) == m.ERR_ARG                        # misaligned
    assert ap(args(stride=6), None) == m.ERR_ARG                       # entry 7 past the stride
    assert ap(args(swa=_p(0x7000), swa_ring=100, swa_stride=100), None) == m.ERR_ARG  # ring < 128
    big = (ctypes.c_int64 * 2)(5, 1 << 23)
    assert ap(args(pos=ctypes.cast(big, ctypes.c_void_p), stride=1 << 24), None) == m.ERR_UNSUPPORTED
    neg = (ctypes.c_int64 * 2)(5, -1)
    assert ap(args(pos=ctypes.cast(neg, ctypes.c_void_p)), None) == m.ERR_ARG
    zero = A()
    assert ap(ctypes.byref(zero), None) == m.OK                         # batch 0: nothing to do


def test_group_state_errors(m):
    st = m.GroupState()
    st.indices = _p()
    layer = (m.Layer * 1)()
    layer[0].mode, layer[0].q, layer[0].swa, layer[0].out = m.MODE_REUSE, _p(), _p(), _p()
    g = m.GroupArgs()
    qp, ne, sp = (ctypes.c_int64 * 1)(999), (ctypes.c_int64 * 1)(1000), (ctypes.c_int64 * 1)(872)
    g.batch, g.n_q, g.ratio = 1, 1, 1
    g.q_pos0, g.n_entries, g.swa_pos0 = (ctypes.cast(x, ctypes.c_void_p) for x in (qp, ne, sp))
    g.swa_stride, g.swa_rows, g.softmax_scale, g.n_layers, g.layers = 128, 128, 1.0, 1, layer
    f = m.lib.csa2_run_group
    assert f(ctypes.byref(g), ctypes.byref(st), _p(), 1 << 30, None) == m.ERR_STATE
    layer[0].mode = m.MODE_REINDEX
    layer[0].idx_q = _p()
    assert f(ctypes.byref(g), ctypes.byref(st), _p(), 1 << 30, None) == m.ERR_STATE
    layer[0].mode = m.MODE_FULL          # FULL without kv
    assert f(ctypes.byref(g), ctypes.byref(st), _p(), 1 << 30, None) == m.ERR_ARG
    st.has_full, st.has_indices, st.batch, st.n_q = 1, 1, 2, 1   # state of another batch size
    layer[0].mode = m.MODE_REUSE
    assert f(ctypes.byref(g), ctypes.byref(st), _p(), 1 << 30, None) == m.ERR_STATE
    assert f(None, ctypes.byref(st), _p(), 1 << 30, None) == m.ERR_ARG


def test_flat_full_drops_an_earlier_pool(m):
    """A state whose pool came from an earlier hierarchical Full layer: a
    flat Full layer replaces the KV, so a pool Reindex after it has no pool
    of that KV to rank and is refused before anything is launched."""
    st = m.GroupState()
    st.indices, st.pool = _p(), _p(0x100000)
    st.has_full, st.has_indices, st.has_pool, st.batch, st.n_q = 1, 1, 1, 1, 1
    kv = m.KV()
    kv.nib, kv.scale, kv.k8, kv.kscale, kv.stride = _p(0x200000), _p(0x300000), _p(0x400000), _p(0x500000), 1000
    layers = (m.Layer * 2)()
    for l in layers:
        l.q, l.swa, l.out, l.idx_q = _p(0x600000), _p(0x700000), _p(0x800000), _p(0x900000)
    layers[0].mode, layers[0].kv = m.MODE_FULL, ctypes.pointer(kv)
    layers[1].mode = m.MODE_REINDEX
    g = m.GroupArgs()
    qp, ne, sp = (ctypes.c_int64 * 1)(999), (ctypes.c_int64 * 1)(1000), (ctypes.c_int64 * 1)(872)
    g.batch, g.n_q, g.ratio = 1, 1, 1
    g.index_kind, g.reindex_kind = m.INDEX_FLAT, m.INDEX_POOL
    g.q_pos0, g.n_entries, g.swa_pos0 = (ctypes.cast(x, ctypes.c_void_p) for x in (qp, ne, sp))
    g.swa_stride, g.swa_rows, g.softmax_scale, g.n_layers, g.layers = 128, 128, 1.0, 2, layers
    f = m.lib.csa2_run_group
    assert f(ctypes.byref(g), ctypes.byref(st), _p(), 1 << 30, None) == m.ERR_STATE
    assert b"POOL" in m.lib.csa2_last_error()
    assert st.has_pool == 1          # a refused call leaves the state as it was
    # the same Reindex alone still finds the earlier pool valid (its workspace
    # check then fails: nothing is launched either way)
    g.n_layers, g.layers = 1, ctypes.cast(ctypes.byref(layers, ctypes.sizeof(m.Layer)), ctypes.POINTER(m.Layer))
    assert f(ctypes.byref(g), ctypes.byref(st), _p(), 16, None) == m.ERR_WORKSPACE


def test_noalloc_validates_like_run_group_and_rejects_calls_past_its_scratch(m):
    f = m.lib.csa2_run_group_noalloc
    st = m.GroupState()
    st.indices = _p()
    layers = (m.Layer * 1)()
    layers[0].q, layers[0].swa, layers[0].out, layers[0].idx_q = _p(0x600000), _p(0x700000), _p(0x800000), _p(0x900000)
    layers[0].mode = m.MODE_REUSE
    n_q, n_ent = 31, 8_000_000
    g = m.GroupArgs()
    qp, ne = (ctypes.c_int64 * 1)(n_ent - n_q), (ctypes.c_int64 * 1)(n_ent)
    g.batch, g.n_q, g.ratio = 1, n_q, 1
    g.q_pos0, g.n_entries = (ctypes.cast(x, ctypes.c_void_p) for x in (qp, ne))
    g.swa_stride, g.swa_ring, g.softmax_scale, g.n_layers, g.layers = 256, 256, 1.0, 1, layers
    assert f(ctypes.byref(g), ctypes.byref(st), None) == m.ERR_STATE   # Reuse before any Full
    assert f(None, ctypes.byref(st), None) == m.ERR_ARG
    kv = m.KV()
    kv.nib, kv.scale, kv.k8, kv.kscale, kv.stride = _p(0x200000), _p(0x300000), _p(0x400000), _p(0x500000), n_ent
    layers[0].mode, layers[0].kv = m.MODE_FULL, ctypes.pointer(kv)
    # 31 query rows over 8 million entries need far more than the scratch holds
    assert f(ctypes.byref(g), ctypes.byref(st), None) == m.ERR_UNSUPPORTED
    msg = m.lib.csa2_last_error()
    assert b"scratch" in msg and str(32 << 20).encode() in msg
    assert st.has_full == 0 and st.has_indices == 0  # a refused call leaves the state as it was


def test_per_head_key_errors(m):
    f = m.lib.csa2_quantize_head_keys
    assert f(None, 8, 256, 1, _p(), _p(0x100), None) == m.ERR_ARG
    assert f(_p(), 8, 64, 1, _p(), _p(0x100), None) == m.ERR_ARG      # ld_k below 256
    assert f(_p(), 7, 256, 2, _p(), _p(0x100), None) == m.ERR_ARG     # odd token count at ratio 2
    assert f(_p(), 0, 256, 1, None, None, None) == m.OK                # nothing to do
    a = m.IndexArgs()
    qp, ne = (ctypes.c_int64 * 1)(999), (ctypes.c_int64 * 1)(1000)
    a.kind, a.batch, a.n_q, a.ratio, a.k, a.n_blocks = m.INDEX_FLAT, 1, 1, 1, 512, 2048
    a.q_pos0, a.n_entries = ctypes.cast(qp, ctypes.c_void_p), ctypes.cast(ne, ctypes.c_void_p)
    a.idx_q, a.k8, a.kscale, a.out_idx, a.k_stride = _p(), _p(0x1000), _p(0x2000), _p(0x3000), 1000
    a.key_heads = 2
    assert m.lib.csa2_index_topk(ctypes.byref(a), _p(), 1 << 30, None) == m.ERR_ARG
    a.key_heads, a.kind = 4, m.INDEX_HIER
    a.bk8, a.bkscale = _p(0x4000), _p(0x5000)
    assert m.lib.csa2_index_topk(ctypes.byref(a), _p(), 1 << 30, None) == m.ERR_UNSUPPORTED
    a.kind, a.n_q = m.INDEX_FLAT, 32                                   # prefill-sized
    assert m.lib.csa2_index_topk(ctypes.byref(a), _p(), 1 << 30, None) == m.ERR_UNSUPPORTED


def _pages(m, table=None, table_stride=1, page_size=128, pool_entries=1024):
    pg = m.Pages()
    pg.table = _p(0x8000) if table is None else table
    pg.table_stride, pg.page_size, pg.pool_entries = table_stride, page_size, pool_entries
    return pg


def test_paged_cache_errors(m):
    """Page descriptions are checked on the host: page size a power of two
    in 128..65536, a table row long enough for the longest sequence, a pool
    inside CSA2_MAX_ENTRIES, an aligned table; the non-decode index kinds and
    prefill-sized calls refuse paged caches."""
    f = m.lib.csa2_index_topk
    ok = _pages(m)                                  # 100 entries fit one page of 128
    bad = [
        (_pages(m, page_size=64), m.ERR_ARG),       # page below 128 entries
        (_pages(m, page_size=200), m.ERR_ARG),      # not a power of two
        (_pages(m, page_size=1 << 17), m.ERR_ARG),  # above 65536
        (_pages(m, table_stride=0), m.ERR_ARG),
        (_pages(m, pool_entries=0), m.ERR_ARG),
        (_pages(m, pool_entries=1 << 23), m.ERR_ARG),   # past CSA2_MAX_ENTRIES
        (_pages(m, table=_p(0x8002)), m.ERR_ARG),       # misaligned table
    ]
    for pg, code in bad:
        assert f(ctypes.byref(_index_args(m, pages=pg, k_stride=0)), _p(), 1 << 30, None) == code
    ne = (ctypes.c_int64 * 2)(300, 100)             # 300 entries need 3 pages of 128
    a = _index_args(m, pages=_pages(m, table_stride=2), k_stride=0)
    a.n_entries = ctypes.cast(ne, ctypes.c_void_p)
    assert f(ctypes.byref(a), _p(), 1 << 30, None) == m.ERR_ARG
    assert b"table_stride" in m.lib.csa2_last_error()
    assert f(ctypes.byref(_index_args(m, pages=ok, kind=m.INDEX_HIER, bk8=_p(), bkscale=_p())), _p(), 1 << 30,
             None) == m.ERR_UNSUPPORTED
    qp = (ctypes.c_int64 * 2)(99, 99)
    a = _index_args(m, pages=ok, n_q=32)
    a.q_pos0 = ctypes.cast(qp, ctypes.c_void_p)
    assert f(ctypes.byref(a), _p(), 1 << 30, None) == m.ERR_UNSUPPORTED

    # attention: the same field checks
    at = m.AttnArgs()
    qp1, sp1 = (ctypes.c_int64 * 1)(300), (ctypes.c_int64 * 1)(173)
    at.batch, at.n_q, at.n_idx = 1, 1, 512
    at.q_pos0, at.swa_pos0 = ctypes.cast(qp1, ctypes.c_void_p), ctypes.cast(sp1, ctypes.c_void_p)
    at.q, at.nib, at.scale, at.idx, at.swa, at.out = _p(), _p(), _p(), _p(), _p(), _p()
    at.swa_rows, at.swa_stride = 128, 128
    at.pages = _pages(m, page_size=96)
    assert m.lib.csa2_sparse_swa_attn(ctypes.byref(at), _p(), 1 << 30, None) == m.ERR_ARG

    # append: an entry past the sequence's page-table row
    pos = (ctypes.c_int64 * 2)(5, 300)
    ap = m.AppendArgs()
    ap.batch, ap.ratio, ap.pos = 2, 1, ctypes.cast(pos, ctypes.c_void_p)
    ap.x, ap.k_in, ap.nib, ap.scale, ap.k8, ap.kscale = _p(), _p(0x1000), _p(0x2000), _p(0x3000), _p(0x4000), _p(0x5000)
    ap.pages = _pages(m, table_stride=2)            # rows of 2 pages: entries < 256
    assert m.lib.csa2_append(ctypes.byref(ap), None) == m.ERR_ARG
    assert b"page-table row" in m.lib.csa2_last_error()

    # group plan: a paged Full layer with hierarchical indexing
    kv = m.KV()
    kv.nib, kv.scale, kv.k8, kv.kscale = _p(), _p(), _p(), _p()
    kv.bk8, kv.bkscale, kv.pages = _p(), _p(), ok
    layer = (m.Layer * 1)()
    layer[0].mode, layer[0].q, layer[0].swa, layer[0].out = m.MODE_FULL, _p(), _p(), _p()
    layer[0].idx_q, layer[0].kv = _p(), ctypes.pointer(kv)
    g = m.GroupArgs()
    qp2, ne2, sp2 = (ctypes.c_int64 * 1)(99), (ctypes.c_int64 * 1)(100), (ctypes.c_int64 * 1)(0)
    g.batch, g.n_q, g.ratio, g.index_kind = 1, 1, 1, m.INDEX_HIER
    g.q_pos0, g.n_entries, g.swa_pos0 = (ctypes.cast(x, ctypes.c_void_p) for x in (qp2, ne2, sp2))
    g.swa_stride, g.swa_rows, g.softmax_scale, g.n_layers, g.layers = 128, 128, 1.0, 1, layer
    st = m.GroupState()
    st.indices = _p()
    assert m.lib.csa2_run_group(ctypes.byref(g), ctypes.byref(st), _p(), 1 << 30, None) == m.ERR_UNSUPPORTED
