"""Python binding of libcsa2, the CSA2 sparse-attention step with an FP4 KV cache.

Argument marshalling only: every step runs in the HIP kernels of libcsa2.so
(built in place by build.py for gfx950).  Importing this package loads the
library and fails loudly when it is missing; there is no CPU fallback.

The call names follow the C ABI in include/csa2.h.  Tensors are torch tensors
on the GPU; the binding allocates outputs when they are not given, checks
dtypes, shapes and contiguity, and passes raw pointers plus the current
stream.  bf16 tensors are passed by their bit patterns.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

D_LATENT, NIB_BYTES, SCALE_BYTES = 512, 256, 32
D_INDEX, H_INDEX, H_ATTN = 64, 4, 16
TOP_K, SWA, BLOCK, N_BLOCKS, MAX_K = 512, 128, 8, 2048, 2048
INDEX_FLAT, INDEX_HIER, INDEX_POOL, INDEX_FLAT_POOL = 0, 1, 2, 3
MODE_FULL, MODE_REINDEX, MODE_REUSE = 0, 1, 2
OK, ERR_ARG, ERR_UNSUPPORTED, ERR_STATE, ERR_WORKSPACE, ERR_HIP = range(6)
(K_QUANTIZE, K_BLOCK_KEYS, K_INDEX_SCAN, K_INDEX_SAMPLE, K_INDEX_SELECT, K_ATTENTION,
 K_PREFILL_SAMPLE, K_ATTENTION_MERGE, K_PREFILL_FILTER, K_PREFILL_SELECT, K_APPEND) = range(11)
KERNEL_NAMES = ["quantize", "block_keys", "index_scan", "index_sample", "index_select", "attention",
                "prefill_sample", "attention_merge", "prefill_filter", "prefill_select", "append"]
ABI_VERSION = 4

_p = ctypes.c_void_p
_i32, _i64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float


class Pages(ctypes.Structure):
    """csa2_pages: a paged cache's page table (a zero table: contiguous)."""
    _fields_ = [("table", _p), ("table_stride", _i64), ("pool_entries", _i64), ("page_size", _i32)]


class IndexArgs(ctypes.Structure):
    _fields_ = [("kind", _i32), ("batch", _i32), ("n_q", _i32), ("ratio", _i32),
                ("q_pos0", _p), ("n_entries", _p), ("idx_q", _p), ("idx_w", _p),
                ("k8", _p), ("kscale", _p), ("k_stride", _i64),
                ("bk8", _p), ("bkscale", _p), ("bk_stride", _i64),
                ("cand", _p), ("n_cand", _i32), ("k", _i32), ("n_blocks", _i32),
                ("out_idx", _p), ("out_pool", _p), ("pages", Pages), ("key_heads", _i32)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("batch", _i32), ("n_q", _i32), ("n_idx", _i32), ("q_pos0", _p),
                ("q", _p), ("nib", _p), ("scale", _p), ("kv_stride", _i64), ("idx", _p),
                ("swa", _p), ("swa_stride", _i64), ("swa_pos0", _p), ("swa_rows", _i64),
                ("softmax_scale", _f32), ("out", _p), ("swa_ring", _i64), ("pages", Pages)]


class KV(ctypes.Structure):
    _fields_ = [("nib", _p), ("scale", _p), ("k8", _p), ("kscale", _p), ("stride", _i64),
                ("bk8", _p), ("bkscale", _p), ("bk_stride", _i64), ("pages", Pages), ("key_heads", _i32)]


class Layer(ctypes.Structure):
    _fields_ = [("mode", _i32), ("q", _p), ("swa", _p), ("idx_q", _p), ("idx_w", _p),
                ("kv", ctypes.POINTER(KV)), ("out", _p)]


class GroupState(ctypes.Structure):
    _fields_ = [("kv", KV), ("indices", _p), ("pool", _p), ("has_full", _i32),
                ("has_indices", _i32), ("has_pool", _i32), ("batch", _i32), ("n_q", _i32)]


class GroupArgs(ctypes.Structure):
    _fields_ = [("batch", _i32), ("n_q", _i32), ("ratio", _i32), ("index_kind", _i32),
                ("reindex_kind", _i32), ("q_pos0", _p), ("n_entries", _p), ("swa_pos0", _p),
                ("swa_stride", _i64), ("swa_rows", _i64), ("softmax_scale", _f32),
                ("n_layers", _i32), ("layers", ctypes.POINTER(Layer)), ("swa_ring", _i64)]


class AppendArgs(ctypes.Structure):
    _fields_ = [("batch", _i32), ("ratio", _i32), ("pos", _p), ("x", _p), ("k_in", _p),
                ("nib", _p), ("scale", _p), ("k8", _p), ("kscale", _p), ("stride", _i64),
                ("bk8", _p), ("bkscale", _p), ("bk_stride", _i64), ("pending", _p),
                ("swa", _p), ("swa_stride", _i64), ("swa_ring", _i64), ("pages", Pages)]


_STRUCTS = [IndexArgs, AttnArgs, KV, Layer, GroupState, GroupArgs, AppendArgs, Pages]


class Csa2Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libcsa2 status {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python sparse_attention_decode_fp4_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    sigs = {
        "csa2_abi_version": (_i32, []),
        "csa2_last_error": (ctypes.c_char_p, []),
        "csa2_struct_size": (ctypes.c_size_t, [_i32]),
        "csa2_workspace_bytes": (ctypes.c_size_t, [_i32, _i32, _i64]),
        "csa2_workspace_init": (_i32, [_p, ctypes.c_size_t, _p]),
        "csa2_workspace_fallbacks": (_i32, [_p, ctypes.POINTER(ctypes.c_uint32), _p]),
        "csa2_quantize_kv": (_i32, [_p, _i64, _i64, _i32, _p, _p, _p, _i64, _p, _p, _p]),
        "csa2_build_block_keys": (_i32, [_p, _p, _i32, _p, _i64, _p, _p, _i64, _p]),
        "csa2_quantize_head_keys": (_i32, [_p, _i64, _i64, _i32, _p, _p, _p]),
        "csa2_index_topk": (_i32, [ctypes.POINTER(IndexArgs), _p, ctypes.c_size_t, _p]),
        "csa2_sparse_swa_attn": (_i32, [ctypes.POINTER(AttnArgs), _p, ctypes.c_size_t, _p]),
        "csa2_run_group": (_i32, [ctypes.POINTER(GroupArgs), ctypes.POINTER(GroupState), _p,
                                  ctypes.c_size_t, _p]),
        "csa2_run_group_noalloc": (_i32, [ctypes.POINTER(GroupArgs), ctypes.POINTER(GroupState), _p]),
        "csa2_append": (_i32, [ctypes.POINTER(AppendArgs), _p]),
        "csa2_profile_enable": (_i32, [_i32]),
        "csa2_profile_reset": (_i32, []),
        "csa2_profile_read": (_i32, [_i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    if lib.csa2_abi_version() != ABI_VERSION:
        raise ImportError("libcsa2 ABI version mismatch")
    for i, st in enumerate(_STRUCTS):
        if lib.csa2_struct_size(i) != ctypes.sizeof(st):
            raise ImportError(f"struct layout mismatch for {st.__name__}")
    return lib


lib = _load()


def _check(rc):
    if rc != OK:
        raise Csa2Error(rc, lib.csa2_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _host_i64(values):
    arr = (ctypes.c_int64 * len(values))(*[int(v) for v in values])
    return arr


def _need(t, dtype, name, device=True):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t


def _opt(t, dtype, name):
    """_need for an optional tensor (None passes)."""
    if t is not None:
        _need(t, dtype, name)
    return t


def _bits16(t, name):
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    _need(t, torch.int16, name)
    return t


# --------------------------------------------------------------------- workspace
class Workspace:
    """Caller-owned scratch memory of libcsa2, zeroed once (csa2_workspace_init)."""

    def __init__(self, max_batch, max_n_q, max_entries, device="cuda", stream=None):
        n = lib.csa2_workspace_bytes(int(max_batch), int(max_n_q), int(max_entries))
        if n == 0:
            raise ValueError("invalid workspace sizes")
        self.nbytes = int(n)
        self.buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.buf.data_ptr()) % 256
        self.ptr = ctypes.c_void_p(self.buf.data_ptr() + off)
        _check(lib.csa2_workspace_init(self.ptr, self.nbytes, _stream(stream)))

    def fallbacks(self, stream=None):
        """Query rows whose top-k took the exact recompute since the workspace
        was zeroed (waits for the stream)."""
        n = ctypes.c_uint32(0)
        _check(lib.csa2_workspace_fallbacks(self.ptr, ctypes.byref(n), _stream(stream)))
        return int(n.value)

    def reset(self, stream=None):
        """Zero the workspace, the fallback counter included."""
        _check(lib.csa2_workspace_init(self.ptr, self.nbytes, _stream(stream)))


def csa2_workspace_bytes(max_batch, max_n_q, max_entries):
    return int(lib.csa2_workspace_bytes(int(max_batch), int(max_n_q), int(max_entries)))


# --------------------------------------------------------------------- encoders
def csa2_quantize_kv(x, ratio=1, k_in=None, out=None, stream=None):
    """Encode tokens x (float32 [n_tok, >=512]) into FP4 entries; with k_in
    (float32 [n_tok, >=64]) also the fp8 indexer keys.  Returns
    (nib u8[n, 256], scale u8[n, 32]) or (nib, scale, k8 u8[n, 64], kscale f32[n])."""
    _need(x, torch.float32, "x")
    n_tok = x.shape[0]
    n = n_tok // ratio
    dev = x.device
    if out is None:
        out = [torch.empty((n, NIB_BYTES), dtype=torch.uint8, device=dev),
               torch.empty((n, SCALE_BYTES), dtype=torch.uint8, device=dev)]
        if k_in is not None:
            out += [torch.empty((n, D_INDEX), dtype=torch.uint8, device=dev),
                    torch.empty((n,), dtype=torch.float32, device=dev)]
    nib, scale = _need(out[0], torch.uint8, "nib"), _need(out[1], torch.uint8, "scale")
    k8 = _need(out[2], torch.uint8, "k8") if k_in is not None else None
    ks = _need(out[3], torch.float32, "kscale") if k_in is not None else None
    if k_in is not None:
        _need(k_in, torch.float32, "k_in")
        if k_in.shape[0] != n_tok:
            raise ValueError("k_in must have as many rows as x")
    _check(lib.csa2_quantize_kv(_ptr(x), n_tok, x.shape[1], ratio, _ptr(nib), _ptr(scale),
                                _ptr(k_in), 0 if k_in is None else k_in.shape[1], _ptr(k8), _ptr(ks),
                                _stream(stream)))
    return tuple(out)


def csa2_quantize_head_keys(k_in, ratio=1, out=None, stream=None):
    """Per-head indexer keys: k_in float32 [n_tok, 4, 64] (or [n_tok, >=256])
    -> (k8 u8[n, 4, 64], kscale f32[n]), one scale per entry over its heads."""
    _need(k_in, torch.float32, "k_in")
    k2 = k_in.reshape(k_in.shape[0], -1)
    n_tok = k2.shape[0]
    n = n_tok // ratio
    if out is None:
        out = [torch.empty((n, H_INDEX, D_INDEX), dtype=torch.uint8, device=k_in.device),
               torch.empty((n,), dtype=torch.float32, device=k_in.device)]
    _need(out[0], torch.uint8, "k8")
    _need(out[1], torch.float32, "kscale")
    _check(lib.csa2_quantize_head_keys(_ptr(k2), n_tok, k2.shape[1], ratio, _ptr(out[0]), _ptr(out[1]),
                                       _stream(stream)))
    return tuple(out)


def csa2_append(x, k_in, pos, nib, scale, k8, kscale, stride, *, ratio=1, bk8=None, bkscale=None,
                bk_stride=0, pending=None, swa=None, swa_ring=0, pages=None, stream=None):
    """One decode step's write side: token pos[b] of sequence b (x float32
    [batch, 512], k_in float32 [batch, 64]) goes into the cache (sequence b
    at entry offset b * stride), its block key (bk8 / bkscale, optional) and
    the window ring swa (bf16 [batch, swa_ring, 512], optional).  Ratio 2
    holds even tokens in pending (float32 [batch, 576]).  With pages
    (make_pages) the cache arrays are pools and stride is not read."""
    _need(x, torch.float32, "x")
    _need(k_in, torch.float32, "k_in")
    for t, dt, nm in ((nib, torch.uint8, "nib"), (scale, torch.uint8, "scale"), (k8, torch.uint8, "k8"),
                      (kscale, torch.float32, "kscale")):
        _need(t, dt, nm)
    _opt(bk8, torch.uint8, "bk8")
    _opt(bkscale, torch.float32, "bkscale")
    _opt(pending, torch.float32, "pending")
    batch = x.shape[0]
    a = AppendArgs()
    a.batch, a.ratio = batch, ratio
    pp = _host_i64(pos)
    a.pos = ctypes.cast(pp, _p)
    a.x, a.k_in = _ptr(x), _ptr(k_in)
    a.nib, a.scale, a.k8, a.kscale, a.stride = _ptr(nib), _ptr(scale), _ptr(k8), _ptr(kscale), stride
    a.bk8, a.bkscale, a.bk_stride = _ptr(bk8), _ptr(bkscale), bk_stride
    a.pending = _ptr(pending)
    _set_pages(a, pages)
    sb = None
    if swa is not None:
        sb = _bits16(swa, "swa")
        a.swa, a.swa_stride, a.swa_ring = _ptr(sb), swa.shape[1], swa_ring
    _check(lib.csa2_append(ctypes.byref(a), _stream(stream)))


def csa2_build_block_keys(k8, kscale, n_entries, k_stride, bk8=None, bkscale=None, bk_stride=None,
                          stream=None):
    """Block keys of batch = len(n_entries) sequences stored k_stride entries apart."""
    _need(k8, torch.uint8, "k8")
    _need(kscale, torch.float32, "kscale")
    batch = len(n_entries)
    if bk_stride is None:
        bk_stride = (k_stride + BLOCK - 1) // BLOCK
    if bk8 is None:
        bk8 = torch.empty((batch * bk_stride, D_INDEX), dtype=torch.uint8, device=k8.device)
        bkscale = torch.empty((batch * bk_stride,), dtype=torch.float32, device=k8.device)
    ne = _host_i64(n_entries)
    _check(lib.csa2_build_block_keys(_ptr(k8), _ptr(kscale), batch, ne, k_stride, _ptr(bk8),
                                     _ptr(bkscale), bk_stride, _stream(stream)))
    return bk8, bkscale


def make_pages(table, page_size, pool_entries):
    """A paged cache's page table: table int32 [batch, table_stride] of page
    indices (position j of sequence b is pool entry table[b, j // page_size]
    * page_size + j % page_size of the nib/scale/k8/kscale pools)."""
    _need(table, torch.int32, "table")
    pg = Pages()
    pg.table, pg.table_stride, pg.pool_entries, pg.page_size = _ptr(table), table.shape[-1], pool_entries, page_size
    pg._table = table
    return pg


def _set_pages(a, pages):
    if pages is not None:
        a.pages = pages


# --------------------------------------------------------------------- indexer
def csa2_index_topk(ws, idx_q, k8, kscale, n_entries, q_pos0, k_stride, *, kind=INDEX_FLAT,
                    ratio=1, idx_w=None, bk8=None, bkscale=None, bk_stride=0, cand=None,
                    k=TOP_K, n_blocks=N_BLOCKS, out_idx=None, out_pool=None, want_pool=False,
                    pages=None, key_heads=1, stream=None):
    """Top-k positions per query.  idx_q u8 [batch, n_q, 4, 64]; returns
    out_idx int32 [batch, n_q, k] (and the pool for HIER or FLAT_POOL when
    want_pool; FLAT_POOL always makes one).  With pages (make_pages)
    k8/kscale are pools and k_stride is not read."""
    _need(idx_q, torch.uint8, "idx_q")
    _need(k8, torch.uint8, "k8")
    _need(kscale, torch.float32, "kscale")
    _opt(idx_w, torch.float32, "idx_w")
    _opt(bk8, torch.uint8, "bk8")
    _opt(bkscale, torch.float32, "bkscale")
    _opt(cand, torch.int32, "cand")
    _opt(out_idx, torch.int32, "out_idx")
    _opt(out_pool, torch.int32, "out_pool")
    batch, n_q = idx_q.shape[0], idx_q.shape[1]
    dev = idx_q.device
    if out_idx is None:
        out_idx = torch.empty((batch, n_q, k), dtype=torch.int32, device=dev)
    if (kind == INDEX_FLAT_POOL or (kind == INDEX_HIER and want_pool)) and out_pool is None:
        out_pool = torch.empty((batch, n_q, n_blocks * BLOCK), dtype=torch.int32, device=dev)
    a = IndexArgs()
    a.kind, a.batch, a.n_q, a.ratio = kind, batch, n_q, ratio
    qp, ne = _host_i64(q_pos0), _host_i64(n_entries)
    a.q_pos0, a.n_entries = ctypes.cast(qp, _p), ctypes.cast(ne, _p)
    a.idx_q, a.idx_w = _ptr(idx_q), _ptr(idx_w)
    a.k8, a.kscale, a.k_stride = _ptr(k8), _ptr(kscale), k_stride
    a.bk8, a.bkscale, a.bk_stride = _ptr(bk8), _ptr(bkscale), bk_stride
    a.cand = _ptr(cand)
    a.n_cand = 0 if cand is None else cand.shape[-1]
    a.k, a.n_blocks = k, n_blocks
    a.out_idx, a.out_pool = _ptr(out_idx), _ptr(out_pool)
    a.key_heads = key_heads
    _set_pages(a, pages)
    _check(lib.csa2_index_topk(ctypes.byref(a), ws.ptr, ws.nbytes, _stream(stream)))
    return (out_idx, out_pool) if want_pool else out_idx


# --------------------------------------------------------------------- attention
def csa2_sparse_swa_attn(ws, q, nib, scale, idx, swa, q_pos0, swa_pos0, kv_stride, *,
                         softmax_scale=1.0, out=None, swa_ring=0, pages=None, stream=None):
    """q bf16 [batch, n_q, 16, 512]; idx int32 [batch, n_q, n_idx]; swa bf16
    [batch, rows, 512] (row r = token swa_pos0[b] + r; with swa_ring > 0 a
    ring, token t at row t % swa_ring, swa_pos0 unused) -> float32 [batch, n_q, 16, 512]."""
    qb = _bits16(q, "q")
    sb = _bits16(swa, "swa")
    _need(idx, torch.int32, "idx")
    _need(nib, torch.uint8, "nib")
    _need(scale, torch.uint8, "scale")
    batch, n_q = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((batch, n_q, H_ATTN, D_LATENT), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    a = AttnArgs()
    a.batch, a.n_q, a.n_idx = batch, n_q, idx.shape[-1]
    qp = _host_i64(q_pos0)
    sp = _host_i64(swa_pos0 if swa_pos0 is not None else [0] * batch)
    a.q_pos0, a.swa_pos0 = ctypes.cast(qp, _p), ctypes.cast(sp, _p)
    a.q, a.nib, a.scale, a.kv_stride = _ptr(qb), _ptr(nib), _ptr(scale), kv_stride
    a.idx, a.swa, a.swa_stride, a.swa_rows = _ptr(idx), _ptr(sb), swa.shape[1], swa.shape[1]
    a.softmax_scale, a.out, a.swa_ring = softmax_scale, _ptr(out), swa_ring
    _set_pages(a, pages)
    _check(lib.csa2_sparse_swa_attn(ctypes.byref(a), ws.ptr, ws.nbytes, _stream(stream)))
    return out


# --------------------------------------------------------------------- group plan
class State:
    """A csa2_group_state plus the device buffers it points at."""

    def __init__(self, batch, n_q, device="cuda", with_pool=False):
        self.indices = torch.full((batch, n_q, TOP_K), -1, dtype=torch.int32, device=device)
        self.pool = (torch.full((batch, n_q, N_BLOCKS * BLOCK), -1, dtype=torch.int32, device=device)
                     if with_pool else None)
        self.c = GroupState()
        self.c.indices = _ptr(self.indices)
        self.c.pool = _ptr(self.pool)
        self._keep = []  # tensors the stored KV pointers refer to


def make_kv(nib, scale, k8, kscale, stride, bk8=None, bkscale=None, bk_stride=0, pages=None, key_heads=1):
    for t, dt, nm in ((nib, torch.uint8, "nib"), (scale, torch.uint8, "scale"), (k8, torch.uint8, "k8"),
                      (kscale, torch.float32, "kscale")):
        _need(t, dt, nm)
    _opt(bk8, torch.uint8, "bk8")
    _opt(bkscale, torch.float32, "bkscale")
    kv = KV()
    kv.nib, kv.scale, kv.k8, kv.kscale, kv.stride = _ptr(nib), _ptr(scale), _ptr(k8), _ptr(kscale), stride
    kv.key_heads = key_heads
    kv.bk8, kv.bkscale, kv.bk_stride = _ptr(bk8), _ptr(bkscale), bk_stride
    _set_pages(kv, pages)
    kv._tensors = (nib, scale, k8, kscale, bk8, bkscale, pages)
    return kv


def csa2_run_group(ws, state, layers, q_pos0, n_entries, swa_pos0, *, ratio=1,
                   index_kind=INDEX_FLAT, reindex_kind=INDEX_FLAT, softmax_scale=1.0, swa_ring=0,
                   stream=None):
    """Run a plan.  layers: list of dicts {mode, q, swa, idx_q?, idx_w?, kv? (make_kv), out?}.
    Returns the float32 outputs [batch, n_q, 16, 512], one per layer."""
    return _group(ws, state, layers, q_pos0, n_entries, swa_pos0, ratio, index_kind, reindex_kind,
                  softmax_scale, swa_ring, stream)


def csa2_run_group_noalloc(state, layers, q_pos0, n_entries, swa_pos0, *, ratio=1,
                           index_kind=INDEX_FLAT, reindex_kind=INDEX_FLAT, softmax_scale=1.0,
                           swa_ring=0, stream=None):
    """csa2_run_group in the library's own device scratch (no workspace).  The
    C call allocates nothing; pass every layer's `out` for a call that makes
    no tensor either."""
    return _group(None, state, layers, q_pos0, n_entries, swa_pos0, ratio, index_kind, reindex_kind,
                  softmax_scale, swa_ring, stream)


def _group(ws, state, layers, q_pos0, n_entries, swa_pos0, ratio, index_kind, reindex_kind,
           softmax_scale, swa_ring, stream):
    n = len(layers)
    arr = (Layer * n)()
    outs, keep = [], []
    batch, n_q = layers[0]["q"].shape[0], layers[0]["q"].shape[1]
    swa_rows = layers[0]["swa"].shape[1]
    for i, L in enumerate(layers):
        q, swa = _bits16(L["q"], "q"), _bits16(L["swa"], "swa")
        if L["swa"].shape[1] != swa_rows:
            raise ValueError("every layer's window buffer must have the same rows")
        out = L.get("out")
        if out is None:
            out = torch.empty((batch, n_q, H_ATTN, D_LATENT), dtype=torch.float32, device=q.device)
        _need(out, torch.float32, "out")
        outs.append(out)
        arr[i].mode = L["mode"]
        arr[i].q, arr[i].swa, arr[i].out = _ptr(q), _ptr(swa), _ptr(out)
        if L["mode"] != MODE_REUSE:
            _need(L["idx_q"], torch.uint8, "idx_q")
            _opt(L.get("idx_w"), torch.float32, "idx_w")
            arr[i].idx_q, arr[i].idx_w = _ptr(L["idx_q"]), _ptr(L.get("idx_w"))
        if L["mode"] == MODE_FULL:
            kv = L["kv"]
            arr[i].kv = ctypes.pointer(kv)
            keep.append(kv)
        keep += [q, swa]
    a = GroupArgs()
    a.batch, a.n_q, a.ratio = batch, n_q, ratio
    a.index_kind, a.reindex_kind = index_kind, reindex_kind
    qp, ne = _host_i64(q_pos0), _host_i64(n_entries)
    sp = _host_i64(swa_pos0 if swa_pos0 is not None else [0] * batch)
    a.q_pos0, a.n_entries, a.swa_pos0 = ctypes.cast(qp, _p), ctypes.cast(ne, _p), ctypes.cast(sp, _p)
    a.swa_stride, a.swa_rows, a.swa_ring = swa_rows, swa_rows, swa_ring
    a.softmax_scale, a.n_layers, a.layers = softmax_scale, n, arr
    if ws is None:
        _check(lib.csa2_run_group_noalloc(ctypes.byref(a), ctypes.byref(state.c), _stream(stream)))
    else:
        _check(lib.csa2_run_group(ctypes.byref(a), ctypes.byref(state.c), ws.ptr, ws.nbytes,
                                  _stream(stream)))
    if any(L["mode"] == MODE_FULL for L in layers):
        state._keep = [kv for kv in keep if isinstance(kv, KV)]
    return outs


# --------------------------------------------------------------------- timing
def csa2_profile_enable(on=True):
    _check(lib.csa2_profile_enable(1 if on else 0))


def csa2_profile_reset():
    _check(lib.csa2_profile_reset())


def csa2_profile_read(kernel):
    """(total milliseconds, launches) of the recorded launches of one kernel class."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib.csa2_profile_read(int(kernel), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


__all__ = [n for n in dir() if n.startswith("csa2_")] + ["Workspace", "State", "make_kv", "Csa2Error"]
