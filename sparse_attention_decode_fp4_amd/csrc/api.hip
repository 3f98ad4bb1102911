// C ABI of libcsa2: argument validation, workspace carving, launches and the
// Full / Reindex / Reuse state machine.  Every check runs before the first
// HIP call, so an invalid call enqueues nothing (and needs no GPU to fail).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "kernels.hpp"

using namespace csa2;

// Scratch of csa2_run_group_noalloc: device memory the library holds on every
// device it runs on, for the life of the process.  On the host this name is
// a stand-in, not a device address: host code uses only the per-device
// address hipGetSymbolAddress returns for it.  Calls on one device share it.
constexpr size_t kScratchBytes = CSA2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(CSA2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int64_t kMaxEntries = (int64_t)kMaxChunks * kScanChunk;
constexpr size_t kWsAlign = 256;
constexpr int64_t kMaxPartialUnits = 2048;  // (layer,row) x split slots of attention partials

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
  size_t stats, chunk_info, seg_list, blocks, nsel, block_max, row_ksm, partial;
  size_t pf_sample, pf_thresh, pf_count, pf_list, total;
  int32_t max_chunks;     // scan chunks per row covered by the segment buffers
  int64_t max_blocks;     // blocks of 8 items per row covered by block_max
  int64_t partial_units;  // (layer,row) x split slots the attention partials hold
};

// Decode-path buffers cover `rows` query rows of up to `max_items` items;
// prefill-path buffers cover `pf_rows` query rows (0 when unused); the
// attention partials, `partial_units` slots.
WsLayout ws_layout(int64_t rows, int64_t max_items, int64_t pf_rows = 0,
                   int64_t partial_units = kMaxPartialUnits) {
  WsLayout w{};
  w.max_chunks = (int32_t)scan_max_chunks(std::max<int64_t>(max_items, 1));
  w.partial_units = partial_units;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = round_up(off + bytes, kWsAlign); return o; };
  w.stats = take(kWsAlign);  // offset 0 in every layout: the fallback counter
  w.chunk_info = take((size_t)rows * w.max_chunks * 16);
  w.seg_list = take((size_t)rows * w.max_chunks * kSeg * 8);
  w.blocks = take((size_t)rows * CSA2_MAX_K * 4);
  w.nsel = take((size_t)rows * 4);
  w.max_blocks = (std::max<int64_t>(max_items, 1) + 7) / 8;
  w.block_max = take((size_t)rows * w.max_blocks * 4);
  w.row_ksm = take((size_t)rows * 4);
  w.partial = take((size_t)partial_units * kPartFloats * 4);
  w.pf_sample = take((size_t)pf_rows * kPfSample * 4);
  w.pf_thresh = take((size_t)pf_rows * 4);
  w.pf_count = take((size_t)pf_rows * kPfSplits * 4);
  w.pf_list = take((size_t)pf_rows * kPfSplits * kPfSeg * 8);
  w.total = off;
  return w;
}

// Layout for calls of `batch` sequences x `n_q` queries: prefill-sized calls
// use the MFMA indexer and need no per-item decode buffers.
WsLayout ws_for(int32_t batch, int32_t n_q, int64_t max_items, int64_t partial_units = kMaxPartialUnits) {
  const int64_t seqs = std::min(batch, kMaxSeqPerLaunch);
  if (n_q >= kPrefillMinQ) return ws_layout(0, 0, seqs * n_q, partial_units);
  return ws_layout(seqs * n_q, max_items, 0, partial_units);
}

template <typename T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }

int check_workspace(void* ws, size_t ws_bytes, const WsLayout& w) {
  if (!ws) return fail(CSA2_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", w.total);
  if (!aligned(ws, kWsAlign)) return fail(CSA2_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < w.total)
    return fail(CSA2_ERR_WORKSPACE, "workspace has %zu bytes, this call needs %zu", ws_bytes, w.total);
  return CSA2_OK;
}

int64_t visible(int64_t q_pos, int32_t ratio, int64_t n_entries) {
  int64_t v = (q_pos + 1) / ratio;
  v = std::min(v, n_entries);
  return v < 0 ? 0 : v;
}

// ------------------------------------------------------------- indexer
// A page description (csa2_pages): sane fields, and, when the longest
// sequence is known (max_ne >= 0), a table row long enough for it.
int validate_pages(const csa2_pages& pg, int64_t max_ne) {
  if (!pg.table) return CSA2_OK;
  if (!aligned(pg.table, 4)) return fail(CSA2_ERR_ARG, "pages.table must be 4-byte aligned");
  if (pg.page_size < 128 || pg.page_size > 65536 || (pg.page_size & (pg.page_size - 1)))
    return fail(CSA2_ERR_ARG, "pages.page_size must be a power of two in 128..65536");
  if (pg.table_stride < 1 || pg.table_stride > 65536) return fail(CSA2_ERR_ARG, "pages.table_stride must be in 1..65536");
  if (pg.pool_entries < 1 || pg.pool_entries > CSA2_MAX_ENTRIES)
    return fail(CSA2_ERR_ARG, "pages.pool_entries must be in 1..%d", CSA2_MAX_ENTRIES);
  if (max_ne >= 0 && pg.table_stride < (max_ne + pg.page_size - 1) / pg.page_size)
    return fail(CSA2_ERR_ARG, "pages.table_stride smaller than the pages of the longest sequence");
  return CSA2_OK;
}

// The kernels' page map of sequences s0.. (none for a contiguous cache).
PageMap page_map(const csa2_pages& pg, int s0) {
  PageMap m{};
  if (!pg.table) return m;
  m.pages = pg.table + (int64_t)s0 * pg.table_stride;
  m.stride = pg.table_stride;
  m.pool = pg.pool_entries;
  int lg = 0;
  while ((1 << lg) < pg.page_size) ++lg;
  m.lg = lg;
  return m;
}

int validate_index(const csa2_index_args* a) {
  if (!a) return fail(CSA2_ERR_ARG, "index args are NULL");
  if (a->kind < CSA2_INDEX_FLAT || a->kind > CSA2_INDEX_FLAT_POOL) return fail(CSA2_ERR_ARG, "bad index kind %d", a->kind);
  if (a->batch < 1 || a->n_q < 1) return fail(CSA2_ERR_ARG, "batch and n_q must be >= 1");
  if (a->ratio != 1 && a->ratio != 2) return fail(CSA2_ERR_ARG, "ratio must be 1 or 2");
  if (a->k < 1 || a->k > CSA2_MAX_K) return fail(CSA2_ERR_UNSUPPORTED, "k must be in 1..%d", CSA2_MAX_K);
  if (!a->q_pos0 || !a->n_entries) return fail(CSA2_ERR_ARG, "q_pos0 and n_entries (host) are required");
  if (!a->idx_q || !a->k8 || !a->kscale || !a->out_idx) return fail(CSA2_ERR_ARG, "idx_q, k8, kscale, out_idx are required");
  if (!aligned(a->idx_q, 16) || !aligned(a->k8, 16)) return fail(CSA2_ERR_ARG, "idx_q and k8 must be 16-byte aligned");
  if (!aligned(a->kscale, 4) || !aligned(a->out_idx, 4) || (a->idx_w && !aligned(a->idx_w, 4)))
    return fail(CSA2_ERR_ARG, "kscale, idx_w, out_idx must be 4-byte aligned");
  int64_t max_ne = 0;
  for (int s = 0; s < a->batch; ++s) {
    if (a->q_pos0[s] < 0) return fail(CSA2_ERR_ARG, "q_pos0[%d] < 0", s);
    if (a->n_entries[s] < 0) return fail(CSA2_ERR_ARG, "n_entries[%d] < 0", s);
    if (a->n_entries[s] > CSA2_MAX_ENTRIES)
      return fail(CSA2_ERR_UNSUPPORTED, "n_entries[%d] above CSA2_MAX_ENTRIES (%d)", s, CSA2_MAX_ENTRIES);
    max_ne = std::max(max_ne, a->n_entries[s]);
  }
  if (max_ne > kMaxEntries) return fail(CSA2_ERR_UNSUPPORTED, "at most %lld entries per sequence", (long long)kMaxEntries);
  if (a->pages.table) {
    if ((a->kind != CSA2_INDEX_FLAT && a->kind != CSA2_INDEX_FLAT_POOL) || a->n_q >= kPrefillMinQ)
      return fail(CSA2_ERR_UNSUPPORTED, "paged caches take FLAT indexing with fewer than %d queries per sequence", kPrefillMinQ);
    if (int rc = validate_pages(a->pages, max_ne)) return rc;
  } else if (a->batch > 1 && a->k_stride < max_ne) {
    return fail(CSA2_ERR_ARG, "k_stride smaller than n_entries");
  }
  if (a->kind == CSA2_INDEX_HIER) {
    if (!a->bk8 || !a->bkscale) return fail(CSA2_ERR_ARG, "HIER needs bk8 and bkscale");
    if (!aligned(a->bk8, 16) || !aligned(a->bkscale, 4)) return fail(CSA2_ERR_ARG, "bk8 must be 16-byte aligned");
    if (a->n_blocks < 1 || a->n_blocks > CSA2_MAX_K) return fail(CSA2_ERR_UNSUPPORTED, "n_blocks must be in 1..%d", CSA2_MAX_K);
    if (a->batch > 1 && a->bk_stride < (max_ne + 7) / 8) return fail(CSA2_ERR_ARG, "bk_stride smaller than the block count");
    if (a->out_pool && !aligned(a->out_pool, 4)) return fail(CSA2_ERR_ARG, "out_pool must be 4-byte aligned");
  }
  if (a->key_heads != 0 && a->key_heads != 1 && a->key_heads != 4)
    return fail(CSA2_ERR_ARG, "key_heads must be 0, 1 or 4");
  if (a->key_heads == 4 && (a->kind == CSA2_INDEX_HIER || a->n_q >= kPrefillMinQ || a->pages.table))
    return fail(CSA2_ERR_UNSUPPORTED,
                "per-head keys take FLAT, FLAT_POOL or POOL indexing with fewer than %d queries on a contiguous cache",
                kPrefillMinQ);
  if (a->kind == CSA2_INDEX_FLAT_POOL) {
    if (!a->out_pool || !aligned(a->out_pool, 4)) return fail(CSA2_ERR_ARG, "FLAT_POOL needs a 4-byte aligned out_pool");
    if (a->n_blocks < 1 || a->n_blocks > CSA2_MAX_K) return fail(CSA2_ERR_UNSUPPORTED, "n_blocks must be in 1..%d", CSA2_MAX_K);
  }
  if (a->kind != CSA2_INDEX_FLAT && a->n_q >= kPrefillMinQ)
    return fail(CSA2_ERR_UNSUPPORTED, "HIER, POOL and FLAT_POOL indexing take fewer than %d queries per sequence",
                kPrefillMinQ);
  if (a->kind == CSA2_INDEX_POOL) {
    if (!a->cand || !aligned(a->cand, 4)) return fail(CSA2_ERR_ARG, "POOL needs a 4-byte aligned cand");
    if (a->n_cand < 1 || a->n_cand > kMaxPool) return fail(CSA2_ERR_UNSUPPORTED, "n_cand must be in 1..%d", kMaxPool);
  }
  return CSA2_OK;
}

int64_t index_max_items(const csa2_index_args* a) {
  int64_t m = 0;
  for (int s = 0; s < a->batch; ++s) m = std::max(m, a->n_entries[s]);
  if (a->kind == CSA2_INDEX_POOL) m = std::max<int64_t>(m, a->n_cand);
  if (a->kind == CSA2_INDEX_HIER || a->kind == CSA2_INDEX_FLAT_POOL)
    m = std::max<int64_t>(m, (int64_t)a->n_blocks * CSA2_BLOCK);
  return m;
}

int run_index(const csa2_index_args* a, void* ws, const WsLayout& w, hipStream_t stream,
              const AttnPass* attn = nullptr, bool* attended = nullptr) {
  if (attended) *attended = false;
  for (int s0 = 0; s0 < a->batch; s0 += kMaxSeqPerLaunch) {
    const int nb = std::min(kMaxSeqPerLaunch, a->batch - s0);
    IndexPass p{};
    p.rows = nb * a->n_q;
    p.n_q = a->n_q;
    p.ratio = a->ratio;
    p.key_heads = a->key_heads == 4 ? 4 : 1;
    int64_t max_vis = 0;
    for (int i = 0; i < nb; ++i) {
      p.seq.a[i] = a->q_pos0[s0 + i];
      p.seq.b[i] = a->n_entries[s0 + i];
      max_vis = std::max(max_vis, visible(a->q_pos0[s0 + i] + a->n_q - 1, a->ratio, a->n_entries[s0 + i]));
    }
    const int64_t row0 = (int64_t)s0 * a->n_q;
    if (max_vis == 0) {  // nothing visible in these sequences: every output is -1
      hipError_t f = launch_fill_u32(reinterpret_cast<uint32_t*>(a->out_idx + row0 * a->k),
                                     (size_t)p.rows * a->k, 0xFFFFFFFFu, stream);
      if (f == hipSuccess && (a->kind == CSA2_INDEX_HIER || a->kind == CSA2_INDEX_FLAT_POOL) && a->out_pool)
        f = launch_fill_u32(reinterpret_cast<uint32_t*>(a->out_pool + row0 * a->n_blocks * CSA2_BLOCK),
                            (size_t)p.rows * a->n_blocks * CSA2_BLOCK, 0xFFFFFFFFu, stream);
      if (f != hipSuccess) return hip_fail(f, "fill");
      continue;
    }
    if (a->n_q >= kPrefillMinQ) {  // prefill chunk: MFMA indexer
      PrefillPass f{};
      f.rows = p.rows; f.n_q = a->n_q; f.ratio = a->ratio; f.k = a->k; f.batch = nb;
      f.tiles_per_seq = (a->n_q + kPfRows - 1) / kPfRows;
      const int tiles = nb * f.tiles_per_seq;
      // key ranges per row tile: enough workgroups to fill the device in one round
      const int slots = prefill_filter_slots(a->idx_w != nullptr);
      f.esplit = std::max(1, std::min(kPfSplits, (slots + tiles - 1) / tiles));
      f.seq = p.seq;
      f.idx_q = a->idx_q + row0 * kHI * kDI;
      f.idx_w = a->idx_w ? a->idx_w + row0 * kHI : nullptr;
      f.k8 = a->k8 + (int64_t)s0 * a->k_stride * kDI;
      f.kscale = a->kscale + (int64_t)s0 * a->k_stride;
      f.k_stride = a->k_stride;
      f.sample = at<float>(ws, w.pf_sample);
      f.thresh = at<float>(ws, w.pf_thresh);
      f.fallbacks = at<uint32_t>(ws, w.stats);
      f.count = at<uint32_t>(ws, w.pf_count);
      f.list = at<uint64_t>(ws, w.pf_list);
      f.out = a->out_idx + row0 * a->k;
      f.out_stride = a->k;
      hipError_t e = launch_prefill_index(f, stream);
      if (e != hipSuccess) return hip_fail(e, "prefill index");
      continue;
    }
    p.idx_q = a->idx_q + row0 * kHI * kDI;
    p.idx_w = a->idx_w ? a->idx_w + row0 * kHI : nullptr;
    p.fallbacks = at<uint32_t>(ws, w.stats);
    p.chunk_info = at<u32x4_t>(ws, w.chunk_info);
    p.seg_list = at<uint64_t>(ws, w.seg_list);
    p.max_chunks = w.max_chunks;
    hipError_t e;
    if (a->kind == CSA2_INDEX_HIER) {
      IndexPass b = p;  // pass 1: blocks
      b.source = kItemsDirect;
      b.block_level = 1;
      b.k = a->n_blocks;
      b.k8 = a->bk8 + (int64_t)s0 * a->bk_stride * kDI;
      b.kscale = a->bkscale + (int64_t)s0 * a->bk_stride;
      b.k_stride = a->bk_stride;
      b.max_items = (max_vis + 7) / 8;
      b.out = at<int32_t>(ws, w.blocks);
      b.out_stride = CSA2_MAX_K;
      b.out_count = at<int32_t>(ws, w.nsel);
      b.out_pool = a->out_pool ? a->out_pool + row0 * a->n_blocks * CSA2_BLOCK : nullptr;
      b.pool_stride = a->n_blocks * CSA2_BLOCK;
      if ((e = launch_index_pass(b, stream)) != hipSuccess) return hip_fail(e, "hierarchical block pass");
      p.source = kItemsBlocks;  // pass 2: positions of the kept blocks
      p.blocks = b.out;
      p.nsel = b.out_count;
      p.max_items = (int64_t)a->n_blocks * CSA2_BLOCK;
    } else if (a->kind == CSA2_INDEX_POOL) {
      p.source = kItemsList;
      p.list = a->cand + row0 * a->n_cand;
      p.list_len = a->n_cand;
      p.max_items = a->n_cand;
    } else {
      p.source = kItemsDirect;
      p.max_items = max_vis;
    }
    p.block_level = 0;
    p.k = a->k;
    p.pm = page_map(a->pages, s0);
    const int64_t koff = a->pages.table ? 0 : (int64_t)s0 * a->k_stride;  // paged: the pool
    p.k8 = a->k8 + koff * kDI * p.key_heads;
    p.kscale = a->kscale + koff;
    p.k_stride = a->k_stride;
    p.out = a->out_idx + row0 * a->k;
    p.out_stride = a->k;
    if (a->kind == CSA2_INDEX_FLAT_POOL) {  // the flat scan keeps its block maxima
      p.block_max = at<uint32_t>(ws, w.block_max);
      p.block_max_stride = w.max_blocks;
      p.row_ksm = at<uint32_t>(ws, w.row_ksm);
    }
    if ((e = launch_index_pass(p, stream, attn, attended)) != hipSuccess)
      return hip_fail(e, "index pass");
    if (a->kind == CSA2_INDEX_FLAT_POOL) {  // then the blocks by their largest token score
      IndexPass b = p;
      b.block_level = 2;
      b.k = a->n_blocks;
      b.max_items = (max_vis + 7) / 8;
      b.out = at<int32_t>(ws, w.blocks);
      b.out_stride = CSA2_MAX_K;
      b.out_count = at<int32_t>(ws, w.nsel);
      b.out_pool = a->out_pool + row0 * a->n_blocks * CSA2_BLOCK;
      b.pool_stride = a->n_blocks * CSA2_BLOCK;
      if ((e = launch_index_pass(b, stream)) != hipSuccess) return hip_fail(e, "block-max pass");
    }
  }
  return CSA2_OK;
}

// ------------------------------------------------------------- attention
constexpr int64_t kMaxRing = (1 << 21) - 1;  // ring rows x 1 KB must fit a 32-bit buffer range

int validate_attn_common(int32_t batch, int32_t n_q, int32_t n_idx, const int64_t* q_pos0,
                         const int64_t* swa_pos0, int64_t swa_rows, int64_t swa_stride, int64_t swa_ring) {
  if (batch < 1 || n_q < 1) return fail(CSA2_ERR_ARG, "batch and n_q must be >= 1");
  if (n_idx < 0 || n_idx > CSA2_MAX_K) return fail(CSA2_ERR_UNSUPPORTED, "n_idx must be in 0..%d", CSA2_MAX_K);
  if (!q_pos0) return fail(CSA2_ERR_ARG, "q_pos0 (host) is required");
  if (swa_ring < 0) return fail(CSA2_ERR_ARG, "swa_ring < 0");
  if (swa_ring > 0) {  // ring: token t at row t mod swa_ring
    if (swa_ring < (int64_t)n_q + CSA2_SWA - 1)
      return fail(CSA2_ERR_ARG, "swa_ring %lld is below n_q + %d", (long long)swa_ring, CSA2_SWA - 1);
    if (swa_ring > kMaxRing) return fail(CSA2_ERR_ARG, "swa_ring above %lld", (long long)kMaxRing);
    if (batch > 1 && swa_stride < swa_ring) return fail(CSA2_ERR_ARG, "swa_stride smaller than swa_ring");
    for (int s = 0; s < batch; ++s)
      if (q_pos0[s] < 0) return fail(CSA2_ERR_ARG, "q_pos0[%d] < 0", s);
    return CSA2_OK;
  }
  if (!swa_pos0) return fail(CSA2_ERR_ARG, "swa_pos0 (host) is required for a linear window");
  if (swa_rows < 1) return fail(CSA2_ERR_ARG, "swa_rows must be >= 1");
  if (batch > 1 && swa_stride < swa_rows) return fail(CSA2_ERR_ARG, "swa_stride smaller than swa_rows");
  for (int s = 0; s < batch; ++s) {
    if (q_pos0[s] < 0) return fail(CSA2_ERR_ARG, "q_pos0[%d] < 0", s);
    const int64_t first = std::max<int64_t>(0, q_pos0[s] - (CSA2_SWA - 1));
    const int64_t last = q_pos0[s] + n_q - 1;
    if (first < swa_pos0[s] || last - swa_pos0[s] >= swa_rows)
      return fail(CSA2_ERR_ARG, "sequence %d: window tokens %lld..%lld not in the buffer (rows %lld..%lld)", s,
                  (long long)first, (long long)last, (long long)swa_pos0[s], (long long)(swa_pos0[s] + swa_rows - 1));
  }
  return CSA2_OK;
}

struct AttnJob {
  int32_t batch, n_q, n_idx;
  const int64_t* q_pos0;
  const int64_t* swa_pos0;
  int64_t swa_ring;
  const uint8_t* nib;
  const uint8_t* scale;
  int64_t kv_stride;
  const int32_t* idx;
  int64_t swa_stride;
  float softmax_scale;
  int n_layers;
  AttnLayer layer[kMaxAttnLayers];
  bool tiles_elsewhere;   // the select launch ran every tile (only the merge is left)
  csa2_pages pages;       // paged nib / scale, or a zero table
};

// Candidate tiles of one (layer, row): the selected entries, then the window.
int attn_tiles(int n_idx) { return (n_idx + kAttnSplit - 1) / kAttnSplit + (CSA2_SWA + kAttnSplit - 1) / kAttnSplit; }

// Workgroups the tiles of a (layer, row) are split over: enough for about
// 1024 workgroups in flight, with at most `cap` partial slots in all; with
// many rows one workgroup walks them all.
int attn_splits(int units, int n_tiles, int64_t cap) {
  int splits = std::max(1, std::min(n_tiles, (1024 + units - 1) / units));
  while (splits > 1 && (int64_t)units * splits > cap) --splits;
  return splits;
}

// The attention pass of sequences s0 .. s0 + nb - 1 of a job.
AttnPass make_attn_pass(const AttnJob& j, int s0, int nb, void* ws, const WsLayout& w) {
  const int n_tiles = attn_tiles(j.n_idx);
  AttnPass p{};
  p.rows = nb * j.n_q;
  p.n_q = j.n_q;
  p.n_idx = j.n_idx;
  p.n_layers = j.n_layers;
  for (int i = 0; i < nb; ++i) {
    p.seq.a[i] = j.q_pos0[s0 + i];
    p.seq.b[i] = j.swa_ring > 0 ? 0 : j.swa_pos0[s0 + i];
  }
  const int64_t row0 = (int64_t)s0 * j.n_q;
  const int64_t koff = j.pages.table ? 0 : (int64_t)s0 * j.kv_stride;  // paged: the pool
  p.nib = j.nib + koff * CSA2_NIB_BYTES;
  p.scale = j.scale + koff * CSA2_SCALE_BYTES;
  p.pm = page_map(j.pages, s0);
  p.kv_stride = j.kv_stride;
  p.idx = j.idx ? j.idx + row0 * j.n_idx : nullptr;
  p.swa_stride = j.swa_stride;
  p.swa_ring = j.swa_ring;
  p.softmax_scale = j.softmax_scale;
  for (int l = 0; l < j.n_layers; ++l) {
    p.layer[l].q = j.layer[l].q + row0 * kH * kD;
    p.layer[l].swa = j.layer[l].swa + (int64_t)s0 * j.swa_stride * kD;
    p.layer[l].out = j.layer[l].out + row0 * kH * kD;
  }
  const int splits = attn_splits(p.n_layers * p.rows, n_tiles, kMaxPartialUnits);
  p.n_tiles = n_tiles;
  p.tiles_per_split = (n_tiles + splits - 1) / splits;
  p.max_splits = (n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  p.partial = at<float>(ws, w.partial);
  p.tiles_elsewhere = j.tiles_elsewhere ? 1 : 0;
  return p;
}

// The tile form (one tile per workgroup) takes the pass.
bool tile_form(const AttnPass& p) { return p.tiles_per_split == 1 && p.max_splits == p.n_tiles; }

int run_attention(const AttnJob& j, void* ws, const WsLayout& w, hipStream_t stream) {
  for (int s0 = 0; s0 < j.batch; s0 += kMaxSeqPerLaunch) {
    const int nb = std::min(kMaxSeqPerLaunch, j.batch - s0);
    const AttnPass p = make_attn_pass(j, s0, nb, ws, w);
    hipError_t e = launch_attention(p, stream);
    if (e != hipSuccess) return hip_fail(e, "attention");
  }
  return CSA2_OK;
}

int validate_kv_ptrs(const uint8_t* nib, const uint8_t* scale) {
  if (!nib || !scale) return fail(CSA2_ERR_ARG, "nib and scale are required");
  if (!aligned(nib, 16) || !aligned(scale, 8)) return fail(CSA2_ERR_ARG, "nib must be 16-byte and scale 8-byte aligned");
  return CSA2_OK;
}

}  // namespace

// ===================================================================== C ABI
extern "C" {

int csa2_abi_version(void) { return CSA2_ABI_VERSION; }

size_t csa2_struct_size(int32_t which) {
  switch (which) {
    case 0: return sizeof(csa2_index_args);
    case 1: return sizeof(csa2_attn_args);
    case 2: return sizeof(csa2_kv);
    case 3: return sizeof(csa2_layer);
    case 4: return sizeof(csa2_group_state);
    case 5: return sizeof(csa2_group_args);
    case 6: return sizeof(csa2_append_args);
    case 7: return sizeof(csa2_pages);
    default: return 0;
  }
}

const char* csa2_last_error(void) { return g_err; }

size_t csa2_workspace_bytes(int32_t max_batch, int32_t max_n_q, int64_t max_entries) {
  if (max_batch < 1 || max_n_q < 1 || max_entries < 0) return 0;
  const int64_t seqs = std::min<int64_t>(max_batch, kMaxSeqPerLaunch);
  const int64_t items = std::max<int64_t>(max_entries, kMaxPool);
  const int64_t dec_rows = seqs * std::min<int64_t>(max_n_q, kPrefillMinQ - 1);
  const int64_t pf_rows = max_n_q >= kPrefillMinQ ? seqs * max_n_q : 0;
  return ws_layout(dec_rows, items, pf_rows).total;
}

int csa2_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace || !aligned(workspace, kWsAlign) || ws_bytes % 4)
    return fail(CSA2_ERR_WORKSPACE, "workspace must be non-NULL, 256-byte aligned, a multiple of 4 bytes");
  hipError_t e = launch_fill_u32(static_cast<uint32_t*>(workspace), ws_bytes / 4, 0u, (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "workspace init");
}

int csa2_append(const csa2_append_args* a, void* stream) {
  if (!a) return fail(CSA2_ERR_ARG, "append args are NULL");
  if (a->batch < 0) return fail(CSA2_ERR_ARG, "batch < 0");
  if (a->batch == 0) return CSA2_OK;
  if (a->ratio != 1 && a->ratio != 2) return fail(CSA2_ERR_ARG, "ratio must be 1 or 2");
  if (!a->pos || !a->x || !a->k_in || !a->nib || !a->scale || !a->k8 || !a->kscale)
    return fail(CSA2_ERR_ARG, "pos (host), x, k_in, nib, scale, k8, kscale are required");
  if (a->ratio == 2 && !a->pending) return fail(CSA2_ERR_ARG, "ratio 2 needs the pending buffer");
  if ((a->bk8 == nullptr) != (a->bkscale == nullptr)) return fail(CSA2_ERR_ARG, "bk8 and bkscale go together");
  if (!aligned(a->x, 16) || !aligned(a->k_in, 16) || !aligned(a->nib, 8) || !aligned(a->k8, 16) ||
      (a->bk8 && !aligned(a->bk8, 16)) || (a->pending && !aligned(a->pending, 16)) ||
      (a->swa && !aligned(a->swa, 16)))
    return fail(CSA2_ERR_ARG, "x, k_in, k8, bk8, pending, swa must be 16-byte aligned, nib 8-byte aligned");
  const bool paged = a->pages.table != nullptr;
  if (paged) {
    if (int rc = validate_pages(a->pages, -1)) return rc;
  } else if (a->batch > 1 && a->stride < 1) {
    return fail(CSA2_ERR_ARG, "stride must be >= 1");
  }
  if (a->swa) {
    if (a->swa_ring < CSA2_SWA) return fail(CSA2_ERR_ARG, "swa_ring must be >= %d", CSA2_SWA);
    if (a->batch > 1 && a->swa_stride < a->swa_ring) return fail(CSA2_ERR_ARG, "swa_stride smaller than swa_ring");
  }
  for (int s = 0; s < a->batch; ++s) {
    if (a->pos[s] < 0) return fail(CSA2_ERR_ARG, "pos[%d] < 0", s);
    const int64_t e = a->pos[s] / a->ratio;
    if (e >= CSA2_MAX_ENTRIES)
      return fail(CSA2_ERR_UNSUPPORTED, "sequence %d: entry %lld at or past CSA2_MAX_ENTRIES", s, (long long)e);
    if (paged && e >= a->pages.table_stride * a->pages.page_size)
      return fail(CSA2_ERR_ARG, "sequence %d: entry %lld past its page-table row", s, (long long)e);
    if (!paged && a->batch > 1 && e >= a->stride)
      return fail(CSA2_ERR_ARG, "sequence %d: entry %lld past stride", s, (long long)e);
    if (a->bk8 && a->batch > 1 && e / CSA2_BLOCK >= a->bk_stride)
      return fail(CSA2_ERR_ARG, "sequence %d: block %lld past bk_stride", s, (long long)(e / CSA2_BLOCK));
  }
  hipStream_t st = (hipStream_t)stream;
  for (int s0 = 0; s0 < a->batch; s0 += kMaxSeqPerLaunch) {
    const int nb = std::min(kMaxSeqPerLaunch, a->batch - s0);
    AppendPass p{};
    p.ratio = a->ratio;
    for (int i = 0; i < nb; ++i) p.seq.a[i] = a->pos[s0 + i];
    p.x = a->x + (int64_t)s0 * CSA2_D_LATENT;
    p.k_in = a->k_in + (int64_t)s0 * CSA2_D_INDEX;
    const int64_t koff = paged ? 0 : (int64_t)s0 * a->stride;  // paged: the pool
    p.nib = a->nib + koff * CSA2_NIB_BYTES;
    p.scale = a->scale + koff * CSA2_SCALE_BYTES;
    p.k8 = a->k8 + koff * CSA2_D_INDEX;
    p.kscale = a->kscale + koff;
    p.stride = a->stride;
    p.pm = page_map(a->pages, s0);
    p.bk8 = a->bk8 ? a->bk8 + (int64_t)s0 * a->bk_stride * CSA2_D_INDEX : nullptr;
    p.bks = a->bkscale ? a->bkscale + (int64_t)s0 * a->bk_stride : nullptr;
    p.bk_stride = a->bk_stride;
    p.pending = a->pending ? a->pending + (int64_t)s0 * (CSA2_D_LATENT + CSA2_D_INDEX) : nullptr;
    p.swa = a->swa ? a->swa + (int64_t)s0 * a->swa_stride * CSA2_D_LATENT : nullptr;
    p.swa_stride = a->swa_stride;
    p.swa_ring = a->swa_ring;
    hipError_t e = launch_append(p, nb, st);
    if (e != hipSuccess) return hip_fail(e, "append");
  }
  return CSA2_OK;
}

int csa2_workspace_fallbacks(const void* workspace, uint32_t* count, void* stream) {
  if (!workspace || !count) return fail(CSA2_ERR_ARG, "workspace and count are required");
  if (!aligned(workspace, kWsAlign)) return fail(CSA2_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(count, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "reading the fallback counter");
}

int csa2_quantize_kv(const float* x, int64_t n_tok, int64_t ld_x, int32_t ratio, uint8_t* nib,
                     uint8_t* scale, const float* k_in, int64_t ld_k, uint8_t* k8, float* kscale,
                     void* stream) {
  if (ratio != 1 && ratio != 2) return fail(CSA2_ERR_ARG, "ratio must be 1 or 2");
  if (n_tok < 0 || n_tok % ratio) return fail(CSA2_ERR_ARG, "n_tok must be >= 0 and a multiple of ratio");
  if (n_tok == 0) return CSA2_OK;
  if (!x || !nib || !scale) return fail(CSA2_ERR_ARG, "x, nib, scale are required");
  if (ld_x < CSA2_D_LATENT || ld_x % 4) return fail(CSA2_ERR_ARG, "ld_x must be >= 512 and a multiple of 4");
  if (!aligned(x, 16) || !aligned(nib, 16)) return fail(CSA2_ERR_ARG, "x and nib must be 16-byte aligned");
  if (k_in) {
    if (!k8 || !kscale) return fail(CSA2_ERR_ARG, "k8 and kscale are required with k_in");
    if (ld_k < CSA2_D_INDEX) return fail(CSA2_ERR_ARG, "ld_k must be >= 64");
    if (!aligned(k_in, 4) || !aligned(k8, 16) || !aligned(kscale, 4))
      return fail(CSA2_ERR_ARG, "k_in/kscale must be 4-byte and k8 16-byte aligned");
  }
  hipError_t e = launch_quantize(x, n_tok / ratio, ld_x, ratio, nib, scale, k_in, ld_k, k8, kscale,
                                 (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "quantize");
}

int csa2_quantize_head_keys(const float* k_in, int64_t n_tok, int64_t ld_k, int32_t ratio, uint8_t* k8,
                            float* kscale, void* stream) {
  if (ratio != 1 && ratio != 2) return fail(CSA2_ERR_ARG, "ratio must be 1 or 2");
  if (n_tok < 0 || n_tok % ratio) return fail(CSA2_ERR_ARG, "n_tok must be >= 0 and a multiple of ratio");
  if (n_tok == 0) return CSA2_OK;
  if (!k_in || !k8 || !kscale) return fail(CSA2_ERR_ARG, "k_in, k8, kscale are required");
  if (ld_k < 4 * CSA2_D_INDEX) return fail(CSA2_ERR_ARG, "ld_k must be >= 256");
  if (!aligned(k_in, 4) || !aligned(k8, 16) || !aligned(kscale, 4))
    return fail(CSA2_ERR_ARG, "k_in/kscale must be 4-byte and k8 16-byte aligned");
  hipError_t e = launch_quantize_head_keys(k_in, n_tok / ratio, ld_k, ratio, k8, kscale, (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "quantize head keys");
}

int csa2_build_block_keys(const uint8_t* k8, const float* kscale, int32_t batch,
                          const int64_t* n_entries, int64_t k_stride, uint8_t* bk8, float* bkscale,
                          int64_t bk_stride, void* stream) {
  if (batch < 0) return fail(CSA2_ERR_ARG, "batch < 0");
  if (batch == 0) return CSA2_OK;
  if (!k8 || !kscale || !n_entries || !bk8 || !bkscale) return fail(CSA2_ERR_ARG, "null argument");
  if (!aligned(k8, 16) || !aligned(bk8, 16) || !aligned(kscale, 4) || !aligned(bkscale, 4))
    return fail(CSA2_ERR_ARG, "k8/bk8 must be 16-byte and scales 4-byte aligned");
  int64_t max_ne = 0;
  for (int s = 0; s < batch; ++s) {
    if (n_entries[s] < 0) return fail(CSA2_ERR_ARG, "n_entries[%d] < 0", s);
    if (n_entries[s] > CSA2_MAX_ENTRIES)
      return fail(CSA2_ERR_UNSUPPORTED, "n_entries[%d] above CSA2_MAX_ENTRIES (%d)", s, CSA2_MAX_ENTRIES);
    max_ne = std::max(max_ne, n_entries[s]);
  }
  if (batch > 1 && (k_stride < max_ne || bk_stride < (max_ne + 7) / 8))
    return fail(CSA2_ERR_ARG, "strides smaller than the data they hold");
  hipError_t e = launch_block_keys(k8, kscale, k_stride, n_entries, batch, bk8, bkscale, bk_stride,
                                   (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : hip_fail(e, "block keys");
}

int csa2_index_topk(const csa2_index_args* a, void* workspace, size_t ws_bytes, void* stream) {
  int rc = validate_index(a);
  if (rc) return rc;
  const WsLayout w = ws_for(a->batch, a->n_q, index_max_items(a));
  if ((rc = check_workspace(workspace, ws_bytes, w))) return rc;
  return run_index(a, workspace, w, (hipStream_t)stream);
}

int csa2_sparse_swa_attn(const csa2_attn_args* a, void* workspace, size_t ws_bytes, void* stream) {
  if (!a) return fail(CSA2_ERR_ARG, "attention args are NULL");
  int rc = validate_attn_common(a->batch, a->n_q, a->n_idx, a->q_pos0, a->swa_pos0, a->swa_rows, a->swa_stride,
                                a->swa_ring);
  if (rc) return rc;
  if ((rc = validate_kv_ptrs(a->nib, a->scale))) return rc;
  if (!a->q || !a->swa || !a->out || (a->n_idx > 0 && !a->idx)) return fail(CSA2_ERR_ARG, "q, swa, out, idx are required");
  if (!aligned(a->q, 16) || !aligned(a->swa, 16) || !aligned(a->out, 16) || (a->idx && !aligned(a->idx, 4)))
    return fail(CSA2_ERR_ARG, "q, swa, out must be 16-byte aligned");
  if (a->batch > 1 && a->kv_stride < 0) return fail(CSA2_ERR_ARG, "kv_stride < 0");
  if ((rc = validate_pages(a->pages, -1))) return rc;
  const WsLayout w = ws_layout(0, 0, 0);  // attention uses only the partials
  if ((rc = check_workspace(workspace, ws_bytes, w))) return rc;
  AttnJob j{};
  j.batch = a->batch; j.n_q = a->n_q; j.n_idx = a->n_idx;
  j.q_pos0 = a->q_pos0; j.swa_pos0 = a->swa_pos0; j.swa_ring = a->swa_ring;
  j.nib = a->nib; j.scale = a->scale; j.kv_stride = a->kv_stride;
  j.idx = a->idx; j.swa_stride = a->swa_stride; j.softmax_scale = a->softmax_scale;
  j.pages = a->pages;
  j.n_layers = 1;
  j.layer[0] = AttnLayer{a->q, a->swa, a->out};
  return run_attention(j, workspace, w, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Partial slots the attention launches of a plan use at most: the plan's
// largest attention job (a layer and the Reuse layers after it) over each
// launch's rows.
int64_t plan_partial_units(const csa2_group_args* a) {
  int max_layers = 0;
  for (int l = 0; l < a->n_layers;) {
    int n = 0;
    do {
      ++n;
      ++l;
    } while (l < a->n_layers && a->layers[l].mode == CSA2_MODE_REUSE && n < kMaxAttnLayers);
    max_layers = std::max(max_layers, n);
  }
  int64_t need = 0;
  const int tiles = attn_tiles(CSA2_TOP_K);
  for (int s0 = 0; s0 < a->batch; s0 += kMaxSeqPerLaunch) {
    const int units = max_layers * std::min(kMaxSeqPerLaunch, a->batch - s0) * a->n_q;
    const int splits = attn_splits(units, tiles, kMaxPartialUnits);
    if (splits > 1) need = std::max<int64_t>(need, (int64_t)units * splits);
  }
  return need;
}

// The library's own scratch for csa2_run_group_noalloc (see there).
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// The current device's copy of the scratch array, its address looked up
// once per device (with that device current).
int scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(CSA2_ERR_UNSUPPORTED, "csa2_run_group_noalloc: device %d (at most %d devices)", dev, kScratchDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned(ptr, kWsAlign)) return fail(CSA2_ERR_HIP, "scratch address is not 256-byte aligned");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return CSA2_OK;
}

// csa2_run_group; with noalloc set, workspace and ws_bytes are ignored and
// the call runs in the device's scratch array, its partials sized to the plan.
int run_group(const csa2_group_args* a, csa2_group_state* st, void* workspace, size_t ws_bytes, hipStream_t stream,
              bool noalloc) {
  if (!a || !st) return fail(CSA2_ERR_ARG, "group args and state are required");
  if (a->n_layers < 1 || !a->layers) return fail(CSA2_ERR_ARG, "at least one layer is required");
  if (a->ratio != 1 && a->ratio != 2) return fail(CSA2_ERR_ARG, "ratio must be 1 or 2");
  if (a->index_kind != CSA2_INDEX_FLAT && a->index_kind != CSA2_INDEX_HIER && a->index_kind != CSA2_INDEX_FLAT_POOL)
    return fail(CSA2_ERR_ARG, "index_kind must be FLAT, HIER or FLAT_POOL");
  if (a->reindex_kind != CSA2_INDEX_FLAT && a->reindex_kind != CSA2_INDEX_POOL)
    return fail(CSA2_ERR_ARG, "reindex_kind must be FLAT or POOL");
  if ((a->index_kind != CSA2_INDEX_FLAT || a->reindex_kind != CSA2_INDEX_FLAT) && a->n_q >= kPrefillMinQ)
    return fail(CSA2_ERR_UNSUPPORTED, "HIER and POOL indexing take fewer than %d queries per sequence", kPrefillMinQ);
  if (!a->n_entries) return fail(CSA2_ERR_ARG, "n_entries (host) is required");
  int rc = validate_attn_common(a->batch, a->n_q, CSA2_TOP_K, a->q_pos0, a->swa_pos0, a->swa_rows, a->swa_stride,
                                a->swa_ring);
  if (rc) return rc;
  if (!st->indices || !aligned(st->indices, 4)) return fail(CSA2_ERR_ARG, "state.indices must be a device buffer");
  // simulate the plan on the host: every mode change is checked before launching
  int has_full = st->has_full, has_idx = st->has_indices, has_pool = st->has_pool;
  bool paged = st->has_full && st->kv.pages.table != nullptr;  // the KV a Reindex layer would index
  if ((has_idx || has_full) && (st->batch != a->batch || st->n_q != a->n_q))
    return fail(CSA2_ERR_STATE, "state was made for batch %d x n_q %d", st->batch, st->n_q);
  int64_t max_ne = 0;
  for (int s = 0; s < a->batch; ++s) {
    if (a->n_entries[s] < 0) return fail(CSA2_ERR_ARG, "n_entries[%d] < 0", s);
    if (a->n_entries[s] > CSA2_MAX_ENTRIES)
      return fail(CSA2_ERR_UNSUPPORTED, "n_entries[%d] above CSA2_MAX_ENTRIES (%d)", s, CSA2_MAX_ENTRIES);
    max_ne = std::max(max_ne, a->n_entries[s]);
  }
  for (int l = 0; l < a->n_layers; ++l) {
    const csa2_layer& L = a->layers[l];
    if (L.mode < CSA2_MODE_FULL || L.mode > CSA2_MODE_REUSE) return fail(CSA2_ERR_ARG, "layer %d: bad mode", l);
    if (!L.q || !L.swa || !L.out || !aligned(L.q, 16) || !aligned(L.swa, 16) || !aligned(L.out, 16))
      return fail(CSA2_ERR_ARG, "layer %d: q, swa, out must be 16-byte aligned device pointers", l);
    if (L.mode == CSA2_MODE_FULL) {
      if (!L.kv) return fail(CSA2_ERR_ARG, "layer %d: FULL needs kv", l);
      if ((rc = validate_kv_ptrs(L.kv->nib, L.kv->scale))) return rc;
      if (!L.kv->k8 || !L.kv->kscale || !aligned(L.kv->k8, 16)) return fail(CSA2_ERR_ARG, "layer %d: kv.k8/kscale", l);
      if (L.kv->pages.table) {
        if (a->index_kind == CSA2_INDEX_HIER || a->n_q >= kPrefillMinQ)
          return fail(CSA2_ERR_UNSUPPORTED, "layer %d: paged caches take FLAT indexing with fewer than %d queries", l,
                      kPrefillMinQ);
        if ((rc = validate_pages(L.kv->pages, max_ne))) return rc;
      } else if (a->batch > 1 && L.kv->stride < max_ne) {
        return fail(CSA2_ERR_ARG, "layer %d: kv.stride < n_entries", l);
      }
      if (a->index_kind == CSA2_INDEX_HIER && (!L.kv->bk8 || !L.kv->bkscale))
        return fail(CSA2_ERR_ARG, "layer %d: HIER needs block keys", l);
      if (L.kv->key_heads != 0 && L.kv->key_heads != 1 && L.kv->key_heads != 4)
        return fail(CSA2_ERR_ARG, "layer %d: kv.key_heads must be 0, 1 or 4", l);
      if (L.kv->key_heads == 4 && (a->index_kind == CSA2_INDEX_HIER || a->n_q >= kPrefillMinQ || L.kv->pages.table))
        return fail(CSA2_ERR_UNSUPPORTED,
                    "layer %d: per-head keys take FLAT or FLAT_POOL indexing with fewer than %d queries on a "
                    "contiguous cache", l, kPrefillMinQ);
      const bool keeps_pool = a->index_kind == CSA2_INDEX_HIER || a->index_kind == CSA2_INDEX_FLAT_POOL;
      if (keeps_pool && !st->pool && a->reindex_kind == CSA2_INDEX_POOL)
        return fail(CSA2_ERR_ARG, "POOL reindexing needs state.pool");
      has_full = has_idx = 1;
      paged = L.kv->pages.table != nullptr;
      // a Full layer replaces the KV: only one that keeps a pool (HIER or
      // FLAT_POOL) leaves one of it (a flat one makes any earlier pool stale)
      has_pool = (keeps_pool && st->pool) ? 1 : 0;
    } else if (L.mode == CSA2_MODE_REINDEX) {
      if (!has_full) return fail(CSA2_ERR_STATE, "layer %d: REINDEX before any FULL layer", l);
      if (a->reindex_kind == CSA2_INDEX_POOL && !has_pool)
        return fail(CSA2_ERR_STATE, "layer %d: POOL REINDEX without a pool from a HIER or FLAT_POOL Full layer", l);
      if (paged && (a->reindex_kind != CSA2_INDEX_FLAT || a->n_q >= kPrefillMinQ))
        return fail(CSA2_ERR_UNSUPPORTED, "layer %d: paged caches take FLAT indexing with fewer than %d queries", l,
                    kPrefillMinQ);
      has_idx = 1;
    } else {
      if (!has_full || !has_idx) return fail(CSA2_ERR_STATE, "layer %d: REUSE before any FULL layer", l);
    }
    if (L.mode != CSA2_MODE_REUSE) {
      if (!L.idx_q || !aligned(L.idx_q, 16)) return fail(CSA2_ERR_ARG, "layer %d: idx_q must be 16-byte aligned", l);
      if (L.idx_w && !aligned(L.idx_w, 4)) return fail(CSA2_ERR_ARG, "layer %d: idx_w alignment", l);
    }
  }
  const int64_t max_items = std::max<int64_t>(max_ne, kMaxPool);
  const WsLayout w = noalloc ? ws_for(a->batch, a->n_q, max_items, plan_partial_units(a))
                             : ws_for(a->batch, a->n_q, max_items);
  if (noalloc) {
    if (w.total > kScratchBytes)
      return fail(CSA2_ERR_UNSUPPORTED,
                  "csa2_run_group_noalloc: this call needs %zu bytes of scratch, the library holds %zu "
                  "(fewer sequences, queries per sequence or entries per call fit)",
                  w.total, kScratchBytes);
    if ((rc = scratch_of_current_device(&workspace))) return rc;
    ws_bytes = kScratchBytes;
  }
  if ((rc = check_workspace(workspace, ws_bytes, w))) return rc;

  hipStream_t s = stream;
  int l = 0;
  while (l < a->n_layers) {
    const csa2_layer& L = a->layers[l];
    if (L.mode == CSA2_MODE_FULL) st->kv = *L.kv;
    // this layer and the Reuse layers after it share KV and indices: one
    // attention launch
    AttnJob j{};
    j.batch = a->batch; j.n_q = a->n_q; j.n_idx = CSA2_TOP_K;
    j.q_pos0 = a->q_pos0; j.swa_pos0 = a->swa_pos0; j.swa_ring = a->swa_ring;
    j.nib = st->kv.nib; j.scale = st->kv.scale; j.kv_stride = st->kv.stride;
    j.idx = st->indices; j.swa_stride = a->swa_stride; j.softmax_scale = a->softmax_scale;
    j.pages = st->kv.pages;
    j.n_layers = 0;
    do {
      const csa2_layer& M = a->layers[l];
      j.layer[j.n_layers++] = AttnLayer{M.q, M.swa, M.out};
      ++l;
    } while (l < a->n_layers && a->layers[l].mode == CSA2_MODE_REUSE && j.n_layers < kMaxAttnLayers);
    if (L.mode != CSA2_MODE_REUSE) {
      csa2_index_args ia{};
      const bool hier = (L.mode == CSA2_MODE_FULL && a->index_kind == CSA2_INDEX_HIER);
      const bool flat_pool = (L.mode == CSA2_MODE_FULL && a->index_kind == CSA2_INDEX_FLAT_POOL && st->pool);
      const bool pool = (L.mode == CSA2_MODE_REINDEX && a->reindex_kind == CSA2_INDEX_POOL);
      ia.kind = hier ? CSA2_INDEX_HIER : flat_pool ? CSA2_INDEX_FLAT_POOL : pool ? CSA2_INDEX_POOL : CSA2_INDEX_FLAT;
      ia.batch = a->batch; ia.n_q = a->n_q; ia.ratio = a->ratio;
      ia.q_pos0 = a->q_pos0; ia.n_entries = a->n_entries;
      ia.idx_q = L.idx_q; ia.idx_w = L.idx_w;
      ia.k8 = st->kv.k8; ia.kscale = st->kv.kscale; ia.k_stride = st->kv.stride;
      ia.bk8 = st->kv.bk8; ia.bkscale = st->kv.bkscale; ia.bk_stride = st->kv.bk_stride;
      ia.cand = st->pool; ia.n_cand = kMaxPool;
      ia.k = CSA2_TOP_K; ia.n_blocks = CSA2_N_BLOCKS;
      ia.out_idx = st->indices;
      ia.out_pool = (hier || flat_pool) ? st->pool : nullptr;
      ia.pages = st->kv.pages;
      ia.key_heads = st->kv.key_heads;
      // a decode index pass in one launch (any kind: the token-level select
      // of HIER and POOL runs over a position list) runs the tile-form
      // attention in its select launch (k_index_select_attend); the
      // attention launch then only merges the partials
      AttnPass wp;
      const AttnPass* tiles = nullptr;
      if (a->batch <= kMaxSeqPerLaunch && a->n_q < kPrefillMinQ) {
        wp = make_attn_pass(j, 0, a->batch, workspace, w);
        if (tile_form(wp)) tiles = &wp;
      }
      bool attended = false;
      if ((rc = run_index(&ia, workspace, w, s, tiles, &attended))) return rc;
      j.tiles_elsewhere = attended;
      if (L.mode == CSA2_MODE_FULL) {
        st->has_full = 1;
        st->has_pool = (hier || flat_pool) ? 1 : 0;
      }
      st->has_indices = 1;
      st->batch = a->batch; st->n_q = a->n_q;
    }
    if ((rc = run_attention(j, workspace, w, s))) return rc;
  }
  return CSA2_OK;
}

}  // namespace

extern "C" {

int csa2_run_group(const csa2_group_args* a, csa2_group_state* st, void* workspace, size_t ws_bytes,
                   void* stream) {
  return run_group(a, st, workspace, ws_bytes, (hipStream_t)stream, false);
}

int csa2_run_group_noalloc(const csa2_group_args* a, csa2_group_state* st, void* stream) {
  prof_suspend(true);  // timing records would create events
  const int rc = run_group(a, st, nullptr, 0, (hipStream_t)stream, true);
  prof_suspend(false);
  return rc;
}

}  // extern "C"
