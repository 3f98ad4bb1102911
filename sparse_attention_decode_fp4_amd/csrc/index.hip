// Indexer + top-k of the CSA2 step.
//
// The pages (agentnet.co.il "DeepSeek launches V4.1-Flash ...", section
// "CSA2: compression along the layer axis") fix only what is selected: 512
// fresh positions per Full or Reindex layer, and for the hierarchical indexer
// a pool of 2,048 blocks of 8 positions.  The score is a reading:
//   s_p = ks_p * sum_h w_h * max(0, q_h . k_p)   over 4 indexer heads.
//
// One pass = three kernels over the rows (query rows) of a call:
//   sample  one 1,024-thread workgroup per row scores a sample of 2,048 of
//           its items, 256 evenly spaced runs of 8 (fp8 MFMA: the sample only
//           steers the threshold) and sets the row threshold T0: the lower
//           edge, at 20 key bits, of the key bin holding the k_s-th largest
//           sample, k_s sized so that about 2.5 k items of the row reach T0
//           (no threshold when the row has at most 2,048 items);
//   scan    streams the fp8 keys once (4 lanes per key, 16 B each, fully
//           coalesced; up to 4 queries of a sequence share a workgroup),
//           scores every item with packed f16 dot products (v_dot2c_f32_f16;
//           fp8 -> f16 is exact) and appends the items scoring at least T0
//           to a segment per (row, chunk), staged in LDS, counting each in
//           a histogram of score bins above T0;
//   select  gathers the segments (about 2.5 k candidates), finds the exact
//           k-th largest (score, -item) key (its bin from the histogram,
//           then a rank among that bin's few keys; a radix when the bins
//           cannot tell), orders the winners by item and writes their
//           positions.  If the candidates cannot hold
//           the answer (fewer than k, or a segment overflowed: the sample
//           misled, e.g. all scores equal) the row is recomputed exactly by
//           itself (radix steps over recomputed keys): slow, exact, rare.
#include "kernels.hpp"
#include "select.hpp"
#include "tile.hpp"

namespace csa2 {

constexpr int kSample = 2048;       // sampled items per row (two per thread of the sample kernel)
constexpr int kBitmapItems = 131072;  // rows with at most this many items order winners by bitmap
constexpr int kSpecChunks = 64;       // rows with at most this many scan chunks (twice this at k > 1,024) gather in one round trip
constexpr int kSpecSlots = 64;        // ... of the first this many slots of each segment

// The row geometry below is all the kernels compute before their first
// loads, so it avoids 64-bit divisions: the ratio is 1 or 2 and chunk sizes
// are powers of two.
__device__ __forceinline__ int64_t row_vis_positions(const IndexPass& p, int row) {
  const int seq = row / p.n_q, i = row - seq * p.n_q;
  const int64_t pos = p.seq.a[seq] + i;
  int64_t vis = p.ratio == 2 ? (pos + 1) >> 1 : pos + 1;
  const int64_t ne = p.seq.b[seq];
  vis = vis < ne ? vis : ne;
  return vis < 0 ? 0 : vis;
}

// Items of a row, and the limit positions must stay below.
__device__ __forceinline__ int64_t row_items(const IndexPass& p, int row, int64_t vis_pos) {
  if (p.source == kItemsDirect) return p.block_level ? (vis_pos + 7) >> 3 : vis_pos;
  if (p.source == kItemsBlocks) return 8 * (int64_t)p.nsel[row];
  return p.list_len;
}

// Items per scan chunk of a row (scan_chunk_items).  Over direct items every
// row of a sequence takes the size of the sequence's last query, which sees
// the most items, so one workgroup can scan a chunk for several queries; the
// select derives the same.
__device__ __forceinline__ int64_t row_chunk_items(const IndexPass& p, int row) {
  const int last = p.source == kItemsDirect ? (row / p.n_q) * p.n_q + p.n_q - 1 : row;
  return scan_chunk_items(row_items(p, last, row_vis_positions(p, last)), p.k);
}

// The same for a kernel compiled for one kind of item source (kDirect: the
// source is kItemsDirect; otherwise a block or position list), so the
// direct path has no branches on the source.
template <bool kDirect>
__device__ __forceinline__ int64_t row_items_of(const IndexPass& p, int row, int64_t vis_pos) {
  if constexpr (kDirect) return p.block_level ? (vis_pos + 7) >> 3 : vis_pos;
  else return p.source == kItemsBlocks ? 8 * (int64_t)p.nsel[row] : (int64_t)p.list_len;
}
template <bool kDirect>
__device__ __forceinline__ int64_t row_chunk_items_of(const IndexPass& p, int row) {
  const int last = kDirect ? (row / p.n_q) * p.n_q + p.n_q - 1 : row;
  return scan_chunk_items(row_items_of<kDirect>(p, last, row_vis_positions(p, last)), p.k);
}

// The sampled threshold of a row, read with a vector load: a scalar load of
// memory the previous kernel wrote would hold up the scalar loads of the
// row geometry (one counter covers them all) until it arrives.
__device__ __forceinline__ float load_thresh(const IndexPass& p, int row) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)(p.thresh + row), 0, 4, kRawBufferWord3);
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0));
}

// Histogram bin of a candidate's score key (candidates are at or above T0).
__device__ __forceinline__ uint32_t hist_bin(uint32_t key32, uint32_t t0key) {
  const uint32_t b = (key32 - t0key) >> kHistShift;
  return b < (uint32_t)(kHistBins - 1) ? b : (uint32_t)(kHistBins - 1);
}

__device__ __forceinline__ int64_t item_position(const IndexPass& p, int row, int64_t item,
                                                 int64_t n_items, int64_t vis_pos, bool& valid) {
  if (item >= n_items) { valid = false; return 0; }
  if (p.source == kItemsDirect) { valid = true; return item; }
  int64_t pos;
  if (p.source == kItemsBlocks)
    pos = 8 * (int64_t)p.blocks[(int64_t)row * CSA2_MAX_K + (item >> 3)] + (item & 7);
  else
    pos = p.list[(int64_t)row * p.list_len + item];
  valid = pos >= 0 && pos < vis_pos;
  return valid ? pos : 0;
}

// Workgroup -> (row, chunk).  With 8 or more rows every row's chunks share
// one XCD (workgroup ids are dealt round-robin over the 8 XCDs), so the
// candidate segments a row writes stay in that XCD's L2 for the select.
__device__ __forceinline__ void map_row_chunk(int rows, int per_row, int& row, int& chunk) {
  const int lin = blockIdx.x;
  if (rows >= kXcds) {
    const int xcd = lin & (kXcds - 1), w = lin >> 3;
    row = xcd + kXcds * (w / per_row);
    chunk = w % per_row;
  } else {
    row = lin / per_row;
    chunk = lin % per_row;
  }
}

static int grid_rows(int rows) { return rows >= kXcds ? (rows + kXcds - 1) / kXcds * kXcds : rows; }

__device__ __forceinline__ void fp8x4_to_f16(uint32_t w, half2_t& lo, half2_t& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
}


__device__ __forceinline__ float key_to_score(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

// Query of a row as packed f16, 16 channels of each head per lane of a quad.
// Query of a row as packed f16, 16 channels of each head per lane of a quad.
// Lane j of a quad (bits b1 b0) keeps head (s ^ 2 b0 ^ b1) in slot s, so the
// quad reduction in quad_score needs three cross-lane adds instead of eight;
// `w_mine` is the weight of head 2 b0 ^ b1, the head the lane ends up with.
__device__ __forceinline__ int quad_head(int slot, int quarter) {
  return slot ^ ((quarter & 1) << 1) ^ (quarter >> 1);
}

__device__ __forceinline__ void load_query_f16(const IndexPass& p, int row, int quarter, half2_t (&q)[kHI][8],
                                               float& w_mine) {
  const uint8_t* qp = p.idx_q + (int64_t)row * (kHI * kDI) + quarter * 16;
#pragma unroll
  for (int s = 0; s < kHI; ++s) {
    const uint4 raw = *reinterpret_cast<const uint4*>(qp + quad_head(s, quarter) * kDI);
    fp8x4_to_f16(raw.x, q[s][0], q[s][1]);
    fp8x4_to_f16(raw.y, q[s][2], q[s][3]);
    fp8x4_to_f16(raw.z, q[s][4], q[s][5]);
    fp8x4_to_f16(raw.w, q[s][6], q[s][7]);
  }
  w_mine = p.idx_w ? p.idx_w[(int64_t)row * kHI + quad_head(0, quarter)] : 1.0f;
}

// This lane's 16 bytes of a key as packed f16 (exact).
__device__ __forceinline__ void key_f16(u32x4_t raw, half2_t (&kh)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) fp8x4_to_f16(raw[j], kh[2 * j], kh[2 * j + 1]);
}

// Score of one key from its 16 bytes in this lane, already as f16 (a lane
// quad holds the key); every lane of the quad returns it.
__device__ __forceinline__ float quad_score_f16(const half2_t (&q)[kHI][8], float w_mine, const half2_t (&kh)[8],
                                                float ks) {
  float d[kHI] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int s = 0; s < kHI; ++s) {
      d[s] = __builtin_amdgcn_fdot2(q[s][2 * j], kh[2 * j], d[s], false);
      d[s] = __builtin_amdgcn_fdot2(q[s][2 * j + 1], kh[2 * j + 1], d[s], false);
    }
  }
  // slot s of the partner lane (lane ^ 1) holds head (s ^ 2) of this lane,
  // and slot 1 of lane ^ 2 the head of slot 0 here
  const float e0 = d[0] + quad_xor1(d[2]);
  const float e1 = d[1] + quad_xor1(d[3]);
  const float f = e0 + quad_xor2(e1);  // full dot product of head quad_head(0, lane)
  float v = w_mine * fmaxf(f, 0.0f);
  v += quad_xor1(v);
  v += quad_xor2(v);
  return ks * v;
}

__device__ __forceinline__ float quad_score(const half2_t (&q)[kHI][8], float w_mine, u32x4_t raw, float ks) {
  half2_t kh[8];
  key_f16(raw, kh);
  return quad_score_f16(q, w_mine, kh, ks);
}

__device__ __forceinline__ float quad_score_at(const IndexPass& p, const half2_t (&q)[kHI][8], float w_mine,
                                               int seq, int quarter, int64_t pos, bool valid) {
  u32x4_t raw = u32x4_t{0, 0, 0, 0};
  float ks = 0.0f;
  if (valid) {
    if (p.pm.pages) {
      const uint32_t e = paged_entry_at(p.pm, seq, pos);
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)p.k8, 0, (int)(p.pm.pool * kDI), kRawBufferWord3);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)p.kscale, 0, (int)(p.pm.pool * 4), kRawBufferWord3);
      raw = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(e * kDI) + quarter * 16, 0, 0);
      ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(e * 4), 0, 0));
    } else {
      raw = *reinterpret_cast<const u32x4_t*>(p.k8 + ((int64_t)seq * p.k_stride + pos) * kDI + quarter * 16);
      ks = p.kscale[(int64_t)seq * p.k_stride + pos];
    }
  }
  return quad_score(q, w_mine, raw, ks);
}


// Exact k-th largest of n keys visited by `visit(n, f)` (f(key) per key), by
// radix steps of 8 bits from bit `top` down.  256 threads; keys are unique
// or the result is the k-th in the multiset order.
template <typename Key, typename Visit>
__device__ Key radix_kth(Visit visit, uint32_t n, uint32_t want, uint32_t* h256, Key* sh_kth, uint32_t* sh_need) {
  const int t = threadIdx.x;
  constexpr int kBits = 8 * (int)sizeof(Key);
  if (t == 0) { *sh_kth = 0; *sh_need = want; }
  for (int shift = kBits - 8; shift >= 0; shift -= 8) {
    h256[t] = 0;
    __syncthreads();
    const Key prefix = *sh_kth;
    const Key hmask = (shift == kBits - 8) ? (Key)0 : (Key)(~(Key)0 << (shift + 8));
    visit(n, [&](Key key) {
      if ((key & hmask) == prefix) hist_add(h256, (uint32_t)(key >> shift) & 255u);
    });
    __syncthreads();
    if (t < 64) {  // one wave: suffix sums over 256 digits, 4 per lane
      const uint32_t nd = *sh_need;
      const uint32_t c0 = h256[4 * t], c1 = h256[4 * t + 1], c2 = h256[4 * t + 2], c3 = h256[4 * t + 3];
      const uint32_t mine = c0 + c1 + c2 + c3;
      uint32_t x = mine;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_down(x, d, 64);
        if (t + d < 64) x += y;
      }
      uint32_t ab = x - mine;
      const uint32_t cs[4] = {c0, c1, c2, c3};
      for (int j = 3; j >= 0; --j) {
        if (ab < nd && ab + cs[j] >= nd) {
          *sh_need = nd - ab;
          *sh_kth = prefix | ((Key)(4 * t + j) << shift);
        }
        ab += cs[j];
      }
    }
    __syncthreads();
  }
  return *sh_kth;
}


// ------------------------------------------------------------------ sample
// Sample size of a row and the rank k_s its threshold is taken at; k_s == 0
// means "no threshold" (every item is a candidate).
__device__ __forceinline__ void sample_plan(int64_t n_items, uint32_t k, int64_t& S, uint32_t& ks) {
  S = n_items < kSample ? n_items : kSample;
  ks = 0;
  if (n_items > (int64_t)k && S > 0) {
    if (S == n_items) {
      // a row this short needs no threshold: every key is a candidate (at
      // most kSample, 128-key chunks), and the select ranks them exactly.
      // A threshold at the k-th sampled score would put the row's answer at
      // the mercy of the sample's MFMA rounding against the scan's.
      ks = 0;
    } else {
      const double want = 2.5 * (double)k * (double)S / (double)n_items + 4.0;
      ks = want >= (double)S ? 0u : (uint32_t)want;
    }
  }
}

// Item of sample slot `slot` (< S): every item when the sample is the whole
// row, otherwise kSample / kSampleRun evenly spaced runs of kSampleRun
// consecutive items, so the sampled keys fill whole cache lines.
constexpr int kSampleRun = 8;
__device__ __forceinline__ int64_t sample_item(int64_t slot, int64_t S, int64_t n_items) {
  if (S == n_items) return slot;
  // S == kSample < n_items here
  return ((slot / kSampleRun) * n_items) / (kSample / kSampleRun) + slot % kSampleRun;
}

// One workgroup of 1,024 threads per row scores the row's sample of 2,048
// keys (256 runs of 8) and turns the order keys, kept in LDS, into the row threshold
// T0: the lower edge, at 20 key bits, of the key bin holding the k_s-th
// largest sample (a 4,096-bin histogram of the top 12 bits, then 256 bins of
// the next 8 within the chosen bin).  T0 = -inf when there is no sample plan
// or fewer than k_s valid samples.
//
// The sample scores only steer T0 (the select kernel checks that at least k
// candidates reached it), so they are computed on fp8 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales) rather than with the scan's
// VALU arithmetic: one MFMA scores 32 sampled keys (B columns) against the
// row's 4 query heads (A rows 0..3, rows 4..31 zero), so the 2,048 keys take
// 64 MFMAs instead of the VALU work of one CU for 2,048 quad scores.
constexpr int kSampleThreads = 1024;
constexpr uint32_t kMfmaUnitScales = 0x7F7F7F7Fu;  // E8M0 127 = 1.0 in every byte
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
template <bool kDirect>
__global__ __launch_bounds__(kSampleThreads) void k_index_sample(IndexPass p) {
  constexpr int NW = kSampleThreads / 64;
  constexpr int kTilesPerWave = kSample / 32 / NW;  // 32-key MFMA tiles per wave
  // Workgroups from the multiple of 8 at or above the row count on are
  // helpers: helper r fetches row r's sample on another CU of the row's XCD,
  // so many of the row's own loads find the lines in that XCD's L2 (one CU
  // alone is bound by its misses in flight; a helper fetching half the
  // sample gained less).
  const int rows_pad = (p.rows + kXcds - 1) / kXcds * kXcds;
  const bool helper = (int)blockIdx.x >= p.rows;
  const int row = helper ? (int)blockIdx.x - rows_pad : (int)blockIdx.x;
  if (row < 0) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int seq = row / p.n_q;
  const int64_t vis = row_vis_positions(p, row);
  const int64_t n_items = row_items_of<kDirect>(p, row, vis);
  int64_t S;
  uint32_t ks;
  sample_plan(n_items, (uint32_t)p.k, S, ks);
  // the row's candidate histogram starts empty (the scan counts into it)
  static_assert(kHistWords == kSampleThreads, "one histogram word per thread");
  if (!helper) p.hist[(int64_t)row * kHistWords + t] = 0u;
  if (ks == 0) {
    if (t == 0 && !helper) p.thresh[row] = -INFINITY;
    return;
  }
  __shared__ uint32_t skey[kSample + 32];  // + a slot per lane for the lanes without a key
  __shared__ uint32_t bins[4096];
  __shared__ uint32_t wsum[NW];
  __shared__ uint32_t sh[3];

  // B operands: lane (l32, half) holds channels 32 half .. +32 of key l32 of
  // each tile (loads issued first: they do not depend on the query).  Every
  // load is an unconditional buffer load: a slot without a key uses the
  // entry index CSA2_MAX_ENTRIES, past the descriptors' ranges, and reads
  // zeros, so no load waits for another.
  // (paged: descriptors over the pool, the entry from the page table, every
  // page-table load issued before the key loads)
  const bool paged = p.pm.pages != nullptr;
  const uint32_t lim = paged ? (uint32_t)p.pm.pool : (uint32_t)CSA2_MAX_ENTRIES;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(paged ? p.k8 : p.k8 + (int64_t)seq * p.k_stride * kDI), 0, (int)(lim * kDI), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(paged ? p.kscale : p.kscale + (int64_t)seq * p.k_stride), 0, (int)(lim * 4), kRawBufferWord3);
  v8i_t B[kTilesPerWave];
  float kv[kTilesPerWave];
  bool valid[kTilesPerWave];
  int64_t pos_u[kTilesPerWave];
  uint32_t page_u[kTilesPerWave];
#pragma unroll
  for (int u = 0; u < kTilesPerWave; ++u) {
    const int64_t slot = (wave * kTilesPerWave + u) * 32 + l32;
    const int64_t item = slot < S ? sample_item(slot, S, n_items) : n_items;
    if constexpr (kDirect) {
      valid[u] = item < n_items;
      pos_u[u] = valid[u] ? item : 0;
    } else {
      pos_u[u] = item_position(p, row, item, n_items, vis, valid[u]);
    }
    page_u[u] = 0;
    if (paged)
      page_u[u] = __builtin_amdgcn_raw_buffer_load_b32(page_row(p.pm, seq),
                                                       valid[u] ? (int)((pos_u[u] >> p.pm.lg) * 4) : (int)(p.pm.stride * 4), 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kTilesPerWave; ++u) {
    const int64_t pos = pos_u[u];
    const uint32_t e = !valid[u] ? lim : paged ? paged_entry(p.pm, page_u[u], pos) : (uint32_t)pos;
    const u32x4_t lo = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(e * kDI) + 32 * half, 0, 0);
    const u32x4_t hi = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(e * kDI) + 32 * half + 16, 0, 0);
    B[u] = v8i_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    kv[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(e * 4), 0, 0));
  }
  if (helper) {  // wait for the lines, then leave
#pragma unroll
    for (int u = 0; u < kTilesPerWave; ++u) asm volatile("" ::"v"(B[u]), "v"(kv[u]));
    return;
  }
  // A operand: row l32 < 4 is query head l32 (channels 32 half .. +32); the
  // other lanes read past the row's 256 bytes and get zeros
  v8i_t A;
  {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.idx_q + (int64_t)row * kHI * kDI), 0, kHI * kDI, kRawBufferWord3);
    const int off = l32 < kHI ? l32 * kDI + 32 * half : kHI * kDI;
    const u32x4_t lo = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
    const u32x4_t hi = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0);
    A = v8i_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  // head weights by vector loads (see load_thresh)
  float w[kHI];
  if (p.idx_w) {
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.idx_w + (int64_t)row * kHI), 0, 4 * kHI, kRawBufferWord3);
#pragma unroll
    for (int h = 0; h < kHI; ++h) w[h] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, 4 * h, 0, 0));
  } else {
#pragma unroll
    for (int h = 0; h < kHI; ++h) w[h] = 1.0f;
  }
  for (int i = t; i < 4096; i += kSampleThreads) bins[i] = 0;
  if (t == 0) { sh[0] = 0xFFFFFFFFu; sh[2] = 0; }
#pragma unroll
  for (int u = 0; u < kTilesPerWave; ++u) {
    v16f_t acc = {};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B[u], acc, 0, 0, 0, kMfmaUnitScales, 0,
                                                          kMfmaUnitScales);
    // The MFMA reads every lane's operands, so it must run with the whole
    // wave active: the empty asm pins it here, in uniform control flow, and
    // the store below is unconditional (instead of a branch on the half
    // that the compiler could sink the MFMA into).
    asm volatile("" ::"v"(acc));
    // lanes 0..31 hold rows 0..3 (the heads) of column l32 in acc[0..3]
    const float sc =
        kv[u] * (w[0] * fmaxf(acc[0], 0.0f) + w[1] * fmaxf(acc[1], 0.0f) + w[2] * fmaxf(acc[2], 0.0f) +
                 w[3] * fmaxf(acc[3], 0.0f));
    skey[half ? kSample + l32 : (wave * kTilesPerWave + u) * 32 + l32] = valid[u] ? score_key(sc) : 0u;
  }
  __syncthreads();
  const uint32_t k0 = skey[2 * t], k1 = skey[2 * t + 1];  // two keys per thread
  if (k0) atomicAdd(&bins[k0 >> 20], 1u);
  if (k1) atomicAdd(&bins[k1 >> 20], 1u);
  __syncthreads();
  // level 1: thread t owns bins 4t .. 4t+3
  const uint4 hb = reinterpret_cast<const uint4*>(bins)[t];
  const uint32_t hv[4] = {hb.x, hb.y, hb.z, hb.w};
  const uint32_t local = hb.x + hb.y + hb.z + hb.w;
  uint32_t total;
  const uint32_t incl = block_incl_scan<NW>(local, wsum, total);
  uint32_t run = total - incl;  // samples in bins above 4t + 3
  if (run < ks && run + local >= ks) {
    for (int j = 3; j >= 0; --j) {
      if (run + hv[j] >= ks) { sh[0] = 4 * t + j; sh[1] = ks - run; break; }
      run += hv[j];
    }
  }
  __syncthreads();
  const uint32_t b1 = sh[0], need = sh[1];
  if (b1 == 0xFFFFFFFFu || b1 == 0u) {  // fewer than k_s valid samples (uniform)
    if (t == 0) p.thresh[row] = -INFINITY;
    return;
  }
  if (t < 256) bins[t] = 0;
  __syncthreads();
  // level 2: the next 8 bits, over the samples in bin b1
  if ((k0 >> 20) == b1) atomicAdd(&bins[(k0 >> 12) & 255u], 1u);
  if ((k1 >> 20) == b1) atomicAdd(&bins[(k1 >> 12) & 255u], 1u);
  __syncthreads();
  const uint32_t c = t < 256 ? bins[t] : 0u;
  uint32_t tot2;
  const uint32_t incl2 = block_incl_scan<NW>(c, wsum, tot2);
  const uint32_t above = tot2 - incl2;  // samples of bin b1 in sub-bins above t
  if (t < 256 && above < need && above + c >= need) sh[2] = t;
  __syncthreads();
  if (t == 0) p.thresh[row] = key_to_score((b1 << 20) | (sh[2] << 12));
}

// ------------------------------------------------------------------ scan

// Workgroup (NQ queries of one sequence, chunk of row_chunk_items items):
// every key of the chunk is scored against each of the queries and those at
// or above a query's threshold T0 become that query's candidates.  kDirect:
// item i is position i (flat keys or block keys); keys and scales are read
// through buffer descriptors whose range ends at the chunk's last item, so
// the hardware returns zeros past it and the loads need no bounds branches.
// Otherwise positions come from a block or position list (one query per
// workgroup).
template <int U, bool kDirect, int NQ, bool kPaged>
__global__ __launch_bounds__(256) void k_index_scan(IndexPass p, int per_row, int n_groups) {
  static_assert(NQ == 1 || kDirect, "queries share a chunk only over direct items");
  static_assert(!kPaged || kDirect, "paged caches are read over direct items");
  // workgroup (group of NQ queries of one sequence, chunk)
  int grp, chunk;
  map_row_chunk(n_groups, per_row, grp, chunk);
  if (grp >= n_groups) return;
  const int qgroups = (p.n_q + NQ - 1) / NQ;
  const int seq = grp / qgroups;
  const int row0 = seq * p.n_q + (grp - seq * qgroups) * NQ;
  const int nq = p.n_q - (row0 - seq * p.n_q) < NQ ? p.n_q - (row0 - seq * p.n_q) : NQ;
  const int64_t csize = row_chunk_items_of<kDirect>(p, row0);  // shared by the rows of a sequence
  const int64_t base = (int64_t)chunk * csize;
  int64_t vis[NQ], n_items[NQ], end = 0;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    vis[i] = i < nq ? row_vis_positions(p, row0 + i) : 0;
    n_items[i] = i < nq ? row_items_of<kDirect>(p, row0 + i, vis[i]) : 0;
    const int64_t e = base + csize < n_items[i] ? base + csize : n_items[i];
    end = e > end ? e : end;
  }
  if (base >= end) return;

  // candidates are staged in LDS and stored after the loop: a global store
  // inside it would make every later wait for the key loads also wait for
  // the store (one counter covers both on gfx9)
  __shared__ uint32_t n_hit[NQ];
  __shared__ uint64_t hits[NQ][kSeg];
  if (threadIdx.x < NQ) n_hit[threadIdx.x] = 0;
  const int quarter = threadIdx.x & 3;
  const int sub = threadIdx.x >> 2;  // item within a 64-item step
  half2_t q[NQ][kHI][8];
  float w_mine[NQ], T0[NQ];  // loaded after the first keys: their loads overlap
  const uint8_t* kb = p.k8 + (int64_t)seq * p.k_stride * kDI;
  const float* sb = p.kscale + (int64_t)seq * p.k_stride;
  // (used by the kDirect loads only.)  Paged: descriptors over the pool, and
  // lane j holds the page-table value of the chunk's page j: a batch of
  // kStep items lies in one page (pages hold at least 128 entries, batches
  // start at multiples of kStep), so its entries are one page's consecutive
  // entries
  constexpr bool paged = kPaged;
  const uint32_t lim = paged ? (uint32_t)p.pm.pool : (uint32_t)end;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(paged ? p.k8 : kb), 0, (int)(lim * kDI), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(paged ? p.kscale : sb), 0, (int)(lim * 4), kRawBufferWord3);
  uint32_t page_lane = 0;
  if constexpr (paged) {
    const int64_t pg = (base >> p.pm.lg) + (threadIdx.x & 63);
    page_lane = __builtin_amdgcn_raw_buffer_load_b32(page_row(p.pm, seq), (int)(pg * 4), 0, 0);
  }

  // U items per lane quad per batch; two batches in flight (double buffer)
  struct Batch {
    u32x4_t raw[U];
    float ks[U];
  };
  auto load = [&](Batch& B, int64_t it0) {
    uint32_t page = 0;
    if constexpr (paged) page = (uint32_t)__shfl((int)page_lane, (int)(((it0 >> p.pm.lg) - (base >> p.pm.lg)) & 63), 64);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t item = it0 + u * 64 + sub;
      if constexpr (kDirect) {
        const uint32_t e = !paged ? (uint32_t)item : item < end ? paged_entry(p.pm, page, item) : lim;
        B.raw[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(e * kDI) + quarter * 16, 0, kLoadNonTemporal);
        B.ks[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(e * 4), 0, 0));
      } else {
        bool valid;
        const int64_t pos = item_position(p, row0, item, end, vis[0], valid);
        if (valid) {
          B.raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + pos * kDI + quarter * 16));
          B.ks[u] = sb[pos];
        } else {
          B.raw[u] = u32x4_t{0, 0, 0, 0};
          B.ks[u] = 0.0f;
        }
      }
    }
  };
  auto score = [&](const Batch& B, int64_t it0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      half2_t kh[8];
      key_f16(B.raw[u], kh);  // converted once for every query of the group
      const int64_t item = it0 + u * 64 + sub;
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const float sc = quad_score_f16(q[i], w_mine[i], kh, B.ks[u]);
        bool take = quarter == 0 && item < n_items[i] && item < base + csize && sc >= T0[i];
        if constexpr (!kDirect) {
          if (take) {  // invalid list entries never become candidates
            bool valid;
            (void)item_position(p, row0, item, end, vis[0], valid);
            take = valid;
          }
        }
        if (take) {
          const uint32_t at = atomicAdd(&n_hit[i], 1u);
          if (at < (uint32_t)kSeg) hits[i][at] = select_key(score_key(sc), (uint32_t)item);
        }
      }
    }
  };
  constexpr int kStep = 64 * U;
  Batch A, Bb;
  int64_t it = base;
  load(A, it);
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int r = i < nq ? row0 + i : row0;
    load_query_f16(p, r, quarter, q[i], w_mine[i]);
    T0[i] = i < nq ? load_thresh(p, r) : INFINITY;
  }
  __syncthreads();  // n_hit is initialised
  // kDirect loads past the chunk read zeros without touching memory, so they
  // are issued unconditionally and every path has the same loads in flight
  while (true) {
    const int64_t nxt = it + kStep;
    if (kDirect || nxt < end) load(Bb, nxt);
    score(A, it);
    if (nxt >= end) break;
    const int64_t nxt2 = nxt + kStep;
    if (kDirect || nxt2 < end) load(A, nxt2);
    score(Bb, nxt);
    if (nxt2 >= end) break;
    it = nxt2;
  }
  __syncthreads();
  static_assert(kSeg <= 256, "one staged candidate per thread");
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    if (i >= nq || base >= n_items[i]) continue;
    const int64_t r = row0 + i;
    uint64_t* seg = p.seg_list + (r * p.max_chunks + chunk) * kSeg;
    const uint32_t n = n_hit[i] < (uint32_t)kSeg ? n_hit[i] : (uint32_t)kSeg;
    if (threadIdx.x < n) {
      const uint64_t h = hits[i][threadIdx.x];
      seg[threadIdx.x] = h;
      // 16-bit bins: a row whose bins could overflow has more candidates
      // than the select's fast path takes, which then ignores the histogram
      const uint32_t b = hist_bin((uint32_t)(h >> 32), score_key(T0[i]));
      atomicAdd(&p.hist[r * kHistWords + (b >> 1)], 1u << (16 * (b & 1u)));
    }
    if (threadIdx.x == 0) p.seg_count[r * p.max_chunks + chunk] = n_hit[i];
  }
}

// A pointer every lane holds the same value of, moved to scalar registers.
__device__ __forceinline__ void* uniform_ptr(const void* q) {
  const uint64_t v = reinterpret_cast<uint64_t>(q);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}
// The scan on fp8 MFMA (direct items): each 32-key tile of the chunk is
// scored against the 4 NQ heads of the NQ queries in one
// v_mfma_scale_f32_32x32x64_f8f6f4 (heads as A rows, keys as B columns,
// exact fp8 codes, unit scales, binary32 accumulation) instead of 16 fdot2
// per key quarter and query on VALU.  Lane (l32, half) holds bytes
// 32 half .. +32 of key l32 of the tile (B) and of head row l32 (A): row
// 4 i + h is head h of query i.  The output gives the four head dots of query
// i for key l32 in the lanes of half i % 2, registers 4 (i / 2) .. +3, so a
// lane scores queries half, half + 2, ...  Wave w takes tiles w, w + 4, ...
// of the chunk with kScanTiles tiles in flight.
constexpr int kScanTiles = 4;
template <int NQ, bool kPaged>
__global__ __launch_bounds__(256) void k_index_scan_mfma(IndexPass p, int per_row, int n_groups) {
  constexpr int NG = (NQ + 1) / 2;  // queries per lane, at most
  int grp, chunk;
  map_row_chunk(n_groups, per_row, grp, chunk);
  if (grp >= n_groups) return;
  const int qgroups = (p.n_q + NQ - 1) / NQ;
  const int seq = grp / qgroups;
  const int row0 = seq * p.n_q + (grp - seq * qgroups) * NQ;
  const int nq = p.n_q - (row0 - seq * p.n_q) < NQ ? p.n_q - (row0 - seq * p.n_q) : NQ;
  const int64_t csize = row_chunk_items_of<true>(p, row0);  // shared by the rows of a sequence
  const int64_t base = (int64_t)chunk * csize;
  int64_t lim_q[NQ], end = 0;  // items of query i in this chunk end at lim_q[i]
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int64_t n = i < nq ? row_items_of<true>(p, row0 + i, row_vis_positions(p, row0 + i)) : 0;
    lim_q[i] = base + csize < n ? base + csize : n;
    end = lim_q[i] > end ? lim_q[i] : end;
  }
  if (base >= end) return;

  __shared__ uint32_t n_hit[NQ];
  __shared__ uint64_t hits[NQ][kSeg];
  if (threadIdx.x < NQ) n_hit[threadIdx.x] = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const uint8_t* kb = p.k8 + (int64_t)seq * p.k_stride * kDI;
  const float* sb = p.kscale + (int64_t)seq * p.k_stride;
  // (the descriptors' fields are read through readfirstlane: they are
  // uniform, and a descriptor the compiler cannot prove uniform costs a
  // waterfall loop around every load)
  const uint32_t lim = (uint32_t)__builtin_amdgcn_readfirstlane((int)(kPaged ? (uint32_t)p.pm.pool : (uint32_t)end));
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(kPaged ? p.k8 : kb), 0, (int)(lim * kDI), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(kPaged ? p.kscale : sb), 0, (int)(lim * 4), kRawBufferWord3);
  // paged: lane j holds the table value of the chunk's page j (a tile lies
  // in one page: pages hold at least 128 entries, tiles start at multiples
  // of 32)
  uint32_t page_lane = 0;
  if constexpr (kPaged) {
    const int64_t pg = (base >> p.pm.lg) + lane;
    page_lane = __builtin_amdgcn_raw_buffer_load_b32(page_row(p.pm, seq), (int)(pg * 4), 0, 0);
  }
  const int n_tiles = (int)((end - base + 31) >> 5);
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + 3) >> 2 : 0;

  struct Tile {
    u32x4_t lo, hi;
    float ks;
  };
  // tile m of this wave; past the chunk the loads read zeros without
  // touching memory (the descriptors end at the chunk, or at the pool)
  auto load_tile = [&](Tile& T, int m) {
    const int64_t item = base + 32 * (int64_t)(wave + 4 * m) + l32;
    uint32_t e;
    if constexpr (kPaged) {
      const uint32_t page = (uint32_t)__shfl((int)page_lane, (int)(((item >> p.pm.lg) - (base >> p.pm.lg)) & 63), 64);
      e = item < end ? paged_entry(p.pm, page, item) : lim;
    } else {
      e = item < end ? (uint32_t)item : lim;
    }
    // (the scale first: the wait for the key bytes then covers it too)
    T.ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(e * 4), 0, 0));
    T.lo = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(e * kDI) + 32 * half, 0, kLoadNonTemporal);
    T.hi = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(e * kDI) + 32 * half + 16, 0, kLoadNonTemporal);
  };
  // A operand: head row l32 of query l32 / 4 (rows past the group's queries
  // read zeros past the descriptor).  These loads, the weights and the
  // thresholds go out before the tiles: every load is unconditional, so the
  // waits for them inside the tile loop do not wait for tile data.
  v8i_t A;
  {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.idx_q + (int64_t)row0 * kHI * kDI), 0, nq * kHI * kDI, kRawBufferWord3);
    const int off = l32 < 4 * NQ ? (l32 >> 2) * kHI * kDI + (l32 & 3) * kDI + 32 * half : NQ * kHI * kDI;
    const u32x4_t lo = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
    const u32x4_t hi = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0);
    A = v8i_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  // this lane's queries i = 2 g + half: head weights, threshold, item limit
  float wq[NG][kHI], t0q[NG];
  int64_t limq[NG];
  float T0[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) T0[i] = load_thresh(p, row0 + (i < nq ? i : 0));
  {
    const bool has_w = p.idx_w != nullptr;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(has_w ? p.idx_w + (int64_t)row0 * kHI : p.thresh), 0, has_w ? nq * kHI * 4 : 0, kRawBufferWord3);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int i = 2 * g + half;
#pragma unroll
      for (int h = 0; h < kHI; ++h) {
        const float wl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, (i * kHI + h) * 4, 0, 0));
        wq[g][h] = has_w ? wl : 1.0f;
      }
    }
  }
  // (kept in this order: waiting for the setup loads must not wait for tiles)
  __builtin_amdgcn_sched_barrier(0);
  Tile T[kScanTiles];
#pragma unroll
  for (int s = 0; s < kScanTiles; ++s) load_tile(T[s], s);
#pragma unroll
  for (int i = 0; i < NQ; ++i) T0[i] = i < nq ? T0[i] : INFINITY;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int ilo = 2 * g, ihi = 2 * g + 1 < NQ ? 2 * g + 1 : 2 * g;
    t0q[g] = half ? (2 * g + 1 < NQ ? T0[ihi] : INFINITY) : T0[ilo];
    limq[g] = half ? (2 * g + 1 < NQ ? lim_q[ihi] : 0) : lim_q[ilo];
  }
  __syncthreads();  // n_hit is initialised

  auto score_tile = [&](const Tile& Tt, int m) {
    const v8i_t Bop = v8i_t{(int)Tt.lo[0], (int)Tt.lo[1], (int)Tt.lo[2], (int)Tt.lo[3],
                            (int)Tt.hi[0], (int)Tt.hi[1], (int)Tt.hi[2], (int)Tt.hi[3]};
    v16f_t acc = {};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, Bop, acc, 0, 0, 0, kMfmaUnitScales, 0,
                                                          kMfmaUnitScales);
    // the whole wave runs the MFMA (uniform control flow, see the sample)
    asm volatile("" ::"v"(acc));
    const int64_t item = base + 32 * (int64_t)(wave + 4 * m) + l32;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const float sc = Tt.ks * (wq[g][0] * fmaxf(acc[4 * g], 0.0f) + wq[g][1] * fmaxf(acc[4 * g + 1], 0.0f) +
                                wq[g][2] * fmaxf(acc[4 * g + 2], 0.0f) + wq[g][3] * fmaxf(acc[4 * g + 3], 0.0f));
      if (item < limq[g] && sc >= t0q[g]) {
        const int i = 2 * g + half;
        const uint32_t at = atomicAdd(&n_hit[i], 1u);
        if (at < (uint32_t)kSeg) hits[i][at] = select_key(score_key(sc), (uint32_t)item);
      }
    }
  };
  // whole groups of kScanTiles tiles, with no branch between the loads (a
  // tile past the chunk reads zeros and its items fail the item limit), so
  // each score waits only for its own tile
  for (int m0 = 0; m0 < my_tiles; m0 += kScanTiles) {
#pragma unroll
    for (int s = 0; s < kScanTiles; ++s) {
      score_tile(T[s], m0 + s);
      load_tile(T[s], m0 + s + kScanTiles);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    if (i >= nq || base >= lim_q[i]) continue;
    const int64_t r = row0 + i;
    uint64_t* seg = p.seg_list + (r * p.max_chunks + chunk) * kSeg;
    const uint32_t n = n_hit[i] < (uint32_t)kSeg ? n_hit[i] : (uint32_t)kSeg;
    if (threadIdx.x < n) {
      const uint64_t h = hits[i][threadIdx.x];
      seg[threadIdx.x] = h;
      const uint32_t b = hist_bin((uint32_t)(h >> 32), score_key(T0[i]));
      atomicAdd(&p.hist[r * kHistWords + (b >> 1)], 1u << (16 * (b & 1u)));
    }
    if (threadIdx.x == 0) p.seg_count[r * p.max_chunks + chunk] = n_hit[i];
  }
}

// ------------------------------------------------------------------ select
__device__ __forceinline__ int32_t item_to_position(const IndexPass& p, int row, uint32_t item) {
  if (p.source == kItemsDirect) return (int32_t)item;
  if (p.source == kItemsBlocks) return 8 * p.blocks[(int64_t)row * CSA2_MAX_K + (item >> 3)] + (int32_t)(item & 7u);
  return p.list[(int64_t)row * p.list_len + item];
}

// LDS slot of bitmap word w: thread t reads words 16t .. 16t+15, so word
// 16t + j sits at j * 256 + t and each of those reads is conflict-free.
__device__ __forceinline__ uint32_t bitmap_slot(uint32_t w) { return (w & 15u) * 256u + (w >> 4); }
static_assert(kBitmapItems / 32 == 16 * 256, "bitmap words: 16 per select thread");
static_assert(kBitmapItems / 32 * 4 <= 256 * 16 * 8, "the word prefixes fit in the candidate array");

// kPer candidates per thread, 256 kPer in all: 16 serves k <= 1,024 (about
// 2.5 k candidates reach the sampled threshold), 32 the 2,048-block stage
template <int kPer>
__device__ __forceinline__ void select_row(const IndexPass& p, const int row) {
  constexpr int kSelCap = 256 * kPer;
  const int t = threadIdx.x, quarter = t & 3;
  const int wave = t >> 6, lane = t & 63;
  // the loads that need only the row go out first: the row's candidate
  // histogram (filled by the scan; every wave holds all of it, lane l the
  // words 16 l .. 16 l + 15, bins 32 l .. 32 l + 31) and the chunk counts
  // (every row has room for 128; chunks past the row's last are masked
  // below)
  uint32_t hw[16];
  {
    const uint4* h4 = reinterpret_cast<const uint4*>(p.hist + (int64_t)row * kHistWords) + 4 * lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 a = h4[i];
      hw[4 * i] = a.x;
      hw[4 * i + 1] = a.y;
      hw[4 * i + 2] = a.z;
      hw[4 * i + 3] = a.w;
    }
  }
  const uint32_t* cnt_row = p.seg_count + (int64_t)row * p.max_chunks;
  const uint64_t* segs = p.seg_list + (int64_t)row * p.max_chunks * kSeg;
  constexpr int kSpecCh = kPer <= 16 ? kSpecChunks : 2 * kSpecChunks;  // chunks gathered in one round trip
  const uint32_t cnt_lane = cnt_row[lane];
  const uint32_t cnt_lane_b = kSpecCh > 64 ? cnt_row[lane + 64] : 0u;  // (every row has room for 128)
  const int seq = row / p.n_q;
  const int64_t vis = row_vis_positions(p, row);
  const int64_t n_items = row_items(p, row, vis);
  const int64_t csize = row_chunk_items(p, row);
  const int nch = (int)scan_chunk_count(n_items, csize);
  const uint32_t k = (uint32_t)p.k;

  __shared__ uint32_t seg_start[kMaxChunks + 1];
  __shared__ uint64_t lc[kSelCap];
  __shared__ uint32_t bitmap[kBitmapItems / 32];
  __shared__ uint32_t win[CSA2_MAX_K];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t h2048[2048];
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t sh3[3];
  __shared__ uint64_t bin_keys[64];
  __shared__ uint32_t hsrc[4][16];
  __shared__ uint64_t sh_kth;
  __shared__ uint32_t sh_need, sh_binn;

  // Rows of at most kSpecCh chunks (64 for k <= 1,024, 128 for the 2,048-block
  // stage) load the first kSpecSlots slots of every segment together with
  // the counts (one memory round trip), two segments per wave instruction:
  // wave w takes chunks 2 (w + 4 j) + lane / 32, lane % 32 their slots
  // 2 (lane % 32) and the next.  Segments hold about 40 candidates on
  // average; fuller ones load the rest afterwards.  Each wave holds the
  // counts of chunks l and l + 64 in lane l, so its own prefix sums give
  // every chunk's start without a workgroup scan.
  const bool spec = nch <= kSpecCh;
  uint4 sv[kSpecCh / 8];
  uint32_t cnt_a = 0, cnt_b = 0, start_a = 0, start_b = 0;
  uint32_t total;
  bool over = false, more = false;
  if (spec) {
    cnt_a = lane < nch ? cnt_lane : 0u;
    cnt_b = lane + 64 < nch ? cnt_lane_b : 0u;
#pragma unroll
    for (int j = 0; j < kSpecCh / 8; ++j) {
      const int ch = 2 * (wave + 4 * j) + (lane >> 5);
      sv[j] = ch < nch ? *reinterpret_cast<const uint4*>(segs + (int64_t)ch * kSeg + 2 * (lane & 31))
                       : make_uint4(0, 0, 0, 0);
    }
    const uint32_t incl_a = wave_incl_add(cnt_a);
    const uint32_t tot_a = (uint32_t)__shfl((int)incl_a, 63, 64);
    start_a = incl_a - cnt_a;
    total = tot_a;
    if constexpr (kSpecCh > 64) {
      const uint32_t incl_b = wave_incl_add(cnt_b);
      start_b = tot_a + incl_b - cnt_b;
      total = tot_a + (uint32_t)__shfl((int)incl_b, 63, 64);
    }
    over = __any(cnt_a > (uint32_t)kSeg || cnt_b > (uint32_t)kSeg);
    more = __any(cnt_a > (uint32_t)kSpecSlots || cnt_b > (uint32_t)kSpecSlots);
  } else {
    // segment counts: thread t owns chunks 16t .. 16t+15
    uint32_t c[16], local = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int ch = 16 * t + j;
      c[j] = ch < nch ? cnt_row[ch] : 0u;
      over |= c[j] > (uint32_t)kSeg;
      local += c[j];
    }
    over = __syncthreads_or(over);
    uint32_t run = block_incl_scan_256(local, wsum, total) - local;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int ch = 16 * t + j;
      if (ch < nch) seg_start[ch] = run;
      run += c[j];
    }
    if (t == 0) seg_start[nch] = total;
    __syncthreads();
  }

  const float T0 = n_items > 0 ? load_thresh(p, row) : -INFINITY;  // written by the sample pass
  const bool fast = !over && total <= (uint32_t)kSelCap && (total >= k || T0 == -INFINITY);
  uint32_t n_win = 0;
  if (fast) {
    if (t == 0) {  // (ordered before their users by the barrier after the gather)
      sh3[0] = 0xFFFFFFFFu;
      sh_binn = 0;
    }
    const bool use_bitmap = n_items <= (int64_t)kBitmapItems;
    if (use_bitmap) {
      uint4* bm4 = reinterpret_cast<uint4*>(bitmap);
      for (int i = t; i < kBitmapItems / 128; i += 256) bm4[i] = make_uint4(0, 0, 0, 0);
    }
    if (spec) {  // the slots loaded above: keep the first count of each chunk
      // count and start of chunk ch (< 128; every lane takes both shuffles)
      auto chunk_of = [&](int ch, uint32_t& n, uint32_t& base) {
        const int l = ch & 63;
        const uint32_t na = (uint32_t)__shfl((int)cnt_a, l, 64), sa = (uint32_t)__shfl((int)start_a, l, 64);
        uint32_t nb = 0, sb = 0;
        if constexpr (kSpecCh > 64) {
          nb = (uint32_t)__shfl((int)cnt_b, l, 64);
          sb = (uint32_t)__shfl((int)start_b, l, 64);
        }
        n = ch < 64 ? na : nb;
        base = ch < 64 ? sa : sb;
      };
#pragma unroll
      for (int j = 0; j < kSpecCh / 8; ++j) {
        const int ch = 2 * (wave + 4 * j) + (lane >> 5);
        uint32_t n, base;
        chunk_of(ch, n, base);
        const uint32_t s0 = 2u * (lane & 31);
        if (ch < nch) {
          if (s0 < n) lc[base + s0] = ((uint64_t)sv[j].y << 32) | sv[j].x;
          if (s0 + 1u < n) lc[base + s0 + 1] = ((uint64_t)sv[j].w << 32) | sv[j].z;
        }
      }
      if (more) {  // the slots past kSpecSlots of fuller segments
        for (int ch = wave; ch < nch; ch += 4) {
          uint32_t n, base;
          chunk_of(ch, n, base);
          const uint32_t i = kSpecSlots + lane;
          if (i < n) lc[base + i] = segs[(int64_t)ch * kSeg + i];
        }
      }
    }
    // otherwise gather the segments: wave w copies chunks w, w + 4, ...,
    // eight chunks (up to 16 independent loads per lane) at a time
    for (int c0 = spec ? nch : wave; c0 < nch; c0 += 32) {
      uint64_t v[8][2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ch = c0 + 4 * j;
        const uint32_t n = ch < nch ? seg_start[ch + 1] - seg_start[ch] : 0u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t i = lane + 64 * h;
          v[j][h] = i < n ? segs[(int64_t)ch * kSeg + i] : 0ull;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ch = c0 + 4 * j;
        const uint32_t n = ch < nch ? seg_start[ch + 1] - seg_start[ch] : 0u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t i = lane + 64 * h;
          if (i < n) lc[seg_start[ch] + i] = v[j][h];
        }
      }
    }
    __syncthreads();
    // candidates into registers: thread t holds lc[t + 256 i]
    // (the passes over the keys stop after the last slot any thread fills:
    // a row has about 1.5 k candidates in 256 kPer slots)
    const int nslots = (int)((total + 255u) / 256u);
    uint64_t key[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const uint32_t g = t + 256 * i;
      key[i] = i < nslots && g < total ? lc[g] : 0ull;  // 0 is below every candidate key
    }
    uint64_t kth = 1ull;
    if (total > k) {
      // the bin holding the k-th largest key, from the histogram: bins above
      // it hold fewer than k keys, with it at least k.  When it is a proper
      // bin with a few keys, the k-th key is ranked among those alone;
      // otherwise (the top bin, which also takes scores far above T0) the
      // radix over every candidate decides.  Every wave finds the bin in its
      // own copy of the histogram and ranks the bin's keys itself, so the
      // only barrier is the one that publishes those keys.
      uint32_t hl = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) hl += (hw[j] & 0xFFFFu) + (hw[j] >> 16);
      const uint32_t hincl = wave_incl_add(hl);
      const uint32_t htot = (uint32_t)__builtin_amdgcn_readlane((int)hincl, 63);
      const uint32_t above_l = htot - hincl;  // keys in bins above 32 lane + 31
      // the lane whose 32 bins hold the k-th key, then (its words through
      // LDS, one bin per lane) the bin
      const unsigned long long hit = __ballot(htot == total && above_l < k && above_l + hl >= k);
      uint32_t kb_bin = 0xFFFFFFFFu, need = 0, in_bin = 0;
      if (hit) {
        const int src = __ffsll((long long)hit) - 1;
        const uint32_t above_src = (uint32_t)__builtin_amdgcn_readlane((int)above_l, src);
        if (lane == src) {
#pragma unroll
          for (int i = 0; i < 16; ++i) hsrc[wave][i] = hw[i];
        }
        __builtin_amdgcn_wave_barrier();
        const uint32_t wj = hsrc[wave][(lane & 31) >> 1];
        const uint32_t c = lane < 32 ? (wj >> (16 * (lane & 1))) & 0xFFFFu : 0u;
        const uint32_t ci = wave_incl_add(c);
        const uint32_t above_j = above_src + (uint32_t)__builtin_amdgcn_readlane((int)ci, 31) - ci;
        const unsigned long long hj = __ballot(lane < 32 && above_j < k && above_j + c >= k);
        if (hj) {
          const int j = __ffsll((long long)hj) - 1;
          kb_bin = 32 * src + j;
          need = k - (uint32_t)__builtin_amdgcn_readlane((int)above_j, j);
          in_bin = (uint32_t)__builtin_amdgcn_readlane((int)c, j);
        }
      }
      bool ranked = false;
      if (kb_bin < (uint32_t)(kHistBins - 1) && in_bin <= 64u) {
        // the bin's keys into LDS, then lane l ranks key l among them with
        // register reads of the other lanes' keys
        const uint32_t t0key = score_key(T0);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          if (i < nslots && key[i] != 0ull && hist_bin((uint32_t)(key[i] >> 32), t0key) == kb_bin) {
            const uint32_t slot = atomicAdd(&sh_binn, 1u);
            if (slot < 64u) bin_keys[slot] = key[i];
          }
        }
        __syncthreads();
        const uint64_t mine = lane < (int)in_bin ? bin_keys[lane] : 0ull;
        uint32_t rank = 0;
        for (uint32_t j = 0; j < in_bin; ++j) {
          const uint64_t other = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mine >> 32), (int)j) << 32) |
                                 (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine, (int)j);
          rank += other > mine ? 1u : 0u;
        }
        // (keys are unique: one lane holds rank need - 1; the same in every wave)
        const unsigned long long pick = __ballot(lane < (int)in_bin && rank == need - 1);
        if (pick) {
          const int src = __ffsll((long long)pick) - 1;
          kth = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mine >> 32), src) << 32) |
                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine, src);
          ranked = true;
        }
      }
      if (!ranked) kth = block_kth_regs<kPer>(key, k, h2048, wsum, sh3);
    }
    // winners: every candidate key >= kth
    if (use_bitmap) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (i < nslots && key[i] >= kth) {
          const uint32_t it = select_key_pos(key[i]);
          atomicOr(&bitmap[bitmap_slot(it >> 5)], 1u << (it & 31u));
        }
      }
      __syncthreads();
      // thread t owns words 16t .. 16t+15 (512 items)
      const uint32_t nwords = (uint32_t)((n_items + 31) / 32);
      uint32_t wb[16], cnt_t = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t wi = 16 * t + j;
        wb[j] = wi < nwords ? bitmap[bitmap_slot(wi)] : 0u;
        cnt_t += __builtin_popcount(wb[j]);
      }
      uint32_t tot;
      uint32_t o = block_incl_scan_256(cnt_t, wsum, tot) - cnt_t;
      n_win = tot;
      // winners before each word, into LDS (over lc: the candidates are in
      // registers now); then each winner's rank is that count plus the set
      // bits below it in its word, and it goes to its slot of `win` (the
      // global stores follow in one coalesced pass)
      uint32_t* wpre = reinterpret_cast<uint32_t*>(lc);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        wpre[bitmap_slot(16 * t + j)] = o;
        o += __builtin_popcount(wb[j]);
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (i < nslots && key[i] >= kth) {
          const uint32_t it = select_key_pos(key[i]), ws = bitmap_slot(it >> 5);
          win[wpre[ws] + __builtin_popcount(bitmap[ws] & ((1u << (it & 31u)) - 1u))] = it;
        }
      }
      __syncthreads();
    } else {
      // compaction, then a bitonic sort padded to a power of two
      if (t == 0) sh_need = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (i < nslots && key[i] >= kth) win[atomicAdd(&sh_need, 1u)] = select_key_pos(key[i]);
      }
      __syncthreads();
      n_win = sh_need;
      uint32_t n2 = 1;
      while (n2 < n_win) n2 <<= 1;
      for (uint32_t i = n_win + t; i < n2; i += 256) win[i] = 0xFFFFFFFFu;
      __syncthreads();
      for (uint32_t size = 2; size <= n2; size <<= 1) {
        for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
          for (uint32_t i = t; i < n2 / 2; i += 256) {
            const uint32_t lo = 2 * i - (i & (stride - 1));
            const uint32_t hi = lo + stride;
            const bool asc = (lo & size) == 0;
            const uint32_t a = win[lo], b = win[hi];
            if ((a > b) == asc) { win[lo] = b; win[hi] = a; }
          }
          __syncthreads();
        }
      }
    }
  } else {
    // exact recompute of this row (rare): radix steps over recomputed keys
    if (t == 0) atomicAdd(p.fallbacks, 1u);
    half2_t q[kHI][8];
    float w_mine;
    load_query_f16(p, row, quarter, q, w_mine);
    auto visit = [&](uint32_t n, auto&& f) {
      for (uint32_t base = 0; base < n; base += 64) {
        const uint32_t item = base + (t >> 2);
        bool valid = false;
        const int64_t pos = item < n ? item_position(p, row, item, n, vis, valid) : 0;
        const float sc = quad_score_at(p, q, w_mine, seq, quarter, pos, valid);
        if (valid && quarter == 0) f(select_key(score_key(sc), item));
      }
    };
    const uint32_t ni = (uint32_t)n_items;
    uint64_t kth = 0;
    // winners must be valid items: count them first
    uint32_t n_valid = 0;
    {
      uint32_t mine = 0;
      for (uint32_t base = 0; base < ni; base += 64) {
        const uint32_t item = base + (t >> 2);
        bool valid = false;
        if (item < ni && quarter == 0) (void)item_position(p, row, item, ni, vis, valid);
        mine += valid ? 1u : 0u;
      }
      (void)block_incl_scan_256(mine, wsum, n_valid);
    }
    if (n_valid > k) kth = radix_kth<uint64_t>(visit, ni, k, h256, &sh_kth, &sh_need);
    for (uint32_t base = 0; base < ni; base += 64) {
      const uint32_t item = base + (t >> 2);
      bool valid = false;
      const int64_t pos = item < ni ? item_position(p, row, item, ni, vis, valid) : 0;
      const float sc = quad_score_at(p, q, w_mine, seq, quarter, pos, valid);
      const bool f = valid && quarter == 0 && select_key(score_key(sc), item) >= kth;
      uint32_t nr;
      const uint32_t o = block_incl_scan_256(f ? 1u : 0u, wsum, nr) - (f ? 1u : 0u);
      if (f && n_win + o < (uint32_t)CSA2_MAX_K) win[n_win + o] = item;
      n_win += nr;
    }
    if (n_win > k) n_win = k;
    __syncthreads();
  }

  // positions of the winners, in ascending order (then -1 up to k, except
  // for block ids); rows that start on 16 bytes take four per store
  int32_t* orow = p.out + (int64_t)row * p.out_stride;
  const uint32_t n_out = p.block_level ? n_win : k;
  if ((reinterpret_cast<uintptr_t>(orow) & 15u) == 0) {
    for (uint32_t j = 4 * t; j < n_out; j += 1024) {
      int32_t v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = j + e < n_win ? item_to_position(p, row, win[j + e]) : -1;
      if (j + 4 <= n_out) {
        *reinterpret_cast<int4*>(orow + j) = make_int4(v[0], v[1], v[2], v[3]);
      } else {
        for (uint32_t e = 0; j + e < n_out; ++e) orow[j + e] = v[e];
      }
    }
  } else {
    for (uint32_t j = t; j < n_out; j += 256) orow[j] = j < n_win ? item_to_position(p, row, win[j]) : -1;
  }
  if (p.out_count && t == 0) p.out_count[row] = (int32_t)n_win;
  if (p.out_pool) {
    // the 8 positions of kept block b (-1 past the visible ones or past the
    // kept blocks) at 8 b .. 8 b + 7: two 16-byte stores per block when the
    // row starts on 16 bytes
    const int32_t n_pool = min(p.pool_stride, (int32_t)kMaxPool);
    int32_t* prow = p.out_pool + (int64_t)row * p.pool_stride;
    auto pool_at = [&](int32_t j) -> int32_t {
      if ((uint32_t)(j >> 3) >= n_win) return -1;
      const int64_t pos = 8 * (int64_t)win[j >> 3] + (j & 7);
      return pos < vis ? (int32_t)pos : -1;
    };
    if ((reinterpret_cast<uintptr_t>(prow) & 15u) == 0 && (n_pool & 7) == 0) {
      for (int32_t b = t; b < n_pool / 8; b += 256) {
        const int64_t base = (uint32_t)b < n_win ? 8 * (int64_t)win[b] : vis;
        int32_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = base + e < vis ? (int32_t)(base + e) : -1;
        int4* d = reinterpret_cast<int4*>(prow + 8 * b);
        d[0] = make_int4(v[0], v[1], v[2], v[3]);
        d[1] = make_int4(v[4], v[5], v[6], v[7]);
      }
    } else {
      for (int32_t j = t; j < n_pool; j += 256) prow[j] = pool_at(j);
    }
  }
}

template <int kPer>
__global__ __launch_bounds__(256) void k_index_select(IndexPass p) {
  select_row<kPer>(p, blockIdx.x);
}

// The select of a decode index pass with the window tiles of the group's
// attention in the same launch: workgroups below p.rows select, each of the
// others takes one window tile of one (layer, row).  The select occupies a
// workgroup per row and leaves the rest of the chip idle, and the window
// tiles need nothing it computes.
template <int kPer>
__global__ __launch_bounds__(256) void k_index_select_window(IndexPass p, AttnPass a) {
  if ((int)blockIdx.x < p.rows) {
    select_row<kPer>(p, blockIdx.x);
    return;
  }
  __shared__ __attribute__((aligned(16))) TileLds s;
  const int n_win_tiles = a.n_tiles - (a.n_idx + kAttnSplit - 1) / kAttnSplit;
  const int per_row = a.n_layers * n_win_tiles;
  // with a multiple of 8 rows, the tiles of row r run on XCD r mod 8 (the
  // XCD of its selected-entry tiles), so the merge finds every partial of
  // the row in one L2
  const int w = blockIdx.x - p.rows;
  int row, jj;
  if (p.rows >= kXcds && p.rows % kXcds == 0) {
    const int xcd = w & (kXcds - 1), k = w >> 3;
    row = xcd + kXcds * (k / per_row);
    jj = k % per_row;
  } else {
    row = w / per_row;
    jj = w - row * per_row;
  }
  window_tile(a, row, jj / n_win_tiles, jj % n_win_tiles, s);
}

__global__ void k_fill_u32(uint32_t* p, size_t n, uint32_t v) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

hipError_t launch_index_pass(const IndexPass& p, hipStream_t stream, const AttnPass* window) {
  if (p.rows == 0 || p.max_items == 0) return hipSuccess;
  // chunks per row, at most: scan_chunk_items keeps a row of n items within
  // max(scan_chunks_min(k), ceil(n / kScanChunk)) chunks
  const int scan_per_row =
      std::max<int>(scan_chunks_min(p.k), (int)((p.max_items + kScanChunk - 1) / kScanChunk));
  if (scan_per_row > p.max_chunks) return hipErrorInvalidValue;
  const int gr = grid_rows(p.rows);
  int h = prof_begin(CSA2_K_INDEX_SAMPLE, stream);
  // (rows, then helpers from the next multiple of 8 on: see k_index_sample)
  const unsigned sgrid_rows = (unsigned)((p.rows + kXcds - 1) / kXcds * kXcds + p.rows);
  if (p.source == kItemsDirect)
    hipLaunchKernelGGL(k_index_sample<true>, dim3(sgrid_rows), dim3(kSampleThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(k_index_sample<false>, dim3(sgrid_rows), dim3(kSampleThreads), 0, stream, p);
  prof_end(h, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  h = prof_begin(CSA2_K_INDEX_SCAN, stream);
  // the queries of a sequence share the scan of a chunk, up to 4 per
  // workgroup (direct items only)
  const int nqg = (p.source != kItemsDirect || p.n_q == 1) ? 1 : p.n_q == 2 ? 2 : 4;
  const int n_groups = p.rows / p.n_q * ((p.n_q + nqg - 1) / nqg);
  const dim3 sgrid((unsigned)(grid_rows(n_groups) * scan_per_row));
  const bool paged = p.pm.pages != nullptr;  // (direct items only: the host refuses the others)
  if (p.source != kItemsDirect)
    hipLaunchKernelGGL((k_index_scan<2, false, 1, false>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else if (nqg == 1 && paged)
    hipLaunchKernelGGL((k_index_scan<2, true, 1, true>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else if (nqg == 1)
    hipLaunchKernelGGL((k_index_scan<2, true, 1, false>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else if (nqg == 2 && paged)
    hipLaunchKernelGGL((k_index_scan_mfma<2, true>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else if (nqg == 2)
    hipLaunchKernelGGL((k_index_scan_mfma<2, false>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else if (paged)
    hipLaunchKernelGGL((k_index_scan_mfma<4, true>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else
    hipLaunchKernelGGL((k_index_scan_mfma<4, false>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  prof_end(h, stream);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  h = prof_begin(CSA2_K_INDEX_SELECT, stream);
  if (p.k > 1024) {
    hipLaunchKernelGGL(k_index_select<32>, dim3((unsigned)p.rows), dim3(256), 0, stream, p);
  } else if (window) {
    const int n_win_tiles = window->n_tiles - (window->n_idx + kAttnSplit - 1) / kAttnSplit;
    const int n_wg = window->rows * window->n_layers * n_win_tiles;
    hipLaunchKernelGGL(k_index_select_window<16>, dim3((unsigned)(p.rows + n_wg)), dim3(256), 0, stream, p, *window);
  } else {
    hipLaunchKernelGGL(k_index_select<16>, dim3((unsigned)p.rows), dim3(256), 0, stream, p);
  }
  prof_end(h, stream);
  return hipGetLastError();
}

}  // namespace csa2
