// Indexer + top-k of the CSA2 step.
//
// The pages (agentnet.co.il "DeepSeek launches V4.1-Flash ...", section
// "CSA2: compression along the layer axis") fix only what is selected: 512
// fresh positions per Full or Reindex layer, and for the hierarchical indexer
// a pool of 2,048 blocks of 8 positions.  The score is a reading:
//   s_p = ks_p * sum_h w_h * max(0, q_h . k_p)   over 4 indexer heads.
//
// One pass = three kernels over the rows (query rows) of a call:
//   scan    streams the fp8 keys once (4 lanes per key, 16 B each, fully
//           coalesced), scores every item with packed f16 dot products
//           (v_dot2c_f32_f16; fp8 -> f16 is exact), writes an order-preserving
//           uint32 score key per item and a 4096-bin histogram of the key's
//           top 12 bits per row;
//   filter  finds the histogram bin T at which the count of items at or above
//           it reaches k, and compacts the items of bin >= T in item order;
//   select  radix-selects, among those few candidates, the exact k-th largest
//           (score, -item) key and writes the winners in ascending order.
// The candidates are exact: every item of the top k lies in a bin >= T.
#include "kernels.hpp"

namespace csa2 {

constexpr int kSelectLds = 6144;    // candidates kept in LDS by the select kernel

__device__ __forceinline__ int64_t row_vis_positions(const IndexPass& p, int row) {
  const int seq = row / p.n_q, i = row - seq * p.n_q;
  const int64_t pos = p.seq.a[seq] + i;
  int64_t vis = (pos + 1) / p.ratio;
  const int64_t ne = p.seq.b[seq];
  vis = vis < ne ? vis : ne;
  return vis < 0 ? 0 : vis;
}

// Items of a row, and the limit positions must stay below.
__device__ __forceinline__ int64_t row_items(const IndexPass& p, int row, int64_t vis_pos) {
  if (p.source == kItemsDirect) return p.block_level ? (vis_pos + 7) / 8 : vis_pos;
  if (p.source == kItemsBlocks) return 8 * (int64_t)p.nsel[row];
  return p.list_len;
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
// scores and histogram a row writes stay in that XCD's L2 for the next pass.
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

// ------------------------------------------------------------------ scan
template <int U>
__global__ __launch_bounds__(256) void k_index_scan(IndexPass p, int per_row) {
  int row, chunk;
  map_row_chunk(p.rows, per_row, row, chunk);
  if (row >= p.rows) return;
  const int64_t vis = row_vis_positions(p, row);
  const int64_t n_items = row_items(p, row, vis);
  const int64_t base = (int64_t)chunk * kScanChunk;
  if (base >= n_items) return;
  const int64_t end = base + kScanChunk < n_items ? base + kScanChunk : n_items;

  __shared__ uint32_t hist[kHistBins];
  for (int i = threadIdx.x; i < kHistBins; i += 256) hist[i] = 0;

  const int quarter = threadIdx.x & 3;
  half2_t q[kHI][8];
  const uint8_t* qp = p.idx_q + (int64_t)row * (kHI * kDI) + quarter * 16;
#pragma unroll
  for (int h = 0; h < kHI; ++h) {
    const uint4 raw = *reinterpret_cast<const uint4*>(qp + h * kDI);
    fp8x4_to_f16(raw.x, q[h][0], q[h][1]);
    fp8x4_to_f16(raw.y, q[h][2], q[h][3]);
    fp8x4_to_f16(raw.z, q[h][4], q[h][5]);
    fp8x4_to_f16(raw.w, q[h][6], q[h][7]);
  }
  float w[kHI];
#pragma unroll
  for (int h = 0; h < kHI; ++h) w[h] = p.idx_w ? p.idx_w[(int64_t)row * kHI + h] : 1.0f;
  __syncthreads();

  const int seq = row / p.n_q;
  const uint8_t* kb = p.k8 + (int64_t)seq * p.k_stride * kDI + quarter * 16;
  const float* sb = p.kscale + (int64_t)seq * p.k_stride;
  uint32_t* so = p.scores + (int64_t)row * p.score_stride;
  const int sub = threadIdx.x >> 2;  // item within a 64-item step

  // U items per lane quad per batch; two batches in flight (double buffer)
  struct Batch {
    u32x4_t raw[U];
    float ks[U];
    bool valid[U];
  };
  auto load = [&](Batch& B, int64_t it0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t item = it0 + u * 64 + sub;
      const int64_t pos = item_position(p, row, item, end, vis, B.valid[u]);
      if (B.valid[u]) {
        B.raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + pos * kDI));
        B.ks[u] = sb[pos];
      } else {
        B.raw[u] = u32x4_t{0, 0, 0, 0};
        B.ks[u] = 0.0f;
      }
    }
  };
  auto score = [&](const Batch& B, int64_t it0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float d[kHI] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        half2_t lo, hi;
        fp8x4_to_f16(B.raw[u][j], lo, hi);
#pragma unroll
        for (int h = 0; h < kHI; ++h) {
          d[h] = __builtin_amdgcn_fdot2(q[h][2 * j], lo, d[h], false);
          d[h] = __builtin_amdgcn_fdot2(q[h][2 * j + 1], hi, d[h], false);
        }
      }
#pragma unroll
      for (int h = 0; h < kHI; ++h) {
        d[h] += quad_xor1(d[h]);
        d[h] += quad_xor2(d[h]);
      }
      float acc = 0.0f;
#pragma unroll
      for (int h = 0; h < kHI; ++h) acc += w[h] * fmaxf(d[h], 0.0f);
      const float sc = B.ks[u] * acc;
      const int64_t item = it0 + u * 64 + sub;
      if (quarter == 0 && item < end) {
        const uint32_t key = B.valid[u] ? score_key(sc) : 0u;
        so[item] = key;
        if (B.valid[u]) atomicAdd(&hist[key >> 20], 1u);
      }
    }
  };
  constexpr int kStep = 64 * U;
  Batch A, Bb;
  int64_t it = base;
  load(A, it);
  while (true) {
    const int64_t nxt = it + kStep;
    if (nxt < end) load(Bb, nxt);
    score(A, it);
    if (nxt >= end) break;
    const int64_t nxt2 = nxt + kStep;
    if (nxt2 < end) load(A, nxt2);
    score(Bb, nxt);
    if (nxt2 >= end) break;
    it = nxt2;
  }
  __syncthreads();
  uint32_t* gh = p.hist + (int64_t)row * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += 256) {
    const uint32_t c = hist[i];
    if (c) atomicAdd(gh + i, c);
  }
}

// ------------------------------------------------------------------ threshold
// Inclusive prefix sum over the 256 threads of a workgroup: shuffles inside
// each wave, one LDS exchange of the four wave totals.
__device__ __forceinline__ uint32_t block_incl_scan_256(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0;
  for (int i = 0; i < wave; ++i) before += wsum[i];
  total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return before + x;
}

// From a row's 4096-bin histogram (256 threads, 16 bins each): the largest
// bin T whose count of items at or above it reaches k (0 if fewer than k
// items exist), and the number of items strictly above T.
__device__ __forceinline__ void row_threshold(const uint32_t* gh, uint32_t k, uint32_t* wsum,
                                              uint32_t* sh2, uint32_t& T, uint32_t& above) {
  const int t = threadIdx.x;
  const uint4* g4 = reinterpret_cast<const uint4*>(gh) + 4 * t;
  uint32_t hb[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = g4[i];
    hb[4 * i] = v.x; hb[4 * i + 1] = v.y; hb[4 * i + 2] = v.z; hb[4 * i + 3] = v.w;
  }
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) local += hb[j];
  // items in bins >= 16t = total - (inclusive prefix up to thread t-1)
  uint32_t total;
  const uint32_t incl = block_incl_scan_256(local, wsum, total);
  const uint32_t at_or_above = total - (incl - local);
  if (t == 0) { sh2[0] = 0; sh2[1] = total; }
  __syncthreads();
  uint32_t run = at_or_above - local;  // items in bins above this thread's 16
  if (run < k && at_or_above >= k) {
    for (int j = 15; j >= 0; --j) {
      const uint32_t nrun = run + hb[j];
      if (nrun >= k) { sh2[0] = 16 * t + j; sh2[1] = run; break; }
      run = nrun;
    }
  }
  __syncthreads();
  T = sh2[0];
  above = sh2[1];  // when T = 0 because fewer than k items exist: all of them
}

// ------------------------------------------------------------------ filter
__global__ __launch_bounds__(256) void k_index_filter(IndexPass p, int per_row) {
  int row, chunk;
  map_row_chunk(p.rows, per_row, row, chunk);
  if (row >= p.rows) return;
  const int64_t vis = row_vis_positions(p, row);
  const int64_t n_items = row_items(p, row, vis);
  const int64_t base = (int64_t)chunk * kFilterChunk;
  if (base >= n_items) return;

  __shared__ uint32_t wsum[4];
  __shared__ uint32_t sh2[2];
  const int t = threadIdx.x;
  uint32_t T, above;
  row_threshold(p.hist + (int64_t)row * kHistBins, (uint32_t)p.k, wsum, sh2, T, above);

  // each thread compacts 32 consecutive items, in item order
  const uint32_t* so = p.scores + (int64_t)row * p.score_stride;
  uint32_t keys[32];
  const int64_t i0 = base + 32 * t;
#pragma unroll
  for (int j = 0; j < 32; j += 4) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (i0 + j < n_items) v = *reinterpret_cast<const uint4*>(so + i0 + j);
    keys[j] = v.x; keys[j + 1] = v.y; keys[j + 2] = v.z; keys[j + 3] = v.w;
  }
  uint32_t flags = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const bool f = (i0 + j < n_items) && keys[j] != 0u && (keys[j] >> 20) >= T;
    flags |= (uint32_t)f << j;
  }
  const uint32_t c = __builtin_popcount(flags);
  uint32_t total;
  uint32_t off = block_incl_scan_256(c, wsum, total) - c;
  uint64_t* co = p.cand + (int64_t)row * p.score_stride + base;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    if (flags & (1u << j)) co[off++] = select_key(keys[j], (uint32_t)(i0 + j));
  }
  if (t == 0) p.fcount[(int64_t)row * p.max_fchunks + chunk] = total;
}

// ------------------------------------------------------------------ select
constexpr int kRankMax = 2048;  // threshold-bin candidates kept in LDS for the radix steps

__global__ __launch_bounds__(256) void k_index_select(IndexPass p) {
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t vis = row_vis_positions(p, row);
  const int64_t n_items = row_items(p, row, vis);
  const int nf = (int)((n_items + kFilterChunk - 1) / kFilterChunk);

  __shared__ uint32_t off[kMaxFChunks + 1];
  __shared__ uint64_t lc[kSelectLds];
  __shared__ uint64_t bt[kRankMax];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t sh2[2];
  __shared__ uint64_t sh_kth;
  __shared__ uint32_t sh_need;

  // chunk offsets: thread t owns chunks 4t .. 4t+3
  uint32_t cnt[4], local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int f = 4 * t + j;
    cnt[j] = f < nf ? p.fcount[(int64_t)row * p.max_fchunks + f] : 0u;
    local += cnt[j];
  }
  uint32_t total;
  uint32_t run = block_incl_scan_256(local, wsum, total) - local;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int f = 4 * t + j;
    if (f <= nf) off[f] = run;
    run += cnt[j];
  }
  __syncthreads();

  uint32_t T, above;
  row_threshold(p.hist + (int64_t)row * kHistBins, (uint32_t)p.k, wsum, sh2, T, above);

  const uint64_t* cbase = p.cand + (int64_t)row * p.score_stride;
  const bool in_lds = total <= (uint32_t)kSelectLds;
  auto fetch = [&](uint32_t g) -> uint64_t {
    int lo = 0, hi = nf - 1;  // last chunk f with off[f] <= g
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= g) lo = mid; else hi = mid - 1;
    }
    return cbase[(int64_t)lo * kFilterChunk + (g - off[lo])];
  };
  if (in_lds) {
    for (uint32_t g = t; g < total; g += 256) lc[g] = fetch(g);
  }
  __syncthreads();
  auto get = [&](uint32_t g) -> uint64_t { return in_lds ? lc[g] : fetch(g); };

  // kth = the k-th largest candidate key (keys are unique); 0 selects all.
  // Radix steps over the key bits below the threshold bin: 8-bit digits at
  // shifts 44, 36, .., 4, then the last 4 bits.  In the common case the
  // threshold-bin keys are first compacted into LDS; otherwise every
  // candidate is visited through `get` (still exact, slower).
  const uint32_t k = (uint32_t)p.k;
  uint64_t kth = 0;
  if (total > k) {
    const uint32_t m = total - above;      // candidates in the threshold bin
    const bool use_bt = in_lds && m <= (uint32_t)kRankMax;
    if (use_bt) {
      uint32_t base_out = 0;
      for (uint32_t g0 = 0; g0 < total; g0 += 256) {
        const uint32_t g = g0 + t;
        const uint64_t key = g < total ? lc[g] : 0ull;
        const bool f = g < total && (uint32_t)(key >> 52) == T;
        uint32_t n_round;
        const uint32_t o = block_incl_scan_256(f ? 1u : 0u, wsum, n_round) - (f ? 1u : 0u);
        if (f) bt[base_out + o] = key;
        base_out += n_round;
      }
    }
    const uint32_t n_keys = use_bt ? m : total;
    if (t == 0) { sh_kth = (uint64_t)T << 52; sh_need = k - above; }
    for (int shift = 44; shift >= 0; shift -= (shift == 4 ? 4 : 8)) {
      const int nb = shift == 0 ? 4 : 8;
      h256[t] = 0;
      __syncthreads();
      const uint64_t prefix = sh_kth;
      const uint64_t hmask = ~0ull << (shift + nb);
      const uint32_t dmask = (1u << nb) - 1u;
      for (uint32_t g = t; g < n_keys; g += 256) {
        const uint64_t key = use_bt ? bt[g] : get(g);
        if ((key & hmask) == prefix) atomicAdd(&h256[(key >> shift) & dmask], 1u);
      }
      __syncthreads();
      if (t < 64) {  // one wave: suffix sums over 256 digits, 4 per lane
        const uint32_t nd = sh_need;
        const uint32_t c0 = h256[4 * t], c1 = h256[4 * t + 1], c2 = h256[4 * t + 2], c3 = h256[4 * t + 3];
        const uint32_t mine = c0 + c1 + c2 + c3;
        uint32_t x = mine;  // inclusive suffix over lanes t..63
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const uint32_t y = __shfl_down(x, d, 64);
          if (t + d < 64) x += y;
        }
        uint32_t ab = x - mine;
        const uint32_t cs[4] = {c0, c1, c2, c3};
        for (int j = 3; j >= 0; --j) {
          if (ab < nd && ab + cs[j] >= nd) {
            sh_need = nd - ab;
            sh_kth = prefix | ((uint64_t)(4 * t + j) << shift);
          }
          ab += cs[j];
        }
      }
      __syncthreads();
      if (shift == 0) break;
    }
    kth = sh_kth;
  }

  // winners (key >= kth) in item order
  const int32_t* blocks = p.blocks;
  uint32_t written = 0;
  for (uint32_t g0 = 0; g0 < total; g0 += 256) {
    const uint32_t g = g0 + t;
    uint64_t key = 0;
    bool f = false;
    if (g < total) { key = get(g); f = key >= kth; }
    uint32_t n_round;
    const uint32_t o = written + block_incl_scan_256(f ? 1u : 0u, wsum, n_round) - (f ? 1u : 0u);
    if (f) {
      const uint32_t item = select_key_pos(key);
      int32_t val;
      if (p.source == kItemsDirect) val = (int32_t)item;
      else if (p.source == kItemsBlocks)
        val = 8 * blocks[(int64_t)row * CSA2_MAX_K + (item >> 3)] + (int32_t)(item & 7u);
      else val = p.list[(int64_t)row * p.list_len + item];
      p.out[(int64_t)row * p.out_stride + o] = val;
    }
    written += n_round;
  }
  // pad, counts, pool, and reset the histogram for the next pass
  if (!p.block_level) {
    for (uint32_t j = written + t; j < k; j += 256) p.out[(int64_t)row * p.out_stride + j] = -1;
  }
  if (p.out_count && t == 0) p.out_count[row] = (int32_t)written;
  if (p.out_pool) {
    __syncthreads();  // block ids written above are read back here
    const int32_t total_pool = CSA2_N_BLOCKS * CSA2_BLOCK;
    for (int32_t j = t; j < p.pool_stride && j < total_pool; j += 256) {
      int32_t v = -1;
      if ((uint32_t)(j >> 3) < written) {
        const int64_t pos = 8 * (int64_t)p.out[(int64_t)row * p.out_stride + (j >> 3)] + (j & 7);
        if (pos < vis) v = (int32_t)pos;
      }
      p.out_pool[(int64_t)row * p.pool_stride + j] = v;
    }
  }
  uint4* gh = reinterpret_cast<uint4*>(p.hist + (int64_t)row * kHistBins);
  for (int i = t; i < kHistBins / 4; i += 256) gh[i] = make_uint4(0, 0, 0, 0);
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

hipError_t launch_index_pass(const IndexPass& p, hipStream_t stream) {
  if (p.rows == 0 || p.max_items == 0) return hipSuccess;
  const int scan_per_row = (int)((p.max_items + kScanChunk - 1) / kScanChunk);
  const int filt_per_row = (int)((p.max_items + kFilterChunk - 1) / kFilterChunk);
  const int gr = grid_rows(p.rows);
  int h = prof_begin(CSA2_K_INDEX_SCAN, stream);
  hipLaunchKernelGGL(k_index_scan<4>, dim3((unsigned)(gr * scan_per_row)), dim3(256), 0, stream, p,
                     scan_per_row);
  prof_end(h, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  h = prof_begin(CSA2_K_INDEX_FILTER, stream);
  hipLaunchKernelGGL(k_index_filter, dim3((unsigned)(gr * filt_per_row)), dim3(256), 0, stream, p,
                     filt_per_row);
  prof_end(h, stream);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  h = prof_begin(CSA2_K_INDEX_SELECT, stream);
  hipLaunchKernelGGL(k_index_select, dim3((unsigned)p.rows), dim3(256), 0, stream, p);
  prof_end(h, stream);
  return hipGetLastError();
}

}  // namespace csa2
