// Indexer + top-k of the CSA2 step.
//
// The pages (agentnet.co.il "DeepSeek launches V4.1-Flash ...", section
// "CSA2: compression along the layer axis") fix only what is selected: 512
// fresh positions per Full or Reindex layer, and for the hierarchical indexer
// a pool of 2,048 blocks of 8 positions.  The score is a reading:
//   s_p = ks_p * sum_h w_h * max(0, q_h . k_p)   over 4 indexer heads.
//
// One pass = two kernels over the rows (query rows) of a call:
//   scan    streams the fp8 keys once.  One query per workgroup: 4 lanes per
//           key, 16 B each, fully coalesced, packed f16 dot products
//           (v_dot2c_f32_f16; fp8 -> f16 is exact).  2 or 4 queries of a
//           sequence: one fp8 MFMA per 32-key tile for all of them.  The
//           workgroup keeps its chunk's scores in LDS and, after the stream,
//           histograms them below the chunk's largest score (1/64 of a
//           binade per bin) to cut two bands: band 0, about the number of
//           the row's winners the chunk can hold at most with any
//           likelihood (a Poisson bound on the expected share), and band 1,
//           the next keys up to the 128-slot segment.  Both go to the
//           (row, chunk) segment with the band edges and the chunk's largest
//           key scale;
//   select  gathers band 0 of every chunk (about 3 k keys), finds the k-th
//           largest (score, -item) key, fetches band 1 only of chunks whose
//           band-0 edge reaches down to it, and settles the set: keys more
//           than twice the score's error bound above the k-th win, keys
//           within it are rescored exactly (float64, the products of E4M3
//           codes summed exactly) and ranked by (score, -position); the
//           winners are ordered by position (segments list their bands in
//           item order, so compacting them in gather order orders them) and
//           written.  A row whose bands cannot hold the answer (a chunk
//           holding more than its segment of the winners, e.g. all scores
//           equal) is recomputed by itself over every item: slow, exact,
//           rare, and counted.  In a decode group the select runs inside the
//           group's attention launch (k_index_select_attend): every tile
//           workgroup selects its row and attends over its share of the
//           winners.
// No separate pass picks a threshold for the scan: each chunk cuts its own
// bands from its own scores, so the scan needs nothing from another kernel.
#include "kernels.hpp"
#include "select.hpp"
#include "tile.hpp"

namespace csa2 {

constexpr int kBitmapItems = 131072;  // rows with at most this many items order winners by bitmap
constexpr int kSpecChunks = 64;       // rows with at most this many scan chunks (twice this at kPer 32) gather in one round trip
constexpr int kSpecSlots = 64;        // ... of the first this many slots of each segment (band 0 fits)
constexpr int kBand0Max = kSpecSlots; // band 0 of a chunk holds at most this many keys
constexpr int kBandMax = 1024;        // near-tie keys one select rescores exactly, at most
// Error bound of a binary32 score against the exact one, as a multiple of
// ks * sum_h |w_h| * sum_c |q_hc| * 448 (448 bounds every E4M3 key code):
// the VALU dot takes at most 18 binary32 roundings per head, each within
// 2^-24 of a partial sum no larger than that; the MFMA accumulation is taken
// as 2^-12 (a measured worst case on random codes was 2.5e-5 of the summed
// magnitudes, 10x below).  A further 2^-20 |s| covers the roundings after
// the dots.
constexpr float kErrValu = 0x1p-18f;
constexpr float kErrMfma = 0x1p-12f;
constexpr float kErrTail = 0x1p-20f;

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

// The same with per-head keys: raw[s] holds this lane's 16 channels of the
// key of head quad_head(s, quarter), the head its query slot s holds.
__device__ __forceinline__ float quad_score_heads(const half2_t (&q)[kHI][8], float w_mine, const u32x4_t (&raw)[kHI],
                                                  float ks) {
  float d[kHI] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kHI; ++s) {
    half2_t kh[8];
    key_f16(raw[s], kh);
#pragma unroll
    for (int j = 0; j < 8; ++j) d[s] = __builtin_amdgcn_fdot2(q[s][j], kh[j], d[s], false);
  }
  const float e0 = d[0] + quad_xor1(d[2]);
  const float e1 = d[1] + quad_xor1(d[3]);
  const float f = e0 + quad_xor2(e1);
  float v = w_mine * fmaxf(f, 0.0f);
  v += quad_xor1(v);
  v += quad_xor2(v);
  return ks * v;
}

__device__ __forceinline__ float quad_score_at(const IndexPass& p, const half2_t (&q)[kHI][8], float w_mine,
                                               int seq, int quarter, int64_t pos, bool valid) {
  if (p.key_heads == 4) {  // per-head keys (contiguous caches only)
    u32x4_t raw[kHI];
    float ks = 0.0f;
    const uint8_t* kp = p.k8 + ((int64_t)seq * p.k_stride + pos) * (4 * kDI) + quarter * 16;
#pragma unroll
    for (int s2 = 0; s2 < kHI; ++s2)
      raw[s2] = valid ? *reinterpret_cast<const u32x4_t*>(kp + quad_head(s2, quarter) * kDI) : u32x4_t{0, 0, 0, 0};
    if (valid) ks = p.kscale[(int64_t)seq * p.k_stride + pos];
    return quad_score_heads(q, w_mine, raw, ks);
  }
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


// Score of item `pos` (as item_position gives it) in the exact recompute:
// the quad score of that position, or for a block-max pass the largest
// score among block `pos`'s visible positions (through the score keys, as
// the scan took it).
__device__ __forceinline__ float item_score_at(const IndexPass& p, const half2_t (&q)[kHI][8], float w_mine, int seq,
                                               int quarter, int64_t pos, bool valid, int64_t vis) {
  if (p.block_level != 2) return quad_score_at(p, q, w_mine, seq, quarter, pos, valid);
  uint32_t best = 0u;
#pragma unroll 1
  for (int j = 0; j < 8; ++j) {
    const int64_t tp = 8 * pos + j;
    const bool v = valid && tp < vis;
    const float sc = quad_score_at(p, q, w_mine, seq, quarter, v ? tp : 0, v);
    if (v) best = max(best, score_key(sc));
  }
  return key_to_score(best);
}

// Exact k-th largest of n keys visited by `visit(n, f)` (f(key) per key), by
// radix steps of 8 bits from bit `top` down.  256 threads; keys are unique
// or the result is the k-th in the multiset order.
template <typename Key, typename Visit>
__device__ __forceinline__ Key radix_kth(Visit visit, uint32_t n, uint32_t want, uint32_t* h256, Key* sh_kth, uint32_t* sh_need) {
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


// ------------------------------------------------------------------ scan
// Band 0 of a chunk: the largest number of the row's winners it may hold
// with any likelihood, from the expected share mu = k * csize / n (at most 8,
// or 16 for k above 1,024, by the chunk sizing): mu + 4 sqrt(mu) + 3 (the
// Poisson tail beyond that is below 1e-5 for mu <= 16), at most the
// select's room shared by the row's chunks.
__device__ __forceinline__ uint32_t band0_size(int64_t n_items, int64_t csize, int64_t nch, int k) {
  const float mu = (float)((int64_t)k * csize) / (float)(n_items > 0 ? n_items : 1);
  uint32_t m0 = (uint32_t)(mu + 4.0f * sqrtf(mu) + 3.0f);
  const int64_t room = (k > 1024 || nch > 128 ? 256 * 32 : 256 * 16) * 3 / 4;
  const int64_t share = room / (nch > 0 ? nch : 1);
  if ((int64_t)m0 > share) m0 = (uint32_t)share;
  if (m0 > (uint32_t)kBand0Max) m0 = kBand0Max;
  return m0 > 0 ? m0 : 1u;
}

// The record of a chunk's candidate bands, as the select reads it back.
//   x: n0 | ntot << 8 | (b0 + 1) << 16 | (b1 + 1) << 24
//   y: the chunk's largest score key mx
//   z: 1 when the chunk dropped no key
//   w: the largest key scale of the chunk (float bits)
// Band 0 holds the keys within the first b0 + 1 bins below mx, band 1 those
// of the bins after it up to b1; a bin is 2^17 key units (1/64 of a binade).
__device__ __forceinline__ uint32_t band_edge(uint32_t mx, int b) {  // keys >= edge lie in bins 0..b
  const uint64_t span = (uint64_t)(b + 1) << 17;
  return b < 0 ? mx + 1u : span > mx ? 1u : mx - (uint32_t)span + 1u;
}
__device__ __forceinline__ uint32_t rec_n0(const u32x4_t& r) { return r[0] & 0xFFu; }
__device__ __forceinline__ uint32_t rec_ntot(const u32x4_t& r) { return (r[0] >> 8) & 0xFFu; }
__device__ __forceinline__ uint32_t rec_thi(const u32x4_t& r) { return band_edge(r[1], (int)((r[0] >> 16) & 0xFFu) - 1); }
// keys the chunk dropped all lie below this (0: it dropped none)
__device__ __forceinline__ uint32_t rec_tlo(const u32x4_t& r) {
  return r[2] ? 0u : band_edge(r[1], (int)(r[0] >> 24) - 1);
}

// Candidate bands of one chunk (see the file comment), from the chunk's
// score keys keys[0 .. n_slots) in LDS (0: no item at that slot; slot i is
// item base + i; the array holds kScanChunk keys).  Band 0 is every key
// within the first b0 + 1 bins below the chunk's largest key, b0 the last
// bin whose running count stays within m0; band 1 the keys of the
// following bins whose running count stays within the segment.  A chunk of
// at most kSeg keys keeps them all (nothing dropped).  mx_lane / ks_lane:
// each lane's largest score key and key scale bits seen (0 if none).  All
// 256 threads call it; the keys must be in LDS (its first barrier publishes
// them), and it may be called again right after it returns.
__device__ __forceinline__ void emit_chunk(const IndexPass& p, int64_t row, int chunk, const uint32_t* keys,
                                           int n_slots, int64_t base, uint32_t m0, uint32_t mx_lane,
                                           uint32_t ks_lane, uint32_t* hist, uint32_t* sh) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const uint32_t mxw = wave_max_u32(mx_lane), ksw = wave_max_u32(ks_lane);
  hist[t] = 0u;
  if (lane == 0) {
    sh[wave] = mxw;
    sh[4 + wave] = ksw;
  }
  __syncthreads();
  const uint32_t mx = max(max(sh[0], sh[1]), max(sh[2], sh[3]));
  const uint32_t ksm = max(max(sh[4], sh[5]), max(sh[6], sh[7]));
  uint32_t k[8];
  {
    const uint4 a = reinterpret_cast<const uint4*>(keys)[2 * t], b = reinterpret_cast<const uint4*>(keys)[2 * t + 1];
    const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) k[j] = 8 * t + j < n_slots ? v[j] : 0u;
  }
  if (p.block_max && p.block_level == 0 && 8 * t < n_slots) {
    // the largest key of block base / 8 + t (its 8 items are k[0 .. 8)),
    // for a block-max pass after this one
    const uint32_t bm = max(max(max(k[0], k[1]), max(k[2], k[3])), max(max(k[4], k[5]), max(k[6], k[7])));
    p.block_max[row * p.block_max_stride + (base >> 3) + t] = bm;
  }
  // bins of the distance below mx; bin 255 takes everything further down
  // (counted by one lane per wave: it can hold most keys)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t d = (mx - k[j]) >> 17;
    const bool near = k[j] != 0u && d < 255u;
    const bool far = k[j] != 0u && d >= 255u;
    if (near) atomicAdd(&hist[d], 1u);
    const unsigned long long fb = __ballot(far);
    if (fb && lane == (__ffsll((long long)fb) - 1)) atomicAdd(&hist[255], (uint32_t)__popcll(fb));
  }
  __syncthreads();
  if (wave == 0) {
    // lane l owns bins 4l .. 4l+3; e_j = keys in bins 0 .. 4l+j
    const uint4 h4 = reinterpret_cast<const uint4*>(hist)[lane];
    const uint32_t mine = h4.x + h4.y + h4.z + h4.w;
    const uint32_t incl = wave_incl_add(mine);
    const uint32_t n_valid = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    const uint32_t e0 = incl - mine + h4.x, e1 = e0 + h4.y, e2 = e1 + h4.z, e3 = incl;
    // cum is non-decreasing: the bins with cum <= m form a prefix, b = its length - 1
    // (bin 255 never counts: it is not a band bin)
    const uint32_t last = lane == 63 ? 0u : 1u;
    const uint32_t c0 = (e0 <= m0) + (e1 <= m0) + (e2 <= m0) + last * (e3 <= m0);
    const uint32_t c1 = (e0 <= (uint32_t)kSeg) + (e1 <= (uint32_t)kSeg) + (e2 <= (uint32_t)kSeg) + last * (e3 <= (uint32_t)kSeg);
    const int b0 = (int)__builtin_amdgcn_readlane((int)wave_incl_add(c0), 63) - 1;
    const int b1 = (int)__builtin_amdgcn_readlane((int)wave_incl_add(c1), 63) - 1;
    auto cum_at = [&](int b) -> uint32_t {
      if (b < 0) return 0u;
      const int j = b & 3;
      const uint32_t e = j == 0 ? e0 : j == 1 ? e1 : j == 2 ? e2 : e3;
      return (uint32_t)__builtin_amdgcn_readlane((int)e, b >> 2);
    };
    const uint32_t n0 = cum_at(b0), n1 = cum_at(b1);
    if (lane == 0) {
      const bool complete = n_valid <= (uint32_t)kSeg;
      sh[8] = band_edge(mx, b0);               // band 0: keys >= this
      sh[9] = complete ? 1u : band_edge(mx, b1);  // band 1: keys >= this (below band 0)
      sh[10] = n0;
      sh[11] = complete ? n_valid : n1;
      sh[14] = n0 | ((complete ? n_valid : n1) << 8) | ((uint32_t)(b0 + 1) << 16) | ((uint32_t)(b1 + 1) << 24);
      sh[15] = complete ? 1u : 0u;
    }
  }
  __syncthreads();
  const uint32_t thi = sh[8], tlo = sh[9], n0 = sh[10];
  // segment slots in item order, without LDS atomics: a lane's band-0
  // (band-1) keys follow those of the lanes and waves before it (one wave
  // prefix sum of both counts, packed), so each band lists its items
  // ascending, which lets the select order its winners by compaction
  uint32_t f0 = 0u, f1 = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    f0 |= (k[j] != 0u && k[j] >= thi ? 1u : 0u) << j;
    f1 |= (k[j] != 0u && k[j] >= tlo && k[j] < thi ? 1u : 0u) << j;
  }
  const uint32_t cnt = (uint32_t)__builtin_popcount(f0) | ((uint32_t)__builtin_popcount(f1) << 16);
  const uint32_t incl = wave_incl_add(cnt);
  if (lane == 63) sh[16 + wave] = incl;
  __syncthreads();
  uint32_t before = incl - cnt;
  for (int w = 0; w < wave; ++w) before += sh[16 + w];
  uint32_t o0 = before & 0xFFFFu, o1 = n0 + (before >> 16);
  const __amdgpu_buffer_rsrc_t rseg = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.seg_list + (row * p.max_chunks + chunk) * kSeg), 0, kSeg * 8, kRawBufferWord3);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool in0 = (f0 >> j) & 1u, in1 = (f1 >> j) & 1u;
    if (in0 || in1) {
      const uint32_t slot = in0 ? o0++ : o1++;
      const uint64_t v = select_key(k[j], (uint32_t)(base + 8 * t + j));
      __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{(uint32_t)v, (uint32_t)(v >> 32)}, rseg, (int)(slot * 8), 0, 0);
    }
  }
  if (t == 0) {
    const __amdgpu_buffer_rsrc_t rinfo = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.chunk_info + row * p.max_chunks + chunk), 0, 16, kRawBufferWord3);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{sh[14], mx, sh[15], ksm}, rinfo, 0, 0, 0);
  }
}

// Workgroup (one query row, chunk of row_chunk_items items): every key of
// the chunk is scored and its score key staged in LDS, then emit_chunk cuts
// the bands.  kDirect: item i is position i (flat keys or block keys); keys
// and scales are read through buffer descriptors whose range ends at the
// chunk's last item, so the hardware returns zeros past it and the loads
// need no bounds branches.  Otherwise positions come from a block or
// position list.
// The LDS of one query's scan workgroup.
struct ScanLds {
  uint32_t skeys[kScanChunk];
  uint32_t hist[256];
  uint32_t sh[24];
};

// Chunk `chunk` of row `row` (base < end): score every item, stage the keys,
// cut and write the bands.
template <int U, bool kDirect, bool kPaged, bool kHeads = false>
__device__ __forceinline__ void scan_chunk(const IndexPass& p, int row, int chunk, int64_t csize, int64_t base,
                                           int64_t end, int64_t vis, int64_t n_items, ScanLds& L) {
  static_assert(!kPaged || kDirect, "paged caches are read over direct items");
  static_assert(!kPaged || !kHeads, "per-head keys are read from contiguous caches");
  // per-head keys: 256 bytes an entry, lane quarter c reads channels
  // 16c .. 16c+15 of each head's key (the head of each query slot)
  constexpr int kKB = kHeads ? 4 * kDI : kDI;  // key bytes per entry
  constexpr int kKH = kHeads ? kHI : 1;        // key loads per item and lane
  const int seq = row / p.n_q;
  uint32_t* skeys = L.skeys;
  uint32_t* hist = L.hist;
  uint32_t* sh = L.sh;
  const int quarter = threadIdx.x & 3;
  const int sub = threadIdx.x >> 2;  // item within a 64-item step
  half2_t q[kHI][8];
  float w_mine;  // loaded after the first keys: their loads overlap
  const uint8_t* kb = p.k8 + (int64_t)seq * p.k_stride * kKB;
  const float* sb = p.kscale + (int64_t)seq * p.k_stride;
  // (used by the kDirect loads only.)  Paged: descriptors over the pool, and
  // lane j holds the page-table value of the chunk's page j: a batch of
  // kStep items lies in one page (pages hold at least 128 entries, batches
  // start at multiples of kStep), so its entries are one page's consecutive
  // entries
  constexpr bool paged = kPaged;
  const uint32_t lim = paged ? (uint32_t)p.pm.pool : (uint32_t)end;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(paged ? p.k8 : kb), 0, (int)(lim * kKB), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(paged ? p.kscale : sb), 0, (int)(lim * 4), kRawBufferWord3);
  int head_off[kKH];  // byte offset of the key slice each load takes
#pragma unroll
  for (int s2 = 0; s2 < kKH; ++s2) head_off[s2] = (kHeads ? quad_head(s2, quarter) * kDI : 0) + quarter * 16;
  uint32_t page_lane = 0;
  if constexpr (paged) {
    const int64_t pg = (base >> p.pm.lg) + (threadIdx.x & 63);
    page_lane = __builtin_amdgcn_raw_buffer_load_b32(page_row(p.pm, seq), (int)(pg * 4), 0, 0);
  }

  // U items per lane quad per batch; two batches in flight (double buffer)
  struct Batch {
    u32x4_t raw[U][kKH];
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
#pragma unroll
        for (int s2 = 0; s2 < kKH; ++s2)
          B.raw[u][s2] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(e * kKB) + head_off[s2], 0, kLoadNonTemporal);
        B.ks[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(e * 4), 0, 0));
      } else {
        bool valid;
        const int64_t pos = item_position(p, row, item, end, vis, valid);
#pragma unroll
        for (int s2 = 0; s2 < kKH; ++s2)
          B.raw[u][s2] = valid ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + pos * kKB + head_off[s2]))
                               : u32x4_t{0, 0, 0, 0};
        B.ks[u] = valid ? sb[pos] : 0.0f;
      }
    }
  };
  uint32_t mx_lane = 0u, ks_lane = 0u;  // running maxima (key scales are >= 0: their bits order them)
  auto score = [&](const Batch& B, int64_t it0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float sc;
      if constexpr (kHeads) sc = quad_score_heads(q, w_mine, B.raw[u], B.ks[u]);
      else sc = quad_score(q, w_mine, B.raw[u][0], B.ks[u]);
      const int64_t item = it0 + u * 64 + sub;
      bool valid = item < end;
      if constexpr (!kDirect) {
        if (valid) {  // invalid list entries never become candidates
          bool ok;
          (void)item_position(p, row, item, end, vis, ok);
          valid = ok;
        }
      }
      const uint32_t key = valid ? score_key(sc) : 0u;
      mx_lane = max(mx_lane, key);
      ks_lane = max(ks_lane, valid ? __float_as_uint(B.ks[u]) : 0u);
      if (quarter == 0 && item < end) skeys[item - base] = key;
    }
  };
  constexpr int kStep = 64 * U;
  Batch A, Bb;
  int64_t it = base;
  load(A, it);
  load_query_f16(p, row, quarter, q, w_mine);
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
  const int64_t nch = scan_chunk_count(n_items, csize);
  emit_chunk(p, row, chunk, skeys, (int)(end - base), base, band0_size(n_items, csize, nch, p.k), mx_lane, ks_lane,
             hist, sh);
}

template <int U, bool kDirect, bool kPaged, bool kHeads = false>
__global__ __launch_bounds__(256) void k_index_scan(IndexPass p, int per_row, int n_groups) {
  int row, chunk;
  map_row_chunk(n_groups, per_row, row, chunk);
  if (row >= n_groups) return;
  const int64_t csize = row_chunk_items_of<kDirect>(p, row);  // shared by the rows of a sequence
  const int64_t base = (int64_t)chunk * csize;
  const int64_t vis = row_vis_positions(p, row);
  const int64_t n_items = row_items_of<kDirect>(p, row, vis);
  const int64_t end = base + csize < n_items ? base + csize : n_items;
  if (base >= end) return;
  __shared__ ScanLds L;
  scan_chunk<U, kDirect, kPaged, kHeads>(p, row, chunk, csize, base, end, vis, n_items, L);
}

// Block-max pass (block_level 2): workgroup (row, chunk of blocks) stages
// the blocks' keys, written by the flat scan of the same rows, and cuts the
// bands as the scan does; the key-scale bound is the row's largest.
__global__ __launch_bounds__(256) void k_index_scan_keys(IndexPass p, int per_row) {
  int row, chunk;
  map_row_chunk(p.rows, per_row, row, chunk);
  if (row >= p.rows) return;
  const int64_t csize = row_chunk_items_of<true>(p, row);
  const int64_t base = (int64_t)chunk * csize;
  const int64_t vis = row_vis_positions(p, row);
  const int64_t n_items = row_items_of<true>(p, row, vis);
  const int64_t end = base + csize < n_items ? base + csize : n_items;
  if (base >= end) return;
  __shared__ ScanLds L;
  const uint32_t* src = p.block_max + (int64_t)row * p.block_max_stride;
  uint32_t mx_lane = 0u;
  for (int64_t i = base + threadIdx.x; i < end; i += 256) {
    const uint32_t key = src[i];
    L.skeys[i - base] = key;
    mx_lane = max(mx_lane, key);
  }
  const uint32_t ks_lane = p.row_ksm[row];
  const int64_t nch = scan_chunk_count(n_items, csize);
  emit_chunk(p, row, chunk, L.skeys, (int)(end - base), base, band0_size(n_items, csize, nch, p.k), mx_lane, ks_lane,
             L.hist, L.sh);
}

// A pointer every lane holds the same value of, moved to scalar registers.
__device__ __forceinline__ void* uniform_ptr(const void* q) {
  const uint64_t v = reinterpret_cast<uint64_t>(q);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}
// The scan on fp8 MFMA (direct items) for NQ queries of one sequence: each
// 32-key tile of the chunk is scored against the 4 NQ heads of the NQ
// queries in one v_mfma_scale_f32_32x32x64_f8f6f4 (heads as A rows, keys as
// B columns, exact fp8 codes, unit scales, binary32 accumulation in the
// unit's own order: the select settles keys near the k-th by exact
// rescoring) instead of 16 fdot2 per key quarter and query on VALU.  Lane
// (l32, half) holds bytes 32 half .. +32 of key l32 of the tile (B) and of
// head row l32 (A): row 4 i + h is head h of query i.  The output gives the
// four head dots of query i for key l32 in the lanes of half i % 2,
// registers 4 (i / 2) .. +3, so a lane scores queries half, half + 2, ...
// Wave w takes tiles w, w + 4, ... of the chunk with kScanTiles tiles in
// flight.  Every query's score keys are staged in LDS, then each query's
// bands are cut by emit_chunk.
constexpr int kScanTiles = 4;
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
constexpr uint32_t kMfmaUnitScales = 0x7F7F7F7Fu;  // E8M0 127 = 1.0 in every byte
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
  int64_t lim_q[NQ], nit_q[NQ], end = 0;  // items of query i in this chunk end at lim_q[i]
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    nit_q[i] = i < nq ? row_items_of<true>(p, row0 + i, row_vis_positions(p, row0 + i)) : 0;
    lim_q[i] = base + csize < nit_q[i] ? base + csize : nit_q[i];
    end = lim_q[i] > end ? lim_q[i] : end;
  }
  if (base >= end) return;

  __shared__ uint32_t skeys[NQ][kScanChunk];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[24];
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
  // read zeros past the descriptor).  These loads and the weights go out
  // before the tiles: every load is unconditional, so the waits for them
  // inside the tile loop do not wait for tile data.
  v8i_t A;
  {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.idx_q + (int64_t)row0 * kHI * kDI), 0, nq * kHI * kDI, kRawBufferWord3);
    const int off = l32 < 4 * NQ ? (l32 >> 2) * kHI * kDI + (l32 & 3) * kDI + 32 * half : NQ * kHI * kDI;
    const u32x4_t lo = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
    const u32x4_t hi = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0);
    A = v8i_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  // this lane's queries i = 2 g + half: head weights and item limit
  float wq[NG][kHI];
  int64_t limq[NG];
  {
    const bool has_w = p.idx_w != nullptr;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(has_w ? p.idx_w + (int64_t)row0 * kHI : nullptr), 0, has_w ? nq * kHI * 4 : 0, kRawBufferWord3);
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
  for (int g = 0; g < NG; ++g) {
    const int ilo = 2 * g, ihi = 2 * g + 1 < NQ ? 2 * g + 1 : 2 * g;
    // (arithmetic, not a select: a select of the two becomes an indexed
    // load of lim_q through scratch)
    const int64_t la = lim_q[ilo], lb = 2 * g + 1 < NQ ? lim_q[ihi] : 0;
    limq[g] = la + (int64_t)half * (lb - la);
  }
  uint32_t mxq[NG], ks_lane = 0u;  // running maxima: this lane's queries' score keys, key scales
#pragma unroll
  for (int g = 0; g < NG; ++g) mxq[g] = 0u;
  auto score_tile = [&](const Tile& Tt, int m) {
    const v8i_t Bop = v8i_t{(int)Tt.lo[0], (int)Tt.lo[1], (int)Tt.lo[2], (int)Tt.lo[3],
                            (int)Tt.hi[0], (int)Tt.hi[1], (int)Tt.hi[2], (int)Tt.hi[3]};
    v16f_t acc = {};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, Bop, acc, 0, 0, 0, kMfmaUnitScales, 0,
                                                          kMfmaUnitScales);
    // the MFMA reads every lane's operands, so it must run with the whole
    // wave active: the empty asm pins it here, in uniform control flow
    asm volatile("" ::"v"(acc));
    const int64_t item = base + 32 * (int64_t)(wave + 4 * m) + l32;
    if (item < end) ks_lane = max(ks_lane, __float_as_uint(Tt.ks));
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const float sc = Tt.ks * (wq[g][0] * fmaxf(acc[4 * g], 0.0f) + wq[g][1] * fmaxf(acc[4 * g + 1], 0.0f) +
                                wq[g][2] * fmaxf(acc[4 * g + 2], 0.0f) + wq[g][3] * fmaxf(acc[4 * g + 3], 0.0f));
      const int i = 2 * g + half;
      const uint32_t key = item < limq[g] ? score_key(sc) : 0u;
      mxq[g] = max(mxq[g], key);
      if (i < NQ && item < end) skeys[i][item - base] = key;
    }
  };
  // whole groups of kScanTiles tiles, with no branch between the loads (a
  // tile past the chunk reads zeros and its items stay past the chunk's
  // end), so each score waits only for its own tile
  for (int m0 = 0; m0 < my_tiles; m0 += kScanTiles) {
#pragma unroll
    for (int s = 0; s < kScanTiles; ++s) {
      score_tile(T[s], m0 + s);
      load_tile(T[s], m0 + s + kScanTiles);
    }
  }
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    if (i < nq && base < lim_q[i]) {  // (uniform)
      const int64_t nch = scan_chunk_count(nit_q[i], csize);
      // query i's maximum lives in the lanes of half i % 2, slot i / 2
      const uint32_t mx_lane = half == (i & 1) ? mxq[i >> 1] : 0u;
      emit_chunk(p, row0 + i, chunk, skeys[i], (int)(lim_q[i] - base), base,
                 band0_size(nit_q[i], csize, nch, p.k), mx_lane, ks_lane, hist, sh);
    }
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

// The query of a row for exact rescoring and the error bound: its 256 code
// values as float64 in LDS (qd[c][h], channel c of head h) and the head
// weights (qw); returns sum_h |w_h| sum_c |q_hc| in every lane.  Every wave
// loads the 256 bytes itself (wave 0 stores them).
__device__ __forceinline__ float load_query_codes(const IndexPass& p, int row, float* qw, double (*qd)[4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.idx_q + (int64_t)row * kHI * kDI), 0, kHI * kDI, kRawBufferWord3);
  const uint32_t c = __builtin_amdgcn_raw_buffer_load_b32(rq, 4 * lane, 0, 0);
  float w = 1.0f;
  if (p.idx_w) {
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.idx_w + (int64_t)row * kHI), 0, 4 * kHI, kRawBufferWord3);
    w = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, 4 * (lane >> 4), 0, 0));
  }
  if (wave == 0) {
    if ((lane & 15) == 0) qw[lane >> 4] = w;
#pragma unroll
    for (int b = 0; b < 4; ++b) qd[4 * (lane & 15) + b][lane >> 4] = (double)e4m3_value((c >> (8 * b)) & 0xFFu);
  }
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) a += e4m3_mag((c >> (8 * j)) & 0x7Fu);  // exact (integers of 2^-9)
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) a += __shfl_xor(a, d, 64);  // the head's L1 norm, exact
  float cw = fabsf(w) * a;
  cw += __shfl_xor(cw, 16, 64);
  cw += __shfl_xor(cw, 32, 64);
  return cw;
}

// Loads of one key's 64 code bytes and scale (position pos of row's
// sequence) into registers: the shared key, or head `head`'s key.
__device__ __forceinline__ void load_key_row(const IndexPass& p, int row, int64_t pos, u32x4_t (&raw)[4], float& ks,
                                             int head) {
  const int seq = row / p.n_q;
  if (p.key_heads == 4) {  // head `head`'s 64 bytes of a per-head key (contiguous caches only)
    const u32x4_t* kp =
        reinterpret_cast<const u32x4_t*>(p.k8 + ((int64_t)seq * p.k_stride + pos) * (4 * kDI) + head * kDI);
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[j] = kp[j];
    ks = p.kscale[(int64_t)seq * p.k_stride + pos];
    return;
  }
  if (p.pm.pages) {
    const uint32_t e = paged_entry_at(p.pm, seq, pos);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.k8, 0, (int)(p.pm.pool * kDI), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.kscale, 0, (int)(p.pm.pool * 4), kRawBufferWord3);
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(e * kDI) + 16 * j, 0, 0);
    ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(e * 4), 0, 0));
  } else {
    const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(p.k8 + ((int64_t)seq * p.k_stride + pos) * kDI);
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[j] = kp[j];
    ks = p.kscale[(int64_t)seq * p.k_stride + pos];
  }
}

// Exact score of item `item` of `row`, float64, in the oracle's order of
// operations: d_h = sum_c q_hc k_c exactly (every E4M3 value is n 2^-9 with
// |n| < 2^18, so each product and every partial sum of 64 is an integer
// multiple of 2^-18 below 2^42: exact in float64, in any order);
// p_h = max(0, d_h) * w_h; s = ks * (((p_0 + p_1) + p_2) + p_3) (with
// per-head keys d_h dots head h's own key).  The four
// lanes of a quad take the four heads (lane quarter h); every lane of the
// quad returns s.  Lanes with valid == false return 0 and load nothing
// (whole quads agree on valid).
// The arithmetic of exact_score_at on a key already in registers.
__device__ __forceinline__ double exact_from_raw(const u32x4_t (&raw)[4], float ks, bool valid,
                                                 const double (*qd)[4], const float* qw) {
#pragma clang fp contract(off)
  const int h = threadIdx.x & 3;
  double s = 0.0;
  double d = 0.0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t kw = raw[j >> 2][j & 3];
    // fp8 -> f32 exactly, two codes per convert
    const f32x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(kw, 1.0f, false);
    const f32x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(kw, 1.0f, true);
    const float kv[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
    for (int b = 0; b < 4; ++b) d = __builtin_fma(qd[4 * j + b][h], (double)kv[b], d);  // exact
  }
  const double ph = (d > 0.0 ? d : 0.0) * (double)qw[h];
  const double p0 = __shfl(ph, (threadIdx.x & ~3) | 0, 64), p1 = __shfl(ph, (threadIdx.x & ~3) | 1, 64);
  const double p2 = __shfl(ph, (threadIdx.x & ~3) | 2, 64), p3 = __shfl(ph, (threadIdx.x & ~3) | 3, 64);
  s = (double)ks * (((p0 + p1) + p2) + p3);
  return valid ? s : 0.0;
}

__device__ __forceinline__ double exact_score_at(const IndexPass& p, int row, int64_t pos, bool valid,
                                                 const double (*qd)[4], const float* qw) {
  u32x4_t raw[4] = {};
  float ks = 0.0f;
  if (valid) load_key_row(p, row, pos, raw, ks, threadIdx.x & 3);  // (shared keys: every lane loads the one key)
  return exact_from_raw(raw, ks, valid, qd, qw);
}

// Exact score of item `item` of `row` (quad-collective, as exact_score_at).
// Items of a block-max pass are blocks: the largest exact score among the
// block's visible positions.
__device__ __forceinline__ double exact_score(const IndexPass& p, int row, uint32_t item, bool valid,
                                              const double (*qd)[4], const float* qw) {
  if (p.block_level != 2) return exact_score_at(p, row, item_to_position(p, row, item), valid, qd, qw);
  const int64_t vis = row_vis_positions(p, row);
  double best = 0.0;
  bool any = false;
#pragma unroll 1
  for (int j = 0; j < 8; ++j) {
    // (the query values are re-read from LDS each time: held across the
    // loop they would take 128 registers)
    asm volatile("" ::: "memory");
    const int64_t pos = 8 * (int64_t)item + j;
    const bool v = valid && pos < vis;
    const double e = exact_score_at(p, row, pos, v, qd, qw);
    if (v && (!any || e > best)) best = e;
    any |= v;
  }
  return best;
}

// Exact ranking of the near-tie band: items bitem[0 .. nb) (nb <= kBandMax)
// are rescored exactly and the r best by (score descending, position
// ascending) are flagged in bwin.  The items of a band are distinct, and
// items ascend with positions (lists are ascending, kept blocks too), so
// position ties are broken by item.
__device__ __forceinline__ void rank_band(const IndexPass& p, int row, uint32_t nb, uint32_t r, const uint32_t* bitem,
                                          double* bscore, uint32_t* bwin, const double (*qd)[4], const float* qw) {
#pragma clang fp contract(off)
  const int t = threadIdx.x;
  if (p.block_level == 2) {  // blocks: each the best of 8 positions (rare, small bands)
    for (uint32_t m0 = 0; m0 < nb; m0 += 64) {
      const uint32_t m = m0 + (t >> 2);
      const bool valid = m < nb;
      const double s = exact_score(p, row, valid ? bitem[m] : 0u, valid, qd, qw);
      if (valid && (t & 3) == 0) bscore[m] = s;
    }
  } else {
    // a quad takes keys m, m + 64, m + 128, m + 192 of a pass: their loads
    // all go out before the arithmetic, so a band of up to 256 keys costs
    // one round trip
    constexpr int kPerQuad = 4;
    for (uint32_t m0 = 0; m0 < nb; m0 += 64 * kPerQuad) {
      u32x4_t raw[kPerQuad][4];
      float ks[kPerQuad];
      // (slot groups past the band are skipped as a whole: the condition is
      // the same for every thread)
#pragma unroll
      for (int i = 0; i < kPerQuad; ++i) {
        const uint32_t m = m0 + (t >> 2) + 64 * i;
        raw[i][0] = raw[i][1] = raw[i][2] = raw[i][3] = u32x4_t{0, 0, 0, 0};
        ks[i] = 0.0f;
        if (m < nb) load_key_row(p, row, item_to_position(p, row, bitem[m]), raw[i], ks[i], t & 3);
      }
      // (the arithmetic key by key: done for the four keys at once the
      // compiler holds all their converted values and the query's at once)
#pragma unroll
      for (int i = 0; i < kPerQuad; ++i) {
        if (m0 + 64 * i >= nb) break;  // uniform
        const uint32_t m = m0 + (t >> 2) + 64 * i;
        const double sc = exact_from_raw(raw[i], ks[i], m < nb, qd, qw);
        if (m < nb && (t & 3) == 0) bscore[m] = sc;
      }
    }
  }
  __syncthreads();
  // rank of band key m = keys of the band ahead of it; a small band's
  // comparisons are split over up to four threads per key (partial ranks
  // summed in bwin), so every thread of the workgroup takes part
  const uint32_t parts = nb <= 64 ? 4u : nb <= 128 ? 2u : 1u;
  for (uint32_t m = t; m < nb; m += 256) bwin[m] = 0u;
  __syncthreads();
  for (uint32_t idx = t; idx < nb * parts; idx += 256) {
    const uint32_t m = idx % nb, part = idx / nb;
    const uint32_t j0 = part * nb / parts, j1 = (part + 1) * nb / parts;
    const double sm = bscore[m];
    const uint32_t im = bitem[m];
    uint32_t rank = 0;
    // eight keys' loads in flight per step: one at a time, the loop is
    // bound by the LDS latency
    uint32_t j = j0;
    for (; j + 8 <= j1; j += 8) {
      double sj[8];
      uint32_t ij[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        sj[u] = bscore[j + u];
        ij[u] = bitem[j + u];
      }
      // (bitwise, not short-circuit: no branch per comparison)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        rank += (sj[u] > sm ? 1u : 0u) | ((sj[u] == sm ? 1u : 0u) & (ij[u] < im ? 1u : 0u));
    }
    for (; j < j1; ++j) {
      const double sj = bscore[j];
      rank += (sj > sm ? 1u : 0u) | ((sj == sm ? 1u : 0u) & (bitem[j] < im ? 1u : 0u));
    }
    atomicAdd(&bwin[m], rank);
  }
  __syncthreads();
  for (uint32_t m = t; m < nb; m += 256) bwin[m] = bwin[m] < r ? 1u : 0u;
  __syncthreads();
}

// Score-key bounds of the near-tie band around the k-th key: keys above hi
// win for sure, keys below lo lose for sure (each score is within delta of
// the exact one, so a key more than 2 delta above the k-th has at most
// k - 1 keys above it exactly, and one more than 2 delta below has at least
// k).  Rounded outwards.
__device__ __forceinline__ void band_bounds(uint64_t kth, float delta, uint32_t& lo, uint32_t& hi) {
  const float s = key_to_score((uint32_t)(kth >> 32));
  const float d2 = 2.0f * delta + kErrTail * fabsf(s) * 2.0f;
  const float up = __builtin_fmaf(d2, 1.0f + 0x1p-12f, s);
  const float dn = __builtin_fmaf(-d2, 1.0f + 0x1p-12f, s);
  hi = score_key(up);
  hi = hi < 0xFFFFFFFFu ? hi + 1u : hi;   // one ulp outwards for the rounding of the fma
  lo = score_key(dn);
  lo = lo > 1u ? lo - 1u : 1u;
}

// The select's LDS: kPer candidates per thread, room for the segment
// starts of kChunks chunks and kWin winners.  The k-th key's histogram
// (2,048 words) shares the bitmap's memory: it is done with before the
// bitmap is cleared for the winners.
template <int kPer, int kChunks, int kWin>
struct SelLds {
  uint64_t lc[256 * kPer];               // candidates; then the near-tie band
  uint32_t bitmap[kBitmapItems / 32];    // winner bitmap; first the histogram
  uint32_t win[kWin];
  uint32_t seg_start[kChunks + 1];
  uint32_t h256[256];
  uint32_t wsum[4];
  uint32_t sh3[3];
  float qw[4];
  double qd[64][4];
  uint64_t bin_keys[64];
  uint64_t sh_kth;
  uint32_t sh_need, sh_binn, sh_nb, sh_nbge;
  uint32_t sh_red[8];
};
template <int kPer>
using SelLdsFull = SelLds<kPer, kMaxChunks, CSA2_MAX_K>;

// kPer candidates per thread, 256 kPer in all: 16 for k <= 1,024, 32 for
// the 2,048-block stage and for rows of more than 128 chunks.  Leaves the
// winners' items in ascending order in S.win (visible to every thread) and
// returns their number.  Only a `writer` writes the row's outputs and counts
// an exact recompute (several workgroups may select the same row).
template <int kPer, class Lds>
__device__ __forceinline__ uint32_t select_row(const IndexPass& p, const int row, Lds& S, const bool writer = true) {
  constexpr int kSelCap = 256 * kPer;
  const int t = threadIdx.x, quarter = t & 3;
  const int wave = t >> 6, lane = t & 63;
  const int seq = row / p.n_q;
  const int64_t vis = row_vis_positions(p, row);
  const int64_t n_items = row_items(p, row, vis);
  const int64_t csize = row_chunk_items(p, row);
  const int nch = (int)scan_chunk_count(n_items, csize);
  const uint32_t k = (uint32_t)p.k;
  const u32x4_t* info_row = p.chunk_info + (int64_t)row * p.max_chunks;
  const uint64_t* segs = p.seg_list + (int64_t)row * p.max_chunks * kSeg;

  static_assert(sizeof(S.lc) == kSelCap * 8, "candidate room");
  constexpr uint32_t kWinCap = sizeof(S.win) / 4;
  uint32_t* seg_start = S.seg_start;
  uint64_t* lc = S.lc;
  uint32_t* bitmap = S.bitmap;
  uint32_t* win = S.win;
  uint32_t* h256 = S.h256;
  uint32_t* h2048 = S.bitmap;  // (the histogram is done before the bitmap is cleared)
  uint32_t* wsum = S.wsum;
  uint32_t* sh3 = S.sh3;
  float* qw = S.qw;
  double (*qd)[4] = S.qd;
  uint64_t* bin_keys = S.bin_keys;
  uint64_t& sh_kth = S.sh_kth;
  uint32_t &sh_need = S.sh_need, &sh_binn = S.sh_binn, &sh_nb = S.sh_nb, &sh_nbge = S.sh_nbge;
  uint32_t* sh_red = S.sh_red;
  auto info_at = [&](int c) __attribute__((always_inline)) -> u32x4_t { return info_row[c]; };
  auto seg_at = [&](int c, uint32_t i) __attribute__((always_inline)) -> uint64_t {
    return segs[(int64_t)c * kSeg + i];
  };
  auto seg2_at = [&](int c, uint32_t i) __attribute__((always_inline)) -> uint4 {  // slots i, i + 1
    return *reinterpret_cast<const uint4*>(segs + (int64_t)c * kSeg + i);
  };
  // the near-tie band (in lc once the candidates are in registers)
  constexpr uint32_t kBandCap = kSelCap / 2 < kBandMax ? kSelCap / 2 : kBandMax;  // 16 bytes a band key
  uint32_t* bitem = reinterpret_cast<uint32_t*>(lc);
  uint32_t* bwin = bitem + kBandCap;
  double* bscore = reinterpret_cast<double*>(lc) + kBandCap;

  // Rows of at most kSpecCh chunks load every chunk's record and the first
  // slots of every segment (band 0 fits: 32 slots when band 0 holds at most
  // 32 keys, else 64) in one round trip: wave w takes chunks
  // G (w + 4 j) + lane / (64 / G), G chunks per wave instruction, each lane
  // two slots.  Every wave holds the records of chunks l and l + 64 in lane
  // l, so its own prefix sums give every chunk's band-0 start and its own
  // ballots decide which chunks need band 1, with no workgroup barrier.
  constexpr int kSpecCh = kPer <= 16 ? kSpecChunks : 2 * kSpecChunks;
  const bool spec = nch <= kSpecCh;
  const bool slots32 = band0_size(n_items, csize, nch, (int)k) <= 32u;
  u32x4_t ia = u32x4_t{0, 0, 0, 0}, ib = u32x4_t{0, 0, 0, 0};
  uint4 sv[kSpecCh / 8];
  if (spec) {
    if (lane < nch) ia = info_at(lane);
    if (kSpecCh > 64 && lane + 64 < nch) ib = info_at(lane + 64);
    if (slots32) {  // 4 chunks of 32 slots per instruction
#pragma unroll
      for (int j = 0; j < kSpecCh / 16; ++j) {
        const int ch = 4 * (wave + 4 * j) + (lane >> 4);
        sv[j] = ch < nch ? seg2_at(ch, 2 * (lane & 15)) : make_uint4(0, 0, 0, 0);
      }
    } else {  // 2 chunks of 64 slots per instruction
#pragma unroll
      for (int j = 0; j < kSpecCh / 8; ++j) {
        const int ch = 2 * (wave + 4 * j) + (lane >> 5);
        sv[j] = ch < nch ? seg2_at(ch, 2 * (lane & 31)) : make_uint4(0, 0, 0, 0);
      }
    }
  }
  const float cq = load_query_codes(p, row, qw, qd);
  // band-0 counts and starts, the row's largest key and key scale
  uint32_t total, rowmax = 0u, ksm = 0u;
  if (spec) {
    const uint32_t na = rec_n0(ia), nb = rec_n0(ib);
    rowmax = wave_max_u32(max(ia[1], ib[1]));
    ksm = wave_max_u32(max(ia[3], ib[3]));
    const uint32_t incl_a = wave_incl_add(na);
    const uint32_t tot_a = (uint32_t)__builtin_amdgcn_readlane((int)incl_a, 63);
    total = tot_a;
    if (wave == 0) seg_start[lane] = incl_a - na;
    if constexpr (kSpecCh > 64) {
      const uint32_t incl_b = wave_incl_add(nb);
      if (wave == 0) seg_start[lane + 64] = tot_a + incl_b - nb;
      total = tot_a + (uint32_t)__builtin_amdgcn_readlane((int)incl_b, 63);
    }
    if (wave == 0 && lane == 0) seg_start[nch] = total;
  } else {
    // thread t owns chunks 16t .. 16t+15 (a row has at most 4,096)
    uint32_t c[16], local = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int ch = 16 * t + j;
      const u32x4_t r = ch < nch ? info_at(ch) : u32x4_t{0, 0, 0, 0};
      c[j] = rec_n0(r);
      rowmax = max(rowmax, r[1]);
      ksm = max(ksm, r[3]);
      local += c[j];
    }
    rowmax = wave_max_u32(rowmax);
    ksm = wave_max_u32(ksm);
    if (lane == 0) {
      sh_red[wave] = rowmax;
      sh_red[4 + wave] = ksm;
    }
    uint32_t run = block_incl_scan_256(local, wsum, total) - local;  // (its barriers publish sh_red)
    rowmax = max(max(sh_red[0], sh_red[1]), max(sh_red[2], sh_red[3]));
    ksm = max(max(sh_red[4], sh_red[5]), max(sh_red[6], sh_red[7]));
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int ch = 16 * t + j;
      if (ch < nch) seg_start[ch] = run;
      run += c[j];
    }
    if (t == 0) seg_start[nch] = total;
  }
  const float delta = (p.mfma_scores ? kErrMfma : kErrValu) * cq * 448.0f * __uint_as_float(ksm);
  if (writer && p.row_ksm && p.block_level == 0 && t == 0) p.row_ksm[row] = ksm;

  bool fast = total <= (uint32_t)kSelCap;
  uint32_t n_win = 0;
  const bool use_bitmap = n_items <= (int64_t)kBitmapItems;
  if (fast) {
    for (int i = t; i < 2048; i += 256) h2048[i] = 0u;
    if (t == 0) {
      sh_nb = 0;
      sh_nbge = 0;
      sh_binn = 0;
      sh_need = 0;
    }
    __syncthreads();  // seg_start, qd, qw
    // band 0 into lc
    if (spec) {
      if (slots32) {
#pragma unroll
        for (int j = 0; j < kSpecCh / 16; ++j) {
          const int ch = 4 * (wave + 4 * j) + (lane >> 4);
          if (ch < nch) {
            const uint32_t b = seg_start[ch], n = seg_start[ch + 1] - b;
            const uint32_t s0 = 2u * (lane & 15);
            if (s0 < n) lc[b + s0] = ((uint64_t)sv[j].y << 32) | sv[j].x;
            if (s0 + 1u < n) lc[b + s0 + 1] = ((uint64_t)sv[j].w << 32) | sv[j].z;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < kSpecCh / 8; ++j) {
          const int ch = 2 * (wave + 4 * j) + (lane >> 5);
          if (ch < nch) {
            const uint32_t b = seg_start[ch], n = seg_start[ch + 1] - b;
            const uint32_t s0 = 2u * (lane & 31);
            if (s0 < n) lc[b + s0] = ((uint64_t)sv[j].y << 32) | sv[j].x;
            if (s0 + 1u < n) lc[b + s0 + 1] = ((uint64_t)sv[j].w << 32) | sv[j].z;
          }
        }
      }
    } else {
      // wave w copies chunks w, w + 4, ..., eight at a time (loads first)
      for (int c0 = wave; c0 < nch; c0 += 32) {
        uint64_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int ch = c0 + 4 * j;
          const uint32_t n = ch < nch ? seg_start[ch + 1] - seg_start[ch] : 0u;
          v[j] = (uint32_t)lane < n ? seg_at(ch, lane) : 0ull;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int ch = c0 + 4 * j;
          const uint32_t n = ch < nch ? seg_start[ch + 1] - seg_start[ch] : 0u;
          if ((uint32_t)lane < n) lc[seg_start[ch] + lane] = v[j];
        }
      }
    }
    __syncthreads();
    uint64_t key[kPer];
    auto to_regs = [&](uint32_t tot) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const uint32_t g = t + 256 * i;
        key[i] = g < tot ? lc[g] : 0ull;  // 0 is below every candidate key
      }
    };
    // the k-th largest key (more than k keys): its bin in a histogram of
    // the distance below the row's largest key (2,048 bins of 2^13 key
    // units, 1/1024 of a binade; the last takes the rest), then its rank
    // among that bin's few keys; a radix over every key when the bin is the
    // last one or holds more than 64
    auto kth_of = [&](bool zeroed) __attribute__((always_inline)) -> uint64_t {
      if (!zeroed) {
        for (int i = t; i < 2048; i += 256) h2048[i] = 0u;
        if (t == 0) sh_binn = 0;
        __syncthreads();
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (key[i] != 0ull) {
          const uint32_t d = (rowmax - (uint32_t)(key[i] >> 32)) >> 13;
          atomicAdd(&h2048[d < 2047u ? d : 2047u], 1u);
        }
      }
      __syncthreads();
      uint32_t hb[8], local = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        hb[j] = h2048[8 * t + j];
        local += hb[j];
      }
      uint32_t tot;
      uint32_t run = block_incl_scan_256(local, wsum, tot) - local;  // keys in bins before 8t
      if (run < k && run + local >= k) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (run < k && run + hb[j] >= k) {
            sh3[0] = 8 * t + j;
            sh3[1] = k - run;
            sh3[2] = hb[j];
          }
          run += hb[j];
        }
      }
      __syncthreads();
      const uint32_t kbin = sh3[0], need = sh3[1], in_bin = sh3[2];
      if (kbin < 2047u && in_bin <= 64u) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          if (key[i] != 0ull && ((rowmax - (uint32_t)(key[i] >> 32)) >> 13) == kbin) {
            const uint32_t slot = atomicAdd(&sh_binn, 1u);
            if (slot < 64u) bin_keys[slot] = key[i];
          }
        }
        __syncthreads();
        // lane l ranks bin key l among them by register reads (every wave alike)
        const uint64_t mine = lane < (int)in_bin ? bin_keys[lane] : 0ull;
        uint32_t rank = 0;
        for (uint32_t j = 0; j < in_bin; ++j) {
          const uint64_t other = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mine >> 32), (int)j) << 32) |
                                 (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine, (int)j);
          rank += other > mine ? 1u : 0u;
        }
        const unsigned long long pick = __ballot(lane < (int)in_bin && rank == need - 1);
        const int src = __ffsll((long long)pick) - 1;
        return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mine >> 32), src) << 32) |
               (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine, src);
      }
      const uint64_t e = block_kth_regs<kPer>(key, k, h2048, wsum, sh3);
      return block_min_at_least<kPer>(key, e);
    };
    to_regs(total);
    uint64_t kth = total > k ? kth_of(true) : 0ull;
    uint32_t lo = 1u, hi = 0xFFFFFFFFu;
    if (total > k) band_bounds(kth, delta, lo, hi);
    // A chunk is open when keys below its band 0 may still reach the band
    // (its band-0 edge lies above the band's lower bound): its band 1 is
    // gathered, a second round trip.  Spec rows decide it by ballot in every
    // wave; the others through thread t's chunks 16t .. 16t+15.
    auto opens = [&](const u32x4_t& r) __attribute__((always_inline)) -> bool {
      return rec_thi(r) > lo && (rec_ntot(r) > rec_n0(r) || r[2] == 0u);
    };
    bool open;
    if (spec) {
      open = __ballot((lane < nch && opens(ia)) || (kSpecCh > 64 && lane + 64 < nch && opens(ib))) != 0ull;
    } else {
      bool any = false;
      for (int j = 0; j < 16; ++j) {
        const int ch = 16 * t + j;
        if (ch < nch) any |= opens(info_at(ch));
      }
      open = __syncthreads_or(any ? 1 : 0) != 0;
    }
    if (open) {
      // band-1 counts of the open chunks and their starts after band 0
      uint32_t n1[16], local = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int ch = 16 * t + j;
        n1[j] = 0u;
        if (ch < nch) {
          const u32x4_t r = info_at(ch);
          if (opens(r)) n1[j] = rec_ntot(r) - rec_n0(r);
        }
        local += n1[j];
      }
      uint32_t more;
      uint32_t run = block_incl_scan_256(local, wsum, more) - local;
      const uint32_t tot2 = total + more;
      fast = tot2 <= (uint32_t)kSelCap;
      if (fast) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int ch = 16 * t + j;
          if (ch < nch) seg_start[ch] = total + run;
          run += n1[j];
        }
        __syncthreads();
        // wave w copies the band 1 of chunks w, w + 4, ..., four at a time
        for (int c0 = wave; c0 < nch; c0 += 16) {
          uint64_t v[4][2];
          uint32_t nn[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int ch = c0 + 4 * j;
            uint32_t n0 = 0u;
            nn[j] = 0u;
            if (ch < nch) {
              const u32x4_t r = info_at(ch);
              n0 = rec_n0(r);
              if (opens(r)) nn[j] = rec_ntot(r) - n0;
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t i = lane + 64 * h;
              v[j][h] = i < nn[j] ? seg_at(ch, n0 + i) : 0ull;
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int ch = c0 + 4 * j;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t i = lane + 64 * h;
              if (i < nn[j]) lc[seg_start[ch] + i] = v[j][h];
            }
          }
        }
        __syncthreads();
        total = tot2;
        to_regs(total);
        kth = total > k ? kth_of(false) : 0ull;
        lo = 1u;
        hi = 0xFFFFFFFFu;
        if (total > k) band_bounds(kth, delta, lo, hi);
        // every chunk's dropped keys (below its band-1 edge) must lie below the band
        bool dropped = false;
        for (int c = t; c < nch; c += 256) dropped |= rec_tlo(info_at(c)) > lo;
        fast = __syncthreads_or(dropped ? 1 : 0) == 0;
      }
    }
    // Without band 1, lc holds band 0 of every chunk in chunk order, and each
    // segment lists its band in item order: the candidates ascend by item,
    // and compacting the winners in lc order orders them
    const bool ordered = !open;
    if (fast && use_bitmap && !ordered) {  // the histogram is done with: clear the bitmap
      uint4* bm4 = reinterpret_cast<uint4*>(bitmap);
      for (int i = t; i < kBitmapItems / 128; i += 256) bm4[i] = make_uint4(0, 0, 0, 0);
      __syncthreads();
    }
    if (fast) {
      // Winners.  With more than k candidates: keys above hi win for sure
      // (into the bitmap at once, when it orders them); keys in [lo, hi]
      // form the near-tie band, of which the keys at or above the k-th
      // number r = k - (sure winners): if the band holds just r keys they
      // all win, otherwise the band is rescored exactly and its r best win.
      // With at most k candidates (and no chunk dropping a key) every
      // candidate wins.
      const bool all = total <= k;
      if (!use_bitmap && t == 0) sh_need = 0;  // (published by the barrier below)
      uint32_t bslot[kPer];  // 1 + the key's slot in the near-tie band; 0 outside it
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        bslot[i] = 0u;
        const uint32_t sk = (uint32_t)(key[i] >> 32);
        if (key[i] == 0ull) continue;
        if (all || sk > hi) {
          const uint32_t it = select_key_pos(key[i]);
          if (use_bitmap && !ordered) atomicOr(&bitmap[bitmap_slot(it >> 5)], 1u << (it & 31u));
        } else if (sk >= lo) {
          const uint32_t at = atomicAdd(&sh_nb, 1u);
          if (at < kBandCap) bitem[at] = select_key_pos(key[i]);
          bslot[i] = at + 1u;
          if (key[i] >= kth) atomicAdd(&sh_nbge, 1u);
        }
      }
      __syncthreads();
      const uint32_t nb = sh_nb, r = sh_nbge;
      if (nb > kBandCap) {
        fast = false;  // a band this wide: the exact recompute settles the row
      } else if (nb > r) {
        rank_band(p, row, nb, r, bitem, bscore, bwin, qd, qw);
      } else {
        for (uint32_t m = t; m < nb; m += 256) bwin[m] = 1u;
        __syncthreads();
      }
      if (fast && ordered) {
        // compaction in lc order (slot t + 256 i): per-wave winner counts of
        // each i, then every thread adds up the counts ahead of its slots
        uint32_t* wcnt = bitmap;  // [kPer][4] (the bitmap is unused here)
        uint64_t bal[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const uint32_t sk = (uint32_t)(key[i] >> 32);
          const bool f = key[i] != 0ull && (all || sk > hi || (bslot[i] != 0u && bwin[bslot[i] - 1u] != 0u));
          bal[i] = __ballot(f);
          if (lane == 0) wcnt[4 * i + wave] = (uint32_t)__popcll(bal[i]);
        }
        __syncthreads();
        uint32_t run = 0u;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const uint4 c4 = reinterpret_cast<const uint4*>(wcnt)[i];
          const uint32_t ahead = run + (wave > 0 ? c4.x : 0u) + (wave > 1 ? c4.y : 0u) + (wave > 2 ? c4.z : 0u);
          if ((bal[i] >> lane) & 1ull) {
            const uint32_t below =
                __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[i] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal[i], 0u));
            win[ahead + below] = select_key_pos(key[i]);
          }
          run += (c4.x + c4.y) + (c4.z + c4.w);
        }
        n_win = run;
        __syncthreads();
      } else if (fast) {
        if (use_bitmap) {
          for (uint32_t m = t; m < nb; m += 256) {
            if (bwin[m]) {
              const uint32_t it = bitem[m];
              atomicOr(&bitmap[bitmap_slot(it >> 5)], 1u << (it & 31u));
            }
          }
          __syncthreads();
          // thread t owns words 16t .. 16t+15 (512 items); each winner goes
          // to slot (winners before its word) + (set bits below it)
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
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            uint32_t b = wb[j];
            while (b) {
              const int bit = __ffs(b) - 1;
              win[o++] = 32u * (16 * t + j) + (uint32_t)bit;
              b &= b - 1u;
            }
          }
          __syncthreads();
        } else {
          // compaction, then a bitonic sort padded to a power of two
#pragma unroll
          for (int i = 0; i < kPer; ++i) {
            const uint32_t sk = (uint32_t)(key[i] >> 32);
            if (key[i] != 0ull && (all || sk > hi)) win[atomicAdd(&sh_need, 1u)] = select_key_pos(key[i]);
          }
          for (uint32_t m = t; m < nb; m += 256)
            if (bwin[m]) win[atomicAdd(&sh_need, 1u)] = bitem[m];
          __syncthreads();
          n_win = sh_need;
          uint32_t n2 = 1;
          while (n2 < n_win) n2 <<= 1;
          for (uint32_t i = n_win + t; i < n2; i += 256) win[i] = 0xFFFFFFFFu;
          __syncthreads();
          for (uint32_t size = 2; size <= n2; size <<= 1) {
            for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
              for (uint32_t i = t; i < n2 / 2; i += 256) {
                const uint32_t lo2 = 2 * i - (i & (stride - 1));
                const uint32_t hi2 = lo2 + stride;
                const bool asc = (lo2 & size) == 0;
                const uint32_t a = win[lo2], b = win[hi2];
                if ((a > b) == asc) {
                  win[lo2] = b;
                  win[hi2] = a;
                }
              }
              __syncthreads();
            }
          }
        }
      }
    }
  }
  if (!fast) {
    // exact recompute of this row (rare): every item's score again, a radix
    // over the (score, -item) keys for the k-th, then the near-tie band
    // rescored exactly as above
    if (t == 0) {
      if (writer) atomicAdd(p.fallbacks, 1u);
      sh_nb = 0;
    }
    half2_t q[kHI][8];
    float w_mine;
    load_query_f16(p, row, quarter, q, w_mine);
    auto visit = [&](uint32_t n, auto&& f) {
      for (uint32_t base = 0; base < n; base += 64) {
        const uint32_t item = base + (t >> 2);
        bool valid = false;
        const int64_t pos = item < n ? item_position(p, row, item, n, vis, valid) : 0;
        const float sc = item_score_at(p, q, w_mine, seq, quarter, pos, valid, vis);
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
    uint32_t lo = 1u, hi = 0xFFFFFFFFu, nb = 0, r = 0;
    // (the fallback scores on VALU even where the scan used MFMA)
    const float delta_v = kErrValu * cq * 448.0f * ksm;
    if (n_valid > k) {
      kth = radix_kth<uint64_t>(visit, ni, k, h256, &sh_kth, &sh_need);
      band_bounds(kth, delta_v, lo, hi);
      // the band's items (at most kBandMax: wider bands keep the binary32 order)
      uint32_t sure_l = 0;
      visit(ni, [&](uint64_t kk) {
        const uint32_t sk = (uint32_t)(kk >> 32);
        if (sk > hi) ++sure_l;
        else if (sk >= lo) {
          const uint32_t at = atomicAdd(&sh_nb, 1u);
          if (at < kBandCap) bitem[at] = select_key_pos(kk);
        }
      });
      uint32_t sure;
      (void)block_incl_scan_256(sure_l, wsum, sure);
      nb = sh_nb;
      r = k - sure;
      if (nb > r && nb <= kBandCap) {
        // ascending items, so the emission below can binary-search them
        if (t == 0) {
          for (uint32_t i = 1; i < nb; ++i) {
            const uint32_t v = bitem[i];
            uint32_t j = i;
            while (j > 0 && bitem[j - 1] > v) { bitem[j] = bitem[j - 1]; --j; }
            bitem[j] = v;
          }
        }
        __syncthreads();
        rank_band(p, row, nb, r, bitem, bscore, bwin, qd, qw);
      }
    }
    const bool ranked = nb > r && nb <= kBandCap;
    for (uint32_t base = 0; base < ni; base += 64) {
      const uint32_t item = base + (t >> 2);
      bool valid = false;
      const int64_t pos = item < ni ? item_position(p, row, item, ni, vis, valid) : 0;
      const float sc = item_score_at(p, q, w_mine, seq, quarter, pos, valid, vis);
      const uint64_t kk = select_key(score_key(sc), item);
      bool f = valid && quarter == 0;
      if (f && n_valid > k) {
        const uint32_t sk = (uint32_t)(kk >> 32);
        if (!ranked) {
          f = kk >= kth;
        } else if (sk > hi) {
          f = true;
        } else if (sk < lo) {
          f = false;
        } else {
          uint32_t a = 0, b = nb;  // binary search of the band's items
          while (a < b) {
            const uint32_t m = (a + b) >> 1;
            if (bitem[m] < item) a = m + 1; else b = m;
          }
          f = a < nb && bitem[a] == item && bwin[a] != 0u;
        }
      }
      uint32_t nr;
      const uint32_t o = block_incl_scan_256(f ? 1u : 0u, wsum, nr) - (f ? 1u : 0u);
      if (f && n_win + o < kWinCap) win[n_win + o] = item;
      n_win += nr;
    }
    if (n_win > k) n_win = k;
    __syncthreads();
  }

  if (!writer) return n_win;
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
  return n_win;
}

template <int kPer>
__global__ __launch_bounds__(256) void k_index_select(IndexPass p) {
  __shared__ SelLdsFull<kPer> S;
  select_row<kPer>(p, blockIdx.x, S);
}

// The select of a decode index pass fused with the group's whole attention
// launch.  Workgroup (row, j) with j < n_sel: selected-entry tile j / n_groups
// of layer pair j % n_groups.  It selects the row's winners itself (every
// such workgroup of a row reaches the same set and order: the select is
// deterministic), takes winners 64 tile .. +63 from LDS and attends over
// them as the tile form does (pair_step); workgroup (row, 0) writes the
// row's indices.  The other workgroups take the window tiles, one
// workgroup per (row, layer) walking its tiles.  Against a
// select launch followed by a tile launch this drops a kernel boundary and
// the tiles' round trip for their positions; the repeated selects read the
// same candidate segments (about 20 KB a row, mostly from L2).  The select
// and the tile take about 78 KB of LDS each, so two workgroups fit on a CU.
__global__ __launch_bounds__(256, 2) void k_index_select_attend(IndexPass p, AttnPass a) {
  __shared__ __attribute__((aligned(16))) union {
    SelLdsFull<16> sel;
    PairLds pair;
  } U;
  const int n_tile_idx = (a.n_idx + kAttnSplit - 1) / kAttnSplit;
  const int n_win_tiles = a.n_tiles - n_tile_idx;
  const int n_groups = (a.n_layers + 1) / 2;
  const int n_sel = n_tile_idx * n_groups;
  const int n_wt = a.n_layers;  // window workgroups per row: one per layer, walking its window tiles
  // the selected-entry workgroups of every row first, then the window
  // tiles, so the dispatcher spreads the long-running ones over the CUs
  // before any CU takes a second workgroup; workgroup ids are dealt
  // round-robin over the 8 XCDs: with a multiple of 8 rows, every workgroup
  // of row r runs on XCD r mod 8
  const int grows = a.rows >= kXcds ? (a.rows + kXcds - 1) / kXcds * kXcds : a.rows;
  const bool sel_part = (int)blockIdx.x < grows * n_sel;
  const int b = sel_part ? (int)blockIdx.x : (int)blockIdx.x - grows * n_sel;
  const int per = sel_part ? n_sel : n_wt;
  int row, j;
  if (a.rows >= kXcds && a.rows % kXcds == 0) {
    const int xcd = b & (kXcds - 1), w = b >> 3;
    row = xcd + kXcds * (w / per);
    j = w % per;
  } else {
    row = b / per;
    j = b - row * per;
  }
  if (!sel_part) j += n_sel;
  if (row >= a.rows) return;
  if (j >= n_sel) {
    for (int wt = 0; wt < n_win_tiles; ++wt) {
      if (wt) __syncthreads();  // the previous tile's readers of the LDS are done
      window_tile(a, row, j - n_sel, wt, U.pair.t);
    }
    return;
  }
  const int tile = j / n_groups, l0 = 2 * (j % n_groups);
  const uint32_t n_win = select_row<16>(p, row, U.sel, j == 0);
  const uint32_t c = (uint32_t)(tile * kAttnSplit + (threadIdx.x & 63));
  const int32_t pos = c < n_win && (int)c < a.n_idx ? item_to_position(p, row, U.sel.win[c]) : -1;
  __syncthreads();  // the winners are read: the LDS becomes the tile
  const int seq = row / a.n_q;
  const int nl = a.n_layers - l0 < 2 ? a.n_layers - l0 : 2;
  const float sc2 = a.softmax_scale * 1.4426950408889634f;  // logits in the log2 domain
  uint4 qb[16];
  EntryFetch f;
  fetch_entry<false>(a, seq, pos, f);
  stage_q_pair(a, l0, nl, row, U.pair, qb);
  store_entry<false>(f, U.pair.t);
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};
  f32x4_t o[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[i][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  pair_step(U.pair, qb, nl == 2 ? 3 : 1, sc2, m_run, l_run, o);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i >= nl) break;  // uniform
    write_partial(a, (l0 + i) * a.rows + row, tile, m_run[i], l_run[i], o[i]);
  }
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

// Scan chunks per row of a pass, at most (the grid's chunk dimension): over
// direct items from every sequence's item count, otherwise from the largest
// row.
static int pass_chunks_per_row(const IndexPass& p) {
  auto chunks = [&](int64_t n) { return n > 0 ? scan_chunk_count(n, scan_chunk_items(n, p.k)) : 0; };
  int64_t m = chunks(p.max_items);
  if (p.source == kItemsDirect) {
    for (int s = 0; s < p.rows / p.n_q; ++s) {
      const int64_t pos = p.seq.a[s] + p.n_q - 1;
      int64_t vis = p.ratio == 2 ? (pos + 1) >> 1 : pos + 1;
      vis = std::min(vis, p.seq.b[s]);
      const int64_t n = p.block_level ? (vis + 7) >> 3 : vis;
      m = std::max(m, chunks(std::min(n, p.max_items)));
    }
  } else {
    // block lists of fewer items can take more, smaller chunks: just below a
    // size where the chunks double, a row has 2 k / chunk_winners(k) of them
    const int64_t peak = 2 * (int64_t)p.k / chunk_winners(p.k);
    m = std::max(m, std::min(peak, (p.max_items + 127) / 128));
  }
  return (int)m;
}

// The fused select + attention launch takes a token-level pass whose
// attention is in the tile form over the pass's own rows and k winners.
static bool attend_fits(const IndexPass& p, const AttnPass& a) {
  return p.block_level == 0 && a.n_idx == p.k && a.rows == p.rows && a.n_layers >= 1 && a.tiles_per_split == 1 &&
         a.max_splits == a.n_tiles;
}

hipError_t launch_index_pass(const IndexPass& p0, hipStream_t stream, const AttnPass* attn, bool* attended) {
  if (attended) *attended = false;
  if (p0.rows == 0 || p0.max_items == 0) return hipSuccess;
  IndexPass p = p0;
  const int scan_per_row = pass_chunks_per_row(p);
  if (scan_per_row > p.max_chunks) return hipErrorInvalidValue;
  // the queries of a sequence share the scan of a chunk, up to 4 per
  // workgroup (direct items only), on fp8 MFMA
  const int nqg = (p.source != kItemsDirect || p.n_q == 1 || p.key_heads == 4) ? 1 : p.n_q == 2 ? 2 : 4;
  p.mfma_scores = nqg > 1 ? 1 : 0;
  const int n_groups = nqg == 1 ? p.rows : p.rows / p.n_q * ((p.n_q + nqg - 1) / nqg);
  const dim3 sgrid((unsigned)(grid_rows(n_groups) * scan_per_row));
  const bool paged = p.pm.pages != nullptr;  // (direct items only: the host refuses the others)
  int h = prof_begin(CSA2_K_INDEX_SCAN, stream);
  if (p.block_level == 2)
    hipLaunchKernelGGL(k_index_scan_keys, dim3((unsigned)(grid_rows(p.rows) * scan_per_row)), dim3(256), 0, stream, p,
                       scan_per_row);
  else if (p.key_heads == 4 && p.source != kItemsDirect)
    hipLaunchKernelGGL((k_index_scan<2, false, false, true>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else if (p.key_heads == 4)
    hipLaunchKernelGGL((k_index_scan<2, true, false, true>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else if (p.source != kItemsDirect)
    hipLaunchKernelGGL((k_index_scan<2, false, false>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else if (nqg == 1 && paged)
    hipLaunchKernelGGL((k_index_scan<2, true, true>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else if (nqg == 1)
    hipLaunchKernelGGL((k_index_scan<2, true, false>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else if (nqg == 2 && paged)
    hipLaunchKernelGGL((k_index_scan_mfma<2, true>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else if (nqg == 2)
    hipLaunchKernelGGL((k_index_scan_mfma<2, false>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else if (paged)
    hipLaunchKernelGGL((k_index_scan_mfma<4, true>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  else
    hipLaunchKernelGGL((k_index_scan_mfma<4, false>), sgrid, dim3(256), 0, stream, p, scan_per_row, n_groups);
  prof_end(h, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  h = prof_begin(CSA2_K_INDEX_SELECT, stream);
  // 32 candidates per thread for the 2,048-block stage and for rows of more
  // than 128 chunks (their band-0 share is sized for that room)
  const bool wide = p.k > 1024 || scan_per_row > 128;
  if (wide) {
    hipLaunchKernelGGL(k_index_select<32>, dim3((unsigned)p.rows), dim3(256), 0, stream, p);
  } else if (attn && attend_fits(p, *attn)) {
    const int n_tile_idx = (attn->n_idx + kAttnSplit - 1) / kAttnSplit;
    const int per_row = n_tile_idx * ((attn->n_layers + 1) / 2) + attn->n_layers;
    const int grows = attn->rows >= kXcds ? (attn->rows + kXcds - 1) / kXcds * kXcds : attn->rows;
    hipLaunchKernelGGL(k_index_select_attend, dim3((unsigned)(grows * per_row)), dim3(256), 0, stream, p, *attn);
    if (attended) *attended = true;
  } else {
    hipLaunchKernelGGL(k_index_select<16>, dim3((unsigned)p.rows), dim3(256), 0, stream, p);
  }
  prof_end(h, stream);
  return hipGetLastError();
}

}  // namespace csa2
