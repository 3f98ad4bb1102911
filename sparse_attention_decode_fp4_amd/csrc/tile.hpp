// Tile pieces of the sparse + SWA attention shared by the attention kernels
// (attn.hip) and the decode select, whose launch also runs a group's
// attention tiles (index.hip): the LDS tile, entry and window loads, the
// staged queries, the online-softmax tile steps and the partial write.
#pragma once

#include "kernels.hpp"

namespace csa2 {

// bf16 per row of E: rows 8 banks apart.  The 16-byte chunk c of row r sits
// at c ^ row_swizzle(r): chunks swapped in pairs in rows with bit 2 set
// (rows r and r + 4 of the 16-byte MFMA operand reads fall in different
// banks) and by halves of 256 bytes in rows with bit 3 set (the transposing
// reads take rows 8 g4 + 0..3, whose bank offsets repeat every 8 rows).
// Measured with the SQ bank-conflict counters: every load and store pattern
// of the attention kernels on this layout runs without conflicts.
constexpr int kEStride = kD + 16;
__device__ __forceinline__ int row_swizzle(int r) { return ((r >> 2) & 1) | (((r >> 3) & 1) << 3); }
constexpr int kPStride = kAttnSplit + 8;

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i mod 4) of the 4-element chunk addressed by lane 4 e + (i / 4), as its
// element e.  So if lane j of group G addresses row r0 + 8 G + j / 4,
// columns c0 + 4 (j mod 4) .. +3 of E, lane (G, i) receives rows r0 + 8 G ..
// +3 of column c0 + i: 4 consecutive k of the B operand of an MFMA.
__device__ __forceinline__ v4i16_t lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)p);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  // exact values only (the rounding of the packing convert changes none);
  // one v_cvt_pk_bf16_f32 instead of a shift and a masked or
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// P values of 4 consecutive rows of one head as bf16 hi and lo parts, hi
// the round-to-nearest-even bf16 of p and lo that of p - hi (relative error
// ~2^-16), one 8-byte LDS store each (16-bit stores of single values
// conflict in the banks and take four times the instructions)
__device__ __forceinline__ void store_p4(const float (&pv)[4], uint16_t* hi_dst, uint16_t* lo_dst) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const bf16x4_t h = {(__bf16)pv[0], (__bf16)pv[1], (__bf16)pv[2], (__bf16)pv[3]};
  const bf16x4_t l = {(__bf16)(pv[0] - (float)h[0]), (__bf16)(pv[1] - (float)h[1]), (__bf16)(pv[2] - (float)h[2]),
                      (__bf16)(pv[3] - (float)h[3])};
  *reinterpret_cast<uint2*>(hi_dst) = __builtin_bit_cast(uint2, h);
  *reinterpret_cast<uint2*>(lo_dst) = __builtin_bit_cast(uint2, l);
}

struct TileLds {
  uint16_t E[kAttnSplit * kEStride];  // [row][channel]
  uint16_t Phi[kH * kPStride];
  uint16_t Plo[kH * kPStride];
  float red[4][kH];
  float alpha[kH];  // the step's rescale factor per head
  uint8_t row_ok[kAttnSplit];
};

// 16 channels (one E4M3 scale group) of one entry as bf16: 8 bytes of E2M1
// codes, low nibble first, times the group scale (exact in bf16).
__device__ __forceinline__ void dequant16(uint2 codes, float s, uint4 (&v)[2]) {
  const uint32_t wds[2] = {codes.x, codes.y};
  uint32_t o[8];
#pragma unroll
  for (int wd = 0; wd < 2; ++wd) {
    const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wds[wd], 1.0f, 0);
    const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wds[wd], 1.0f, 1);
    const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wds[wd], 1.0f, 2);
    const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wds[wd], 1.0f, 3);
    o[4 * wd + 0] = pack_bf16(v0.x * s, v0.y * s);
    o[4 * wd + 1] = pack_bf16(v1.x * s, v1.y * s);
    o[4 * wd + 2] = pack_bf16(v2.x * s, v2.y * s);
    o[4 * wd + 3] = pack_bf16(v3.x * s, v3.y * s);
  }
  v[0] = make_uint4(o[0], o[1], o[2], o[3]);
  v[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// A selected-entry tile in flight, in one of two lane layouts (kByRow).
// Both read 64-byte or longer runs of each entry per wave instruction (a
// lane per entry, 16 bytes each, would touch 64 lines per instruction and
// take several times as long).
//   kByRow = false: in load step i (0..3) wave w takes entries
//     16 w + 4 i + lane / 16, lane % 16 reading 16 bytes of codes (channels
//     32 (lane % 16) .. +31, two scale groups) and those groups' two scales:
//     4 whole entries (8 lines) per instruction, the fewest lines and the
//     shortest fetch for a tile fetched once (decode).  Its LDS stores put
//     16 lanes on one row at 64-byte steps, which conflict four ways.
//   kByRow = true: lane (g = lane / 16, l16) of wave w holds entry
//     16 w + l16 and in step i reads channels 32 (4 i + g) .. +31: 64 bytes
//     of each of 16 entries per instruction, and the 16 consecutive lanes
//     of a store write 16 rows at one column, without bank conflicts (the
//     stores of a tile take a quarter of the LDS cycles).  For kernels that
//     stream many tiles through LDS (prefill, multi-token rows).
struct EntryFetch {
  uint4 raw[4];
  uint32_t sc[4];  // the two E4M3 scales of step i in bits 0..15
  uint32_t valid;  // kByRow: the lane's entry is present; else bit i: the entry of step i
};

__device__ __forceinline__ int32_t tile_position(const AttnPass& p, int tile, int row) {
  const int c = tile * kAttnSplit + (threadIdx.x & 63);
  return c < p.n_idx ? p.idx[(int64_t)row * p.n_idx + c] : -1;
}

// `pos_lane` is the position of entry lane % 64 of the tile (-1: empty), as
// tile_position gives it.  Every load is an unconditional buffer load on a
// descriptor at the sequence start (or over the pool of a paged cache): an
// empty slot uses the entry index at the descriptors' limit
// (CSA2_MAX_ENTRIES, or the pool size), so the hardware returns zeros
// without touching memory.  No load waits on another.
template <bool kByRow>
__device__ __forceinline__ void fetch_entry(const AttnPass& p, int seq, int32_t pos_lane, EntryFetch& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  // paged caches: descriptors over the pool, and each lane first turns its
  // position into a pool entry (one page-table load)
  const bool paged = p.pm.pages != nullptr;
  const uint32_t lim = paged ? (uint32_t)p.pm.pool : (uint32_t)CSA2_MAX_ENTRIES;
  const int64_t s0 = paged ? 0 : (int64_t)seq * p.kv_stride;
  const __amdgpu_buffer_rsrc_t rn = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.nib + s0 * CSA2_NIB_BYTES), 0, (int)(lim * CSA2_NIB_BYTES), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.scale + s0 * CSA2_SCALE_BYTES), 0, (int)(lim * CSA2_SCALE_BYTES), kRawBufferWord3);
  uint32_t e_lane = pos_lane >= 0 ? (uint32_t)pos_lane : lim;
  if (paged && pos_lane >= 0) e_lane = paged_entry_at(p.pm, seq, pos_lane);
  if (kByRow) {
    const int src = 16 * wave + l16;  // the lane's entry
    const int32_t pos = __shfl(pos_lane, src, 64);
    const uint32_t e = (uint32_t)__shfl((int)e_lane, src, 64);
    f.valid = pos >= 0 ? 1u : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = 4 * i + g;  // 32 channels: code bytes 16 piece .., scale bytes 2 piece ..
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rn, (int)(e * CSA2_NIB_BYTES) + 16 * piece, 0, 0);
      f.raw[i] = make_uint4(v[0], v[1], v[2], v[3]);
      f.sc[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(e * CSA2_SCALE_BYTES) + 2 * piece, 0, 0);
    }
  } else {
    f.valid = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int src = 16 * wave + 4 * i + g;
      const int32_t pos = __shfl(pos_lane, src, 64);
      const uint32_t e = (uint32_t)__shfl((int)e_lane, src, 64);
      f.valid |= (pos >= 0 ? 1u : 0u) << i;
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rn, (int)(e * CSA2_NIB_BYTES) + 16 * l16, 0, 0);
      f.raw[i] = make_uint4(v[0], v[1], v[2], v[3]);
      f.sc[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(e * CSA2_SCALE_BYTES) + 2 * l16, 0, 0);
    }
  }
}

// Dequantise a fetched tile into E (zeros for empty slots).  kByRow: in step
// i each lane writes channels 32 (4 i + g) .. +31 of its own row; else the
// 16 lanes of an entry write its whole row, 64 bytes each.  Chunk c of row
// r sits at c ^ row_swizzle(r).
template <bool kByRow>
__device__ __forceinline__ void store_entry(const EntryFetch& f, TileLds& s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int er = kByRow ? 16 * wave + l16 : 16 * wave + 4 * i + g;
    const int sw = row_swizzle(er);
    uint16_t* dst = s.E + er * kEStride;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint4 v[2];
      dequant16(half ? make_uint2(f.raw[i].z, f.raw[i].w) : make_uint2(f.raw[i].x, f.raw[i].y),
                e4m3_value((f.sc[i] >> (8 * half)) & 0xFFu), v);
      const int c = kByRow ? 4 * (4 * i + g) + 2 * half : 4 * l16 + 2 * half;
      *reinterpret_cast<uint4*>(dst + 8 * (c ^ sw)) = v[0];
      *reinterpret_cast<uint4*>(dst + 8 * ((c + 1) ^ sw)) = v[1];
    }
    if (!kByRow && l16 == 0) s.row_ok[er] = (uint8_t)((f.valid >> i) & 1u);
  }
  if (kByRow && g == 0) s.row_ok[16 * wave + l16] = (uint8_t)f.valid;
}

// A window tile: wave w copies rows 16 w .. +15 of the tile, one row (1 KB,
// 16 bytes per lane) per load.  The loads go through a buffer descriptor, so
// rows past the window read as zeros and all sixteen loads are issued before
// any wait: linear windows use a descriptor from the query's first window
// row to its last; a ring uses the whole ring, token t at row t mod
// swa_ring, and an out-of-range offset for rows past the window.
struct WindowFetch {
  uint4 v[16];
};

__device__ __forceinline__ void fetch_window(const AttnPass& p, const AttnLayer& L, int wtile, int seq, int64_t t0,
                                             int n_win, WindowFetch& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int w0 = wtile * kAttnSplit + 16 * wave;  // window index of the wave's first row
  __amdgpu_buffer_rsrc_t rw;
  int ring = 0, r_first = 0;
  if (p.swa_ring > 0) {
    ring = (int)p.swa_ring;
    rw = __builtin_amdgcn_make_buffer_rsrc((void*)(L.swa + (int64_t)seq * p.swa_stride * kD), 0, ring * kD * 2,
                                           kRawBufferWord3);
    r_first = (int)(t0 % ring);
  } else {
    const int64_t r0 = t0 - p.seq.b[seq];
    rw = __builtin_amdgcn_make_buffer_rsrc((void*)(L.swa + ((int64_t)seq * p.swa_stride + r0) * kD), 0,
                                           n_win * kD * 2, kRawBufferWord3);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int wi = w0 + i;
    int off;
    if (ring > 0) {
      int r = r_first + wi;  // wi < 128 <= ring: one wrap at most
      r = r >= ring ? r - ring : r;
      off = wi < n_win ? r * kD * 2 + 16 * lane : ring * kD * 2;
    } else {
      off = wi * kD * 2 + 16 * lane;
    }
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
    f.v[i] = make_uint4(x[0], x[1], x[2], x[3]);
  }
}

__device__ __forceinline__ void store_window(const WindowFetch& f, int wtile, int n_win, TileLds& s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int sw = row_swizzle(16 * wave + i);
    *reinterpret_cast<uint4*>(s.E + (16 * wave + i) * kEStride + 8 * (lane ^ sw)) = f.v[i];
  }
  if (lane < 16) s.row_ok[16 * wave + lane] = wtile * kAttnSplit + 16 * wave + lane < n_win ? 1 : 0;
}

__device__ __forceinline__ void load_window(const AttnPass& p, const AttnLayer& L, int wtile, int seq, int64_t t0,
                                            int n_win, TileLds& s) {
  WindowFetch f;
  fetch_window(p, L, wtile, seq, t0, n_win, f);
  store_window(f, wtile, n_win, s);
}

// Gather tile `tile` (selected entries first, then window rows) into E.
__device__ __forceinline__ void load_tile(const AttnPass& p, const AttnLayer& L, int tile, int n_tile_idx, int row,
                                          int seq, int64_t t0, int n_win, TileLds& s) {
  if (tile < n_tile_idx) {
    EntryFetch f;
    fetch_entry<false>(p, seq, tile_position(p, tile, row), f);
    store_entry<false>(f, s);
  } else {
    load_window(p, L, tile - n_tile_idx, seq, t0, n_win, s);
  }
}

__device__ __forceinline__ void load_q(const uint16_t* q, int row, uint4 (&qb)[16]) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  const uint16_t* qrow = q + ((int64_t)row * kH + l16) * kD + 8 * g4;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qb[ks] = *reinterpret_cast<const uint4*>(qrow + 32 * ks);
}

// The queries of NL layers for the tile form, loaded once per workgroup:
// thread t reads bytes 16 t + 4 KB i of each layer's 16 KB (whole lines per
// wave instruction), the rows go to E (head h of layer j at row 16 j + h),
// and every wave then reads its MFMA operands from there.  Each wave loading
// its operands from memory would request the query four times over in
// half-line pieces.  Ends with E free again.
template <int NL>
__device__ __forceinline__ void stage_q(const AttnPass& p, int l0, int nl, int row, TileLds& s,
                                        uint4 (&qb)[NL][16]) {
  const int t = threadIdx.x, lane = t & 63, l16 = lane & 15, g4 = lane >> 4;
  uint4 v[NL][4];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    // a layer past the last loads the first layer's query again, unused
    const uint4* src = reinterpret_cast<const uint4*>(p.layer[l0 + (j < nl ? j : 0)].q + (int64_t)row * kH * kD);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[j][i] = src[t + 256 * i];
  }
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    if (j < nl) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = 8 * (t + 256 * i);  // bf16 index within the layer's [16][512]
        *reinterpret_cast<uint4*>(s.E + (16 * j + (o >> 9)) * kEStride + (o & 511)) = v[j][i];
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    if (j < nl) {
      const uint16_t* qrow = s.E + (16 * j + l16) * kEStride + 8 * g4;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qb[j][ks] = *reinterpret_cast<const uint4*>(qrow + 32 * ks);
    }
  }
  __syncthreads();
}

// One tile step for all 16 heads of a (layer, row): S^T = E . Q^T,
// online-softmax update of (m, l) and O = alpha O + P . E.  If `q_next` is
// given, the Q^T operands of the next layer are loaded into `qb` as soon as
// this step's S^T no longer needs them.  Starts with a workgroup barrier.
__device__ __forceinline__ void tile_step(TileLds& s, uint4 (&qb)[16], const uint16_t* q_next, int row, float sc2,
                                          float& m_run, float& l_run, f32x4_t (&o)[8]) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  __syncthreads();  // the tile is in LDS; the previous step's readers of P / red are done
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // row 16 wave + l16: logical chunk 4 ks + g4 at (4 ks + g4) ^ row_swizzle
  const uint16_t* arow = s.E + (16 * wave + l16) * kEStride + 8 * (g4 ^ ((l16 >> 2) & 1));
  const int d3 = (l16 & 8) ? 64 : 0;  // bit 3 of the row: k blocks swapped in pairs of two
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const uint4 a = *reinterpret_cast<const uint4*>(arow + 32 * ks + ((ks & 2) ? -d3 : d3));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qb[ks]), acc, 0, 0, 0);
  }
  if (q_next) load_q(q_next, row, qb);
  float lg[4];
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    lg[r] = s.row_ok[16 * wave + 4 * g4 + r] ? acc[r] * sc2 : -INFINITY;
    mx = fmaxf(mx, lg[r]);
  }
  mx = max_xor32(max_xor16(mx));
  if (g4 == 0) s.red[wave][l16] = mx;
  __syncthreads();
  const float m_tile = fmaxf(fmaxf(s.red[0][l16], s.red[1][l16]), fmaxf(s.red[2][l16], s.red[3][l16]));
  const float m_new = fmaxf(m_run, m_tile);
  const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
  if (wave == 0 && g4 == 0) s.alpha[l16] = alpha;  // read after the barriers below
  float sum = 0.0f;
  float pv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pv[r] = (m_new == -INFINITY) ? 0.0f : exp2f(lg[r] - m_new);
    sum += pv[r];
  }
  store_p4(pv, s.Phi + l16 * kPStride + 16 * wave + 4 * g4, s.Plo + l16 * kPStride + 16 * wave + 4 * g4);
  sum = sum_xor32(sum_xor16(sum));
  __syncthreads();  // red[] (tile maxima) is read by everyone before reuse
  if (g4 == 0) s.red[wave][l16] = sum;
  __syncthreads();
  l_run = l_run * alpha + (s.red[0][l16] + s.red[1][l16] + s.red[2][l16] + s.red[3][l16]);
  m_run = m_new;

  // O = alpha * O + P . E   (rows 4 g4 .. +3 of O are heads 4 g4 .. +3)
  const float4 aa = *reinterpret_cast<const float4*>(&s.alpha[4 * g4]);
  const float arow_alpha[4] = {aa.x, aa.y, aa.z, aa.w};
  const uint4 ahi0 = *reinterpret_cast<const uint4*>(s.Phi + l16 * kPStride + 8 * g4);
  const uint4 ahi1 = *reinterpret_cast<const uint4*>(s.Phi + l16 * kPStride + 32 + 8 * g4);
  const uint4 alo0 = *reinterpret_cast<const uint4*>(s.Plo + l16 * kPStride + 8 * g4);
  const uint4 alo1 = *reinterpret_cast<const uint4*>(s.Plo + l16 * kPStride + 32 + 8 * g4);
  // transposing reads of E: lane (g4, l16) addresses row 8 g4 + l16 / 4 (+4,
  // +32) and 4 channels at 4 (l16 % 4) of each 16-channel block
  const uint16_t* bbase = s.E + (8 * g4 + (l16 >> 2)) * kEStride + 128 * wave + 4 * (l16 & 3);
  const int d8 = (g4 & 1) ? 64 : 0;  // rows with bit 3 set: halves of 256 bytes swapped
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const uint16_t* bp = bbase + 16 * nt + (nt < 4 ? d8 : -d8);
    const int dsw = (l16 & 2) ? -8 : 8;  // rows +4 and +36 hold their chunks swapped in pairs
    const v4i16_t k0 = lds_read_tr16(bp), k1 = lds_read_tr16(bp + 4 * kEStride + dsw);
    const v4i16_t k2 = lds_read_tr16(bp + 32 * kEStride), k3 = lds_read_tr16(bp + 36 * kEStride + dsw);
    const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7));
    const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(k2, k3, 0, 1, 2, 3, 4, 5, 6, 7));
    f32x4_t acc2;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc2[r] = o[nt][r] * arow_alpha[r];
    acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ahi0), b0, acc2, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(alo0), b0, acc2, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ahi1), b1, acc2, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(alo1), b1, acc2, 0, 0, 0);
    o[nt] = acc2;
  }
}

// Partial softmax of one (layer, row) and split: O / l in fp16, m and l.
// Lane (l16, g4) of wave w holds heads 4 g4 .. +3 of channels 128 w + 16 nt
// + l16: 8 bytes per channel.
__device__ __forceinline__ void write_partial(const AttnPass& p, int unit, int split, float m_run, float l_run,
                                              const f32x4_t (&o)[8]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  float* part = p.partial + ((int64_t)unit * p.max_splits + split) * kPartFloats;
  uint16_t* po = reinterpret_cast<uint16_t*>(part);
  float inv[4], down[4], up[4];
  // a partial of one selected-entry tile holds convex combinations of
  // dequantised entries, |value| <= 6 * 448 < 2^15: no scaling to search for
  const bool bounded = p.tiles_per_split == 1 && split < (p.n_idx + kAttnSplit - 1) / kAttnSplit;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float l = __shfl(l_run, 4 * g4 + r, 64);  // l of head 4 g4 + r
    inv[r] = l > 0.0f ? 1.0f / l : 0.0f;
    if (bounded) {
      down[r] = up[r] = 1.0f;
      continue;
    }
    // the largest |O / l| of head 4 g4 + r over this wave's 128 channels
    // (the 16 lanes of g4, 8 each): its float32 exponent field, since the
    // bit patterns of non-negative floats order as integers
    uint32_t mb = 0u;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) mb = max(mb, __float_as_uint(o[nt][r] * inv[r]) & 0x7FFFFFFFu);
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, d, 64));
    // below 2^15 (biased exponent < 142) the values go as they are; else
    // scale by 2^-e so the largest is below 2^15 (exact: a power of two)
    const int e = (int)(mb >> 23) - 141 > 0 ? (int)(mb >> 23) - 141 : 0;
    down[r] = __uint_as_float((uint32_t)(127 - e) << 23);
    up[r] = __uint_as_float((uint32_t)(127 + e) << 23);
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int ch = 128 * wave + 16 * nt + l16;
    const half2_t a = {(_Float16)(o[nt][0] * inv[0] * down[0]), (_Float16)(o[nt][1] * inv[1] * down[1])};
    const half2_t b = {(_Float16)(o[nt][2] * inv[2] * down[2]), (_Float16)(o[nt][3] * inv[3] * down[3])};
    *reinterpret_cast<uint2*>(po + ch * kH + 4 * g4) =
        make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
  }
  if (l16 < 4) part[kPartUp + kH * wave + 4 * g4 + l16] = l16 == 0 ? up[0] : l16 == 1 ? up[1] : l16 == 2 ? up[2] : up[3];
  if (wave == 0 && g4 == 0) {
    part[kPartOWords + l16] = m_run;
    part[kPartOWords + kH + l16] = l_run;
  }
}

__device__ __forceinline__ int64_t window_start(const AttnPass& p, int row, int& n_win) {
  const int seq = row / p.n_q, qi = row - seq * p.n_q;
  const int64_t q_pos = p.seq.a[seq] + qi;
  const int64_t t0 = q_pos - (CSA2_SWA - 1) > 0 ? q_pos - (CSA2_SWA - 1) : 0;
  n_win = (int)(q_pos - t0 + 1);
  return t0;
}

// One window tile of one (layer, row) in a workgroup of its own: its
// partial softmax is split n_tile_idx + wtile of the (layer, row).  The
// window loads go out before the query staging, so both round trips overlap.
__device__ __forceinline__ void window_tile(const AttnPass& p, int row, int layer, int wtile, TileLds& s) {
  const int seq = row / p.n_q;
  int n_win;
  const int64_t t0 = window_start(p, row, n_win);
  const int n_tile_idx = (p.n_idx + kAttnSplit - 1) / kAttnSplit;
  const float sc2 = p.softmax_scale * 1.4426950408889634f;  // logits in the log2 domain
  uint4 qb[1][16];
  WindowFetch wf;
  fetch_window(p, p.layer[layer], wtile, seq, t0, n_win, wf);
  stage_q<1>(p, layer, 1, row, s, qb);
  store_window(wf, wtile, n_win, s);
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t o[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  tile_step(s, qb[0], nullptr, row, sc2, m_run, l_run, o);
  write_partial(p, layer * p.rows + row, n_tile_idx + wtile, m_run, l_run, o);
}

// The pair step (the pair and tile forms of attn.hip, and the decode select
// that attends over its own winners in index.hip): a tile serves two layers
// at once.  Waves 0-1 score
// the first layer (rows 0-31 and 32-63 of a tile), waves 2-3 the second, so
// a wave holds only its own layer's Q^T operands; every wave then updates
// both layers' O for its quarter of the channels.  A selected-entry tile is
// gathered and dequantised once for the two layers; a window tile belongs to
// one layer (the other's waves sit out its scoring).  Against the walk form
// this halves the dequantisation and the tile loads per layer (prefill
// attention of six layers 2.01 -> 1.59 ms).  The P . E products take one
// layer after the other, so one layer's P operands are live at a time and
// the kernel fits 2 waves per SIMD without spills (reading the transposed E
// operands once for both layers spilled and ran no faster).
struct PairLds {
  TileLds t;                       // E, row_ok, P of the first layer, tile maxima per scoring wave
  uint16_t Phi1[kH * kPStride];    // P of the second layer
  uint16_t Plo1[kH * kPStride];
  float red2[4][kH];               // per scoring wave: exponential sums per head
  float alpha2[2][kH];             // the step's rescale factor per (layer, head)
};

// One tile for the layers in `active` (bit j: layer j of the pair): S^T for
// the scoring waves, online-softmax update of both layers' (m, l), and
// O = alpha O + P . E.  Starts with a workgroup barrier.
__device__ __forceinline__ void pair_step(PairLds& s, const uint4 (&qb)[16], int active, float sc2, float (&m_run)[2],
                                          float (&l_run)[2], f32x4_t (&o)[2][8]) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int L = wave >> 1, hb = wave & 1;  // this wave scores layer L, rows 32 hb .. +31
  const bool scorer = (active >> L) & 1;   // (uniform)
  uint16_t* const phi[2] = {s.t.Phi, s.Phi1};
  uint16_t* const plo[2] = {s.t.Plo, s.Plo1};
  __syncthreads();  // the tile is in LDS; the previous step's readers of P / red are done
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  if (scorer) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = 32 * hb + 16 * rb + l16;
      // logical chunk 4 ks + g4 of row r at (4 ks + g4) ^ row_swizzle(r)
      const uint16_t* arow = s.t.E + r * kEStride + 8 * (g4 ^ ((r >> 2) & 1));
      const int d3 = (r & 8) ? 64 : 0;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(arow + 32 * ks + ((ks & 2) ? -d3 : d3));
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qb[ks]), acc[rb], 0, 0, 0);
      }
    }
  }
  // lane (l16, g4) holds head l16 of rows 32 hb + 16 rb + 4 g4 + r
  float lg[2][4];
  float mx = -INFINITY;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int cr = 32 * hb + 16 * rb + 4 * g4 + r;
      lg[rb][r] = scorer && s.t.row_ok[cr] ? acc[rb][r] * sc2 : -INFINITY;
      mx = fmaxf(mx, lg[rb][r]);
    }
  mx = max_xor32(max_xor16(mx));
  if (g4 == 0) s.t.red[wave][l16] = mx;
  __syncthreads();
  float m_new[2], alpha[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float m_tile = (active >> j) & 1 ? fmaxf(s.t.red[2 * j][l16], s.t.red[2 * j + 1][l16]) : -INFINITY;
    m_new[j] = fmaxf(m_run[j], m_tile);
    alpha[j] = m_run[j] == -INFINITY ? 0.0f : exp2f(m_run[j] - m_new[j]);
    if (wave == 0 && g4 == 0) s.alpha2[j][l16] = alpha[j];  // read after the barrier below
  }
  if (scorer) {
    const float mn = L == 0 ? m_new[0] : m_new[1];
    float sum = 0.0f;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = mn == -INFINITY ? 0.0f : exp2f(lg[rb][r] - mn);
        sum += pv[r];
      }
      const int c0 = l16 * kPStride + 32 * hb + 16 * rb + 4 * g4;
      store_p4(pv, (L == 0 ? phi[0] : phi[1]) + c0, (L == 0 ? plo[0] : plo[1]) + c0);
    }
    sum = sum_xor32(sum_xor16(sum));
    if (g4 == 0) s.red2[wave][l16] = sum;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float add = (active >> j) & 1 ? s.red2[2 * j][l16] + s.red2[2 * j + 1][l16] : 0.0f;
    l_run[j] = l_run[j] * alpha[j] + add;
    m_run[j] = m_new[j];
  }
  // O = alpha O + P . E for each active layer (rows 4 g4 .. +3 of O are
  // heads 4 g4 .. +3)
  float arow_alpha[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float4 aa = *reinterpret_cast<const float4*>(&s.alpha2[j][4 * g4]);
    arow_alpha[j][0] = aa.x;
    arow_alpha[j][1] = aa.y;
    arow_alpha[j][2] = aa.z;
    arow_alpha[j][3] = aa.w;
  }
  // transposing reads of E: lane (g4, l16) addresses row 8 g4 + l16 / 4 (+4,
  // +32) and 4 channels at 4 (l16 % 4) of each 16-channel block; one layer
  // after the other, so one layer's P operands are live at a time
  const uint16_t* bbase = s.t.E + (8 * g4 + (l16 >> 2)) * kEStride + 128 * wave + 4 * (l16 & 3);
  const int d8 = (g4 & 1) ? 64 : 0;  // rows with bit 3 set: halves of 256 bytes swapped
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (!((active >> j) & 1)) continue;  // (uniform)
    const uint16_t* pj = j == 0 ? s.t.Phi : s.Phi1;
    const uint16_t* qj = j == 0 ? s.t.Plo : s.Plo1;
    const uint4 ph0 = *reinterpret_cast<const uint4*>(pj + l16 * kPStride + 8 * g4);
    const uint4 ph1 = *reinterpret_cast<const uint4*>(pj + l16 * kPStride + 32 + 8 * g4);
    const uint4 pl0 = *reinterpret_cast<const uint4*>(qj + l16 * kPStride + 8 * g4);
    const uint4 pl1 = *reinterpret_cast<const uint4*>(qj + l16 * kPStride + 32 + 8 * g4);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const uint16_t* bp = bbase + 16 * nt + (nt < 4 ? d8 : -d8);
      const int dsw = (l16 & 2) ? -8 : 8;  // rows +4 and +36 hold their chunks swapped in pairs
      const v4i16_t k0 = lds_read_tr16(bp), k1 = lds_read_tr16(bp + 4 * kEStride + dsw);
      const v4i16_t k2 = lds_read_tr16(bp + 32 * kEStride), k3 = lds_read_tr16(bp + 36 * kEStride + dsw);
      const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7));
      const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(k2, k3, 0, 1, 2, 3, 4, 5, 6, 7));
      f32x4_t acc2;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc2[r] = o[j][nt][r] * arow_alpha[j][r];
      acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ph0), b0, acc2, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pl0), b0, acc2, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ph1), b1, acc2, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pl1), b1, acc2, 0, 0, 0);
      o[j][nt] = acc2;
    }
  }
}

// The queries of the pair, staged through E: layer j at rows 16 j .. +15
// (thread t reads bytes 16 t + 4 KB i of each layer's 16 KB, whole lines per
// wave instruction); each wave then reads the Q^T operands of the layer it
// scores.  Ends with E free again.
__device__ __forceinline__ void stage_q_pair(const AttnPass& p, int l0, int nl, int row, PairLds& s, uint4 (&qb)[16]) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l16 = lane & 15, g4 = lane >> 4;
  uint4 v[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    // a layer past the last loads the first layer's query again, unused
    const uint4* src = reinterpret_cast<const uint4*>(p.layer[l0 + (j < nl ? j : 0)].q + (int64_t)row * kH * kD);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[j][i] = src[t + 256 * i];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = 8 * (t + 256 * i);  // bf16 index within the layer's [16][512]
      *reinterpret_cast<uint4*>(s.t.E + (16 * j + (o >> 9)) * kEStride + (o & 511)) = v[j][i];
    }
  __syncthreads();
  const uint16_t* qrow = s.t.E + (16 * (wave >> 1) + l16) * kEStride + 8 * g4;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qb[ks] = *reinterpret_cast<const uint4*>(qrow + 32 * ks);
  __syncthreads();
}

}  // namespace csa2
