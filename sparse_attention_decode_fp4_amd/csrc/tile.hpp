// Tile pieces of the sparse + SWA attention shared by the attention kernels
// (attn.hip) and the decode select, whose launch also runs the window tiles
// of a group (index.hip): the LDS tile, entry and window loads, the staged
// queries, one online-softmax tile step and the partial write.
#pragma once

#include "kernels.hpp"

namespace csa2 {

// bf16 per row of E: rows 8 banks apart, so the transposing reads (4 rows x
// 32 bytes per cycle) do not conflict.  Consecutive lanes write consecutive
// rows, and in rows whose bit 2 is set the 16-byte chunks are swapped in
// pairs (chunk c at c ^ 1), so rows r and r + 4 of the 16-byte MFMA operand
// reads and writes fall in different banks.
constexpr int kEStride = kD + 16;
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

__device__ __forceinline__ uint32_t bf16_round(float x) {  // round to nearest even, bf16 bits
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  // exact values only: truncation equals rounding
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

struct TileLds {
  uint16_t E[kAttnSplit * kEStride];  // [row][channel]
  uint16_t Phi[kH * kPStride];
  uint16_t Plo[kH * kPStride];
  float red[4][kH];
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

// A selected-entry tile in flight, read with consecutive lanes on
// consecutive bytes: in load step i (0..3) wave w takes entries
// 16 w + 4 i + lane / 16, lane % 16 reading 16 bytes of codes (channels
// 32 (lane % 16) .. +31, two scale groups) and those groups' two scales.  A
// wave instruction thus covers four whole entries; a lane per entry, 16
// bytes each, would touch 64 lines per instruction and take several times
// as long to load the same tile.
struct EntryFetch {
  uint4 raw[4];
  uint32_t sc[4];  // the two E4M3 scales of step i in bits 0..15
  uint32_t valid;  // bit i: the entry of step i is present
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
__device__ __forceinline__ void fetch_entry(const AttnPass& p, int seq, int32_t pos_lane, EntryFetch& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15;
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
  f.valid = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int src = 16 * wave + 4 * i + (lane >> 4);
    const int32_t pos = __shfl(pos_lane, src, 64);
    const uint32_t e = (uint32_t)__shfl((int)e_lane, src, 64);
    f.valid |= (pos >= 0 ? 1u : 0u) << i;
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rn, (int)(e * CSA2_NIB_BYTES) + 16 * l16, 0, 0);
    f.raw[i] = make_uint4(v[0], v[1], v[2], v[3]);
    f.sc[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(e * CSA2_SCALE_BYTES) + 2 * l16, 0, 0);
  }
}

// Dequantise a fetched tile into E (zeros for empty slots): each lane
// writes 64 bytes of one row, the 16 lanes of an entry its whole row.
__device__ __forceinline__ void store_entry(const EntryFetch& f, TileLds& s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int er = 16 * wave + 4 * i + (lane >> 4);
    const int sw = i & 1;  // bit 2 of er: chunk c of the row sits at c ^ sw
    uint16_t* dst = s.E + er * kEStride;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint4 v[2];
      dequant16(half ? make_uint2(f.raw[i].z, f.raw[i].w) : make_uint2(f.raw[i].x, f.raw[i].y),
                e4m3_value((f.sc[i] >> (8 * half)) & 0xFFu), v);
      const int c = 4 * l16 + 2 * half;
      *reinterpret_cast<uint4*>(dst + 8 * (c ^ sw)) = v[0];
      *reinterpret_cast<uint4*>(dst + 8 * ((c + 1) ^ sw)) = v[1];
    }
    if (l16 == 0) s.row_ok[er] = (uint8_t)((f.valid >> i) & 1u);
  }
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
    const int sw = (i >> 2) & 1;  // bit 2 of row 16 wave + i
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
    fetch_entry(p, seq, tile_position(p, tile, row), f);
    store_entry(f, s);
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
  const uint16_t* arow = s.E + (16 * wave + l16) * kEStride + 8 * (g4 ^ ((l16 >> 2) & 1));
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const uint4 a = *reinterpret_cast<const uint4*>(arow + 32 * ks);
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
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (g4 == 0) s.red[wave][l16] = mx;
  __syncthreads();
  const float m_tile = fmaxf(fmaxf(s.red[0][l16], s.red[1][l16]), fmaxf(s.red[2][l16], s.red[3][l16]));
  const float m_new = fmaxf(m_run, m_tile);
  const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
  float sum = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int cr = 16 * wave + 4 * g4 + r;
    const float pv = (m_new == -INFINITY) ? 0.0f : exp2f(lg[r] - m_new);
    sum += pv;
    const uint32_t hi = bf16_round(pv);
    s.Phi[l16 * kPStride + cr] = (uint16_t)hi;
    s.Plo[l16 * kPStride + cr] = (uint16_t)bf16_round(pv - __uint_as_float(hi << 16));
  }
  sum += __shfl_xor(sum, 16, 64);
  sum += __shfl_xor(sum, 32, 64);
  __syncthreads();  // red[] (tile maxima) is read by everyone before reuse
  if (g4 == 0) s.red[wave][l16] = sum;
  __syncthreads();
  l_run = l_run * alpha + (s.red[0][l16] + s.red[1][l16] + s.red[2][l16] + s.red[3][l16]);
  m_run = m_new;

  // O = alpha * O + P . E   (the rescale factor of row 4*g4+r lives in lane 4*g4+r)
  float arow_alpha[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) arow_alpha[r] = __shfl(alpha, 4 * g4 + r, 64);
  const uint4 ahi0 = *reinterpret_cast<const uint4*>(s.Phi + l16 * kPStride + 8 * g4);
  const uint4 ahi1 = *reinterpret_cast<const uint4*>(s.Phi + l16 * kPStride + 32 + 8 * g4);
  const uint4 alo0 = *reinterpret_cast<const uint4*>(s.Plo + l16 * kPStride + 8 * g4);
  const uint4 alo1 = *reinterpret_cast<const uint4*>(s.Plo + l16 * kPStride + 32 + 8 * g4);
  // transposing reads of E: lane (g4, l16) addresses row 8 g4 + l16 / 4 (+4,
  // +32) and 4 channels at 4 (l16 % 4) of each 16-channel block
  const uint16_t* bbase = s.E + (8 * g4 + (l16 >> 2)) * kEStride + 128 * wave + 4 * (l16 & 3);
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const uint16_t* bp = bbase + 16 * nt;
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
  float inv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float l = __shfl(l_run, 4 * g4 + r, 64);  // l of head 4 g4 + r
    inv[r] = l > 0.0f ? 1.0f / l : 0.0f;
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int ch = 128 * wave + 16 * nt + l16;
    const half2_t a = {(_Float16)(o[nt][0] * inv[0]), (_Float16)(o[nt][1] * inv[1])};  // round to nearest
    const half2_t b = {(_Float16)(o[nt][2] * inv[2]), (_Float16)(o[nt][3] * inv[3])};
    *reinterpret_cast<uint2*>(po + ch * kH + 4 * g4) =
        make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
  }
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

}  // namespace csa2
