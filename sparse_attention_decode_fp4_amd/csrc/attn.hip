// Sparse + sliding-window attention of the CSA2 step.
//
// Readings (the pages give no formula): the FP4 latent of an entry serves as
// both key and value; a query at token p attends, in one softmax, over the
// selected entries and the bf16 window rows of tokens max(0, p-127)..p
// (ai-wave.ru "DeepSeek V4.1-Flash: 1M context, FP4 KV cache ...", second
// paragraph: a 128-token window in every layer).
//
// The 16 heads share every gathered row, so a workgroup runs two real dense
// contractions per tile of 64 candidate rows on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16) with float32 accumulation:
//   S^T[64 rows][16 heads] = E[64][512] . Q^T      (wave w: rows 16w..16w+15)
//   O[16][512] += P[16][64] . E[64][512]            (wave w: channels 128w..)
// The tile sits in LDS row-major (E).  The first product contracts over
// channels and reads its E operand with 16-byte loads; the second contracts
// over rows and reads its E operand with the transposing LDS load of gfx950
// (ds_read_b64_tr_b16), two per MFMA.  E2M1 x E4M3 products are exact in bf16,
// so only P is rounded: it is split into bf16 hi + lo parts (relative error
// ~2^-16).  Two forms:
//   walk   a workgroup walks `tiles_per_split` tiles of one row for a group
//          of LG layers, one online softmax per layer, a selected-entry tile
//          dequantised once for the group (many rows: prefill chunks);
//   tiles  one tile per workgroup (few rows: decode); the tiles of selected
//          entries are shared by all layers of the launch, since the layers
//          of a group attend over the same entries, so each is gathered and
//          dequantised once and then serves every layer.
// When a (layer, row) is split over several workgroups, a second kernel
// merges the partial softmaxes in split order, so results do not depend on
// scheduling.
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
// descriptor at the sequence start: an empty slot uses the entry index
// CSA2_MAX_ENTRIES, whose offsets reach the descriptors' ranges, so the
// hardware returns zeros without touching memory.  No load waits on another.
__device__ __forceinline__ void fetch_entry(const AttnPass& p, int seq, int32_t pos_lane, EntryFetch& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15;
  const int64_t s0 = (int64_t)seq * p.kv_stride;
  const __amdgpu_buffer_rsrc_t rn = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.nib + s0 * CSA2_NIB_BYTES), 0, CSA2_MAX_ENTRIES * CSA2_NIB_BYTES, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.scale + s0 * CSA2_SCALE_BYTES), 0, CSA2_MAX_ENTRIES * CSA2_SCALE_BYTES, kRawBufferWord3);
  f.valid = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t pos = __shfl(pos_lane, 16 * wave + 4 * i + (lane >> 4), 64);
    const uint32_t e = pos >= 0 ? (uint32_t)pos : (uint32_t)CSA2_MAX_ENTRIES;
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

// Tile-parallel form (one tile per workgroup, partials merged afterwards):
// workgroup (row, j).  j < n_tile_idx * n_groups: selected-entry tile
// j / n_groups for layer group j % n_groups (layers LG g .. LG g + LG - 1):
// the layers of a group attend over the same entries, so a tile is gathered
// and dequantised once per layer group and then used by each of its layers
// in turn (the layer loop is unrolled, so waiting for the next layer's Q
// does not wait for this layer's partial stores); otherwise a window tile
// of one layer.
template <int LG>
__global__ __launch_bounds__(256) void k_attention_tiles(AttnPass p) {
  const int n_tile_idx = (p.n_idx + kAttnSplit - 1) / kAttnSplit;
  const int n_win_tiles = p.n_tiles - n_tile_idx;
  const int n_groups = (p.n_layers + LG - 1) / LG;
  const int n_sel = n_tile_idx * n_groups;
  const int per_row = n_sel + p.n_layers * n_win_tiles;
  // workgroup ids are dealt round-robin over the 8 XCDs: with 8 or more rows,
  // all workgroups of a row run on one XCD, which then reads the row's
  // queries from memory once
  int row, j;
  if (p.rows >= kXcds) {
    const int xcd = blockIdx.x & (kXcds - 1), w = blockIdx.x >> 3;
    row = xcd + kXcds * (w / per_row);
    j = w % per_row;
  } else {
    row = blockIdx.x / per_row;
    j = blockIdx.x - row * per_row;
  }
  if (row >= p.rows) return;
  const int seq = row / p.n_q;
  int n_win;
  const int64_t t0 = window_start(p, row, n_win);
  __shared__ __attribute__((aligned(16))) TileLds s;
  const float sc2 = p.softmax_scale * 1.4426950408889634f;  // logits in the log2 domain
  float m_run, l_run;
  f32x4_t o[8];
  auto reset = [&]() {
    m_run = -INFINITY;
    l_run = 0.0f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  if (j < n_sel) {
    const int tile = j / n_groups, l0 = LG * (j % n_groups);
    const int nl = p.n_layers - l0 < LG ? p.n_layers - l0 : LG;
    // the positions and the queries go out together; the entries follow as
    // soon as the positions are in
    const int32_t pos = tile_position(p, tile, row);
    uint4 qb[LG][16];
    EntryFetch f;
    fetch_entry(p, seq, pos, f);
    stage_q<LG>(p, l0, nl, row, s, qb);
    store_entry(f, s);
#pragma unroll
    for (int i = 0; i < LG; ++i) {
      const int l = l0 + i;
      if (i >= nl) break;  // uniform
      reset();
      tile_step(s, qb[i], nullptr, row, sc2, m_run, l_run, o);
      write_partial(p, l * p.rows + row, tile, m_run, l_run, o);
    }
  } else {
    const int jj = j - n_sel, layer = jj / n_win_tiles, tile = n_tile_idx + jj % n_win_tiles;
    uint4 qb[1][16];
    WindowFetch wf;
    fetch_window(p, p.layer[layer], tile - n_tile_idx, seq, t0, n_win, wf);
    stage_q<1>(p, layer, 1, row, s, qb);
    store_window(wf, tile - n_tile_idx, n_win, s);
    reset();
    tile_step(s, qb[0], nullptr, row, sc2, m_run, l_run, o);
    write_partial(p, layer * p.rows + row, tile, m_run, l_run, o);
  }
}

// Walk form: workgroup (group of LG layers, row, split) walks its tiles
// with one online softmax per layer.  The selected-entry tiles are shared by
// the layers (dequantised once per tile for the group), window tiles are
// per layer.  Selected-entry tiles are software-pipelined: the entries of
// tile i + 1 and the positions of tile i + 2 are in flight while tile i is
// computed.
template <int LG>
__global__ __launch_bounds__(256, 2) void k_attention(AttnPass p) {
  const int n_groups = (p.n_layers + LG - 1) / LG;
  const int units = n_groups * p.rows;
  int unit, split;
  {
    const int lin = blockIdx.x;
    if (units >= kXcds && p.max_splits > 1) {  // the splits of a unit share one XCD
      const int xcd = lin & (kXcds - 1), w = lin >> 3;
      unit = xcd + kXcds * (w / p.max_splits);
      split = w % p.max_splits;
    } else if (units >= kXcds) {
      // one workgroup per unit: each XCD takes a contiguous range of units,
      // so the queries resident on it together are consecutive tokens whose
      // windows overlap in all but one row, and the rows come from its L2
      const int xcd = lin & (kXcds - 1), w = lin >> 3;
      unit = xcd * ((units + kXcds - 1) / kXcds) + w;
      split = 0;
    } else {
      unit = lin / p.max_splits;
      split = lin % p.max_splits;
    }
  }
  if (unit >= units) return;
  const int grp = unit / p.rows, row = unit - grp * p.rows;
  const int l0 = LG * grp;
  const int nl = p.n_layers - l0 < LG ? p.n_layers - l0 : LG;
  const int seq = row / p.n_q;
  int n_win;
  const int64_t t0 = window_start(p, row, n_win);
  const int n_tile_idx = (p.n_idx + kAttnSplit - 1) / kAttnSplit;
  const int tile_begin = split * p.tiles_per_split;
  int tile_end = tile_begin + p.tiles_per_split;
  tile_end = tile_end < p.n_tiles ? tile_end : p.n_tiles;

  __shared__ __attribute__((aligned(16))) TileLds s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const float sc2 = p.softmax_scale * 1.4426950408889634f;  // logits in the log2 domain
  uint4 qb[LG][16];
  float m_run[LG], l_run[LG];  // per head l16 (replicated)
  f32x4_t o[LG][8];            // O[4*g4+r][128*wave + 16*nt + l16]
#pragma unroll
  for (int i = 0; i < LG; ++i) {
    if (i < nl) load_q(p.layer[l0 + i].q, row, qb[i]);
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[i][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int last_sel = (tile_end < n_tile_idx ? tile_end : n_tile_idx) - 1;  // last selected-entry tile here
  EntryFetch f;
  int32_t pos_next = -1;
  if (tile_begin <= last_sel) {
    fetch_entry(p, seq, tile_position(p, tile_begin, row), f);
    if (tile_begin + 1 <= last_sel) pos_next = tile_position(p, tile_begin + 1, row);
  }
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    if (tile > tile_begin) __syncthreads();  // the previous tile's readers of E are done
    if (tile <= last_sel) {
      store_entry(f, s);
      if (tile + 1 <= last_sel) {
        fetch_entry(p, seq, pos_next, f);
        if (tile + 2 <= last_sel) pos_next = tile_position(p, tile + 2, row);
      }
#pragma unroll
      for (int i = 0; i < LG; ++i)
        if (i < nl) tile_step(s, qb[i], nullptr, row, sc2, m_run[i], l_run[i], o[i]);
    } else {
#pragma unroll
      for (int i = 0; i < LG; ++i) {
        if (i >= nl) break;
        if (i > 0) __syncthreads();  // the previous layer's readers of E are done
        load_window(p, p.layer[l0 + i], tile - n_tile_idx, seq, t0, n_win, s);
        tile_step(s, qb[i], nullptr, row, sc2, m_run[i], l_run[i], o[i]);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < LG; ++i) {
    if (i >= nl) break;
    if (p.max_splits == 1) {  // whole row in this workgroup: write the output
      float l_out[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) l_out[r] = __shfl(l_run[i], 4 * g4 + r, 64);
      float* out = p.layer[l0 + i].out;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int ch = 128 * wave + 16 * nt + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float inv = l_out[r] > 0.0f ? 1.0f / l_out[r] : 0.0f;
          out[((int64_t)row * kH + 4 * g4 + r) * kD + ch] = o[i][nt][r] * inv;
        }
      }
    } else {
      write_partial(p, (l0 + i) * p.rows + row, split, m_run[i], l_run[i], o[i]);
    }
  }
}

// Merge of the split partial softmaxes, in split order.  A kernel of its
// own: the kernel boundary orders the partial writes before these reads on
// every XCD, which in-kernel device-scope fences would do by writing back
// the whole L2.  Workgroup (unit, channel quarter): thread t sums channel
// 128 quarter + t / 2, heads 8 (t % 2) .. +8 (16 contiguous bytes of each
// partial), with per-head weights l_s exp2(m_s - M) / L that 16 threads work
// out in LDS from the (m, l) of every split, loaded in one round trip while
// the partial loads of up to 16 splits are in flight.
constexpr int kMaxMergeSplits = 64;
constexpr int kMergeBatch = 16;
__global__ __launch_bounds__(256) void k_attention_merge(AttnPass p) {
  const int unit = blockIdx.x >> 2, quarter = blockIdx.x & 3;
  const int layer = unit / p.rows, row = unit - layer * p.rows;
  const int t = threadIdx.x;
  const int ch = 128 * quarter + (t >> 1), h0 = 8 * (t & 1);
  const int ns = p.max_splits;
  const float* pb = p.partial + (int64_t)unit * ns * kPartFloats;
  __shared__ float wgt[kMaxMergeSplits][kH];
  __shared__ float lsh[kMaxMergeSplits][kH];
  float acc[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) acc[h] = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += kMergeBatch) {
    uint4 v[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int s = s0 + u < ns ? s0 + u : ns - 1;
      const uint16_t* ps = reinterpret_cast<const uint16_t*>(pb + (int64_t)s * kPartFloats) + ch * kH + h0;
      v[u] = *reinterpret_cast<const uint4*>(ps);
    }
    if (s0 == 0) {
      for (int i = t; i < ns * kH; i += 256) {  // (split, head) = (i / 16, i % 16)
        const float* ps = pb + (int64_t)(i / kH) * kPartFloats + kPartOWords;
        wgt[i / kH][i % kH] = ps[i % kH];
        lsh[i / kH][i % kH] = ps[kH + i % kH];
      }
      __syncthreads();
      if (t < kH) {  // head t
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, wgt[s][t]);
        float L = 0.0f;
        for (int s = 0; s < ns; ++s) {
          const float m = wgt[s][t];
          const float w = m == -INFINITY ? 0.0f : exp2f(m - M) * lsh[s][t];
          wgt[s][t] = w;
          L += w;
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        for (int s = 0; s < ns; ++s) wgt[s][t] *= inv;
      }
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      if (s0 + u >= ns) break;
      const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const half2_t pr = __builtin_bit_cast(half2_t, wd[h >> 1]);
        acc[h] += wgt[s0 + u][h0 + h] * (float)pr[h & 1];
      }
    }
  }
  float* dst = p.layer[layer].out + ((int64_t)row * kH + h0) * kD + ch;
#pragma unroll
  for (int h = 0; h < 8; ++h) dst[h * kD] = acc[h];
}

hipError_t launch_attention(const AttnPass& p, hipStream_t stream) {
  const int units = p.n_layers * p.rows;
  if (units == 0) return hipSuccess;
  // walk form: one layer per workgroup (a pair of layers needs about 320
  // registers, and the single wave per SIMD that leaves costs more than the
  // shared dequantisation saves)
  constexpr int kWalkLG = 1;
  const int wunits = (p.n_layers + kWalkLG - 1) / kWalkLG * p.rows;
  const int gu = wunits >= kXcds ? (wunits + kXcds - 1) / kXcds * kXcds : wunits;
  int h = prof_begin(CSA2_K_ATTENTION, stream);
  const int n_tile_idx = (p.n_idx + kAttnSplit - 1) / kAttnSplit;
  if (p.tiles_per_split == 1 && p.max_splits == p.n_tiles) {
    // one tile per workgroup: selected-entry tiles are shared by the layers
    // layer groups of two: gathering a tile twice is cheap next to running
    // four layers one after another in one workgroup
    constexpr int LG = 2;
    const int n_groups = (p.n_layers + LG - 1) / LG;
    const int per_row = n_tile_idx * n_groups + p.n_layers * (p.n_tiles - n_tile_idx);
    const int grows = p.rows >= kXcds ? (p.rows + kXcds - 1) / kXcds * kXcds : p.rows;
    hipLaunchKernelGGL(k_attention_tiles<LG>, dim3((unsigned)(grows * per_row)), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(k_attention<kWalkLG>, dim3((unsigned)(gu * p.max_splits)), dim3(256), 0, stream, p);
  }
  prof_end(h, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_splits == 1) return e;
  if (p.max_splits > kMaxMergeSplits) return hipErrorInvalidValue;
  h = prof_begin(CSA2_K_ATTENTION_MERGE, stream);
  hipLaunchKernelGGL(k_attention_merge, dim3((unsigned)(4 * units)), dim3(256), 0, stream, p);
  prof_end(h, stream);
  return hipGetLastError();
}

}  // namespace csa2
