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
// E2M1 x E4M3 products are exact in bf16, so only P is rounded: it is split
// into bf16 hi + lo parts (relative error ~2^-16).  A workgroup walks
// `tiles_per_split` tiles with an online softmax.  When a (layer, row) is
// split over several workgroups, a second kernel merges the partial
// softmaxes in split order, so results do not depend on scheduling.
#include "kernels.hpp"

namespace csa2 {

constexpr int kEStride = kD + 8;     // bf16 elements per LDS row (padding against bank conflicts)
constexpr int kPStride = kAttnSplit + 8;
constexpr int kPartStride = kD + 4;  // floats per head in a partial: O[512], m, l, 2 pad

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  // exact values only: truncation equals rounding
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t bf16_round(float x) {  // round to nearest even, bf16 bits
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Gather one tile of 64 candidate rows into LDS as bf16 (thread: row t/4,
// quarter t%4 = 128 channels).  Returns whether this thread's row is real.
__device__ __forceinline__ bool load_tile(const AttnPass& p, const AttnLayer& L, int tile,
                                          int n_tile_idx, int row, int seq, int64_t t0, int n_win,
                                          uint16_t* E) {
  const int t = threadIdx.x, er = t >> 2, quarter = t & 3;
  uint16_t* dst = E + er * kEStride + quarter * 128;
  bool valid;
  if (tile < n_tile_idx) {
    const int c = tile * kAttnSplit + er;
    const int32_t pos = c < p.n_idx ? p.idx[(int64_t)row * p.n_idx + c] : -1;
    valid = pos >= 0;
    if (valid) {
      const int64_t ent = (int64_t)seq * p.kv_stride + pos;
      const uint8_t* nb = p.nib + ent * CSA2_NIB_BYTES + quarter * 64;
      const uint8_t* sb = p.scale + ent * CSA2_SCALE_BYTES + quarter * 8;
      uint4 raw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] = *reinterpret_cast<const uint4*>(nb + 16 * i);
      const uint2 sc = *reinterpret_cast<const uint2*>(sb);
      const uint32_t scw[2] = {sc.x, sc.y};
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // 16 bytes = 32 channels = 2 scale groups
        const uint32_t wds[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int g = 2 * i + half;  // scale group within this quarter
          const float s = e4m3_value((scw[g >> 2] >> (8 * (g & 3))) & 0xFFu);
          uint32_t outw[8];
#pragma unroll
          for (int wd = 0; wd < 2; ++wd) {
            const uint32_t word = wds[2 * half + wd];
            // byte b -> (low nibble, high nibble) = consecutive channels; scale 1: exact
            const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
            const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
            const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
            const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
            outw[4 * wd + 0] = pack_bf16(v0.x * s, v0.y * s);
            outw[4 * wd + 1] = pack_bf16(v1.x * s, v1.y * s);
            outw[4 * wd + 2] = pack_bf16(v2.x * s, v2.y * s);
            outw[4 * wd + 3] = pack_bf16(v3.x * s, v3.y * s);
          }
          *reinterpret_cast<uint4*>(dst + 32 * i + 16 * half) =
              make_uint4(outw[0], outw[1], outw[2], outw[3]);
          *reinterpret_cast<uint4*>(dst + 32 * i + 16 * half + 8) =
              make_uint4(outw[4], outw[5], outw[6], outw[7]);
        }
      }
    }
  } else {
    const int wi = (tile - n_tile_idx) * kAttnSplit + er;
    valid = wi < n_win;
    if (valid) {
      const int64_t r = t0 + wi - p.seq.b[seq];
      const uint16_t* src = L.swa + ((int64_t)seq * p.swa_stride + r) * kD + quarter * 128;
      uint4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const uint4*>(src + 8 * i);
#pragma unroll
      for (int i = 0; i < 16; ++i) *reinterpret_cast<uint4*>(dst + 8 * i) = v[i];
    }
  }
  if (!valid) {
#pragma unroll
    for (int i = 0; i < 16; ++i) *reinterpret_cast<uint4*>(dst + 8 * i) = make_uint4(0, 0, 0, 0);
  }
  return valid;
}

__global__ __launch_bounds__(256) void k_attention(AttnPass p) {
  const int units = p.n_layers * p.rows;
  int unit, split;
  {
    const int lin = blockIdx.x;
    if (units >= kXcds && p.max_splits > 1) {  // the splits of a unit share one XCD
      const int xcd = lin & (kXcds - 1), w = lin >> 3;
      unit = xcd + kXcds * (w / p.max_splits);
      split = w % p.max_splits;
    } else {
      unit = lin / p.max_splits;
      split = lin % p.max_splits;
    }
  }
  if (unit >= units) return;
  const int layer = unit / p.rows, row = unit - layer * p.rows;
  const int seq = row / p.n_q, qi = row - seq * p.n_q;
  const AttnLayer& L = p.layer[layer];
  const int64_t q_pos = p.seq.a[seq] + qi;
  const int64_t t0 = q_pos - (CSA2_SWA - 1) > 0 ? q_pos - (CSA2_SWA - 1) : 0;
  const int n_win = (int)(q_pos - t0 + 1);
  const int n_tile_idx = (p.n_idx + kAttnSplit - 1) / kAttnSplit;
  const int tile_begin = split * p.tiles_per_split;
  int tile_end = tile_begin + p.tiles_per_split;
  tile_end = tile_end < p.n_tiles ? tile_end : p.n_tiles;

  __shared__ __attribute__((aligned(16))) uint16_t E[kAttnSplit * kEStride];
  __shared__ __attribute__((aligned(16))) uint16_t Phi[kH * kPStride];
  __shared__ __attribute__((aligned(16))) uint16_t Plo[kH * kPStride];
  __shared__ float red[4][kH];
  __shared__ uint8_t row_ok[kAttnSplit];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;

  // Q^T operands of all 16 k-steps: head l16, channels 32*ks + 8*g4 .. +8
  const uint16_t* qrow = L.q + ((int64_t)row * kH + l16) * kD + 8 * g4;
  uint4 qb[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qb[ks] = *reinterpret_cast<const uint4*>(qrow + 32 * ks);

  const float sc2 = p.softmax_scale * 1.4426950408889634f;  // logits in the log2 domain
  float m_run = -INFINITY, l_run = 0.0f;                     // per head l16 (replicated)
  f32x4_t o[8];                                              // O[4*g4+r][128*wave + 16*nt + l16]
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int tile = tile_begin; tile < tile_end; ++tile) {
    __syncthreads();  // the previous tile's readers of E / P are done
    const bool valid = load_tile(p, L, tile, n_tile_idx, row, seq, t0, n_win, E);
    if ((t & 3) == 0) row_ok[t >> 2] = valid ? 1 : 0;
    __syncthreads();

    // S^T tile of this wave: candidate rows 16*wave .. +16, all 16 heads
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* arow = E + (16 * wave + l16) * kEStride + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const uint4 a = *reinterpret_cast<const uint4*>(arow + 32 * ks);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qb[ks]), acc, 0, 0, 0);
    }
    float lg[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lg[r] = row_ok[16 * wave + 4 * g4 + r] ? acc[r] * sc2 : -INFINITY;
      mx = fmaxf(mx, lg[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (g4 == 0) red[wave][l16] = mx;
    __syncthreads();
    const float m_tile = fmaxf(fmaxf(red[0][l16], red[1][l16]), fmaxf(red[2][l16], red[3][l16]));
    const float m_new = fmaxf(m_run, m_tile);
    const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int cr = 16 * wave + 4 * g4 + r;
      const float pv = (m_new == -INFINITY) ? 0.0f : exp2f(lg[r] - m_new);
      sum += pv;
      const uint32_t hi = bf16_round(pv);
      Phi[l16 * kPStride + cr] = (uint16_t)hi;
      Plo[l16 * kPStride + cr] = (uint16_t)bf16_round(pv - __uint_as_float(hi << 16));
    }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    __syncthreads();  // red[] (tile maxima) is read by everyone before reuse
    if (g4 == 0) red[wave][l16] = sum;
    __syncthreads();
    l_run = l_run * alpha + (red[0][l16] + red[1][l16] + red[2][l16] + red[3][l16]);
    m_run = m_new;

    // O = alpha * O + P . E   (the rescale factor of row 4*g4+r lives in lane 4*g4+r)
    float arow_alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) arow_alpha[r] = __shfl(alpha, 4 * g4 + r, 64);
    const uint4 ahi0 = *reinterpret_cast<const uint4*>(Phi + l16 * kPStride + 8 * g4);
    const uint4 ahi1 = *reinterpret_cast<const uint4*>(Phi + l16 * kPStride + 32 + 8 * g4);
    const uint4 alo0 = *reinterpret_cast<const uint4*>(Plo + l16 * kPStride + 8 * g4);
    const uint4 alo1 = *reinterpret_cast<const uint4*>(Plo + l16 * kPStride + 32 + 8 * g4);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int ch = 128 * wave + 16 * nt + l16;
      f32x4_t acc2;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc2[r] = o[nt][r] * arow_alpha[r];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint16_t* col = E + (32 * kk + 8 * g4) * kEStride + ch;
        uint32_t bw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bw[j] = (uint32_t)col[(2 * j) * kEStride] | ((uint32_t)col[(2 * j + 1) * kEStride] << 16);
        const bf16x8_t b = as_bf16x8(make_uint4(bw[0], bw[1], bw[2], bw[3]));
        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk ? ahi1 : ahi0), b, acc2, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk ? alo1 : alo0), b, acc2, 0, 0, 0);
      }
      o[nt] = acc2;
    }
  }

  // final normaliser of the head held in each output row 4*g4+r
  float m_out[4], l_out[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_out[r] = __shfl(m_run, 4 * g4 + r, 64);
    l_out[r] = __shfl(l_run, 4 * g4 + r, 64);
  }

  if (p.max_splits == 1) {  // whole row in this workgroup: write the output
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int ch = 128 * wave + 16 * nt + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float inv = l_out[r] > 0.0f ? 1.0f / l_out[r] : 0.0f;
        L.out[((int64_t)row * kH + 4 * g4 + r) * kD + ch] = o[nt][r] * inv;
      }
    }
    return;
  }

  float* part = p.partial + (((int64_t)unit * p.max_splits + split) * kH) * kPartStride;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int ch = 128 * wave + 16 * nt + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) part[(4 * g4 + r) * kPartStride + ch] = o[nt][r];
  }
  if (wave == 0 && g4 == 0) {
    part[l16 * kPartStride + kD] = m_run;
    part[l16 * kPartStride + kD + 1] = l_run;
  }
}

// Merge of the split partial softmaxes, in split order.  A kernel of its own:
// the kernel boundary orders the partial writes before these reads on every
// XCD, which in-kernel device-scope fences would do by writing back the whole
// L2.  Workgroup (unit, quarter): 4 heads x 512 channels, 16 per thread.
__global__ __launch_bounds__(128) void k_attention_merge(AttnPass p) {
  const int unit = blockIdx.x >> 2, quarter = blockIdx.x & 3;
  const int layer = unit / p.rows, row = unit - layer * p.rows;
  const int t = threadIdx.x;
  const int h = 4 * quarter + (t >> 5), c0 = (t & 31) * 16;
  const float* pb = p.partial + ((int64_t)unit * p.max_splits * kH) * kPartStride;
  float M = -INFINITY;
  for (int s = 0; s < p.max_splits; ++s) M = fmaxf(M, pb[(s * kH + h) * kPartStride + kD]);
  float acc_o[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc_o[j] = 0.0f;
  float lsum = 0.0f;
  // four splits per step: their loads are issued together
  for (int s0 = 0; s0 < p.max_splits; s0 += 4) {
    float4 v[4][4];
    float ms[4], ls[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = s0 + u < p.max_splits ? s0 + u : p.max_splits - 1;
      const float* ps = pb + (s * kH + h) * kPartStride;
      ms[u] = s0 + u < p.max_splits ? ps[kD] : -INFINITY;
      ls[u] = ps[kD + 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[u][j] = *reinterpret_cast<const float4*>(ps + c0 + 4 * j);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wgt = (ms[u] == -INFINITY) ? 0.0f : exp2f(ms[u] - M);
      lsum += wgt * ls[u];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc_o[4 * j] += wgt * v[u][j].x; acc_o[4 * j + 1] += wgt * v[u][j].y;
        acc_o[4 * j + 2] += wgt * v[u][j].z; acc_o[4 * j + 3] += wgt * v[u][j].w;
      }
    }
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  float* dsto = p.layer[layer].out + ((int64_t)row * kH + h) * kD + c0;
#pragma unroll
  for (int j = 0; j < 16; j += 4)
    *reinterpret_cast<float4*>(dsto + j) =
        make_float4(acc_o[j] * inv, acc_o[j + 1] * inv, acc_o[j + 2] * inv, acc_o[j + 3] * inv);
}

hipError_t launch_attention(const AttnPass& p, hipStream_t stream) {
  const int units = p.n_layers * p.rows;
  if (units == 0) return hipSuccess;
  const int gu = (units >= kXcds && p.max_splits > 1) ? (units + kXcds - 1) / kXcds * kXcds : units;
  int h = prof_begin(CSA2_K_ATTENTION, stream);
  hipLaunchKernelGGL(k_attention, dim3((unsigned)(gu * p.max_splits)), dim3(256), 0, stream, p);
  prof_end(h, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_splits == 1) return e;
  h = prof_begin(CSA2_K_ATTENTION_MERGE, stream);
  hipLaunchKernelGGL(k_attention_merge, dim3((unsigned)(4 * units)), dim3(128), 0, stream, p);
  prof_end(h, stream);
  return hipGetLastError();
}

}  // namespace csa2
