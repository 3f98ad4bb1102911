// Cache encoders: FP4 main KV, fp8 indexer key (with the ratio-2 pair mean),
// and the hierarchical block keys.
//
// Main-KV format (ai-wave.ru "DeepSeek V4.1-Flash: 1M context, FP4 KV cache
// ...", fourth paragraph; agentnet.co.il "DeepSeek launches V4.1-Flash ...",
// section "Quantization and deployment"): E2M1 values, one E4M3 scale per 16
// channels, no global scale.  Rounding decisions use exact binary32 products
// and IEEE-rounded divisions (f32_div / f32_add / f32_mul), so the
// stored bytes do not depend on FMA contraction or fast-math.
#include "kernels.hpp"

// Stored bytes must follow binary32 rounding of every step: no mul+add fusion.
#pragma clang fp contract(off)

namespace csa2 {

// One thread per 16-channel block of one entry: 32 threads per latent row, so
// a 256-thread workgroup encodes 8 entries.  The first four threads of each
// entry's group also encode the 64-channel indexer key (16 channels each).
__global__ __launch_bounds__(256) void k_quantize(
    const float* __restrict__ x, int64_t ld_x, int32_t ratio, int64_t n_entries,
    uint8_t* __restrict__ nib, uint8_t* __restrict__ scale,
    const float* __restrict__ kin, int64_t ld_k, uint8_t* __restrict__ k8,
    float* __restrict__ kscale) {
  const int64_t entry = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int blk = threadIdx.x & 31;
  if (entry >= n_entries) return;  // whole 32-lane groups leave together

  // ---- main latent block
  float v[16];
  const float* r0 = x + entry * ratio * ld_x + blk * 16;
  if (ratio == 1) {
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      float4 t = *reinterpret_cast<const float4*>(r0 + i);
      v[i] = t.x; v[i + 1] = t.y; v[i + 2] = t.z; v[i + 3] = t.w;
    }
  } else {
    const float* r1 = r0 + ld_x;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      float4 a = *reinterpret_cast<const float4*>(r0 + i);
      float4 b = *reinterpret_cast<const float4*>(r1 + i);
      v[i] = f32_mul(f32_add(a.x, b.x), 0.5f);
      v[i + 1] = f32_mul(f32_add(a.y, b.y), 0.5f);
      v[i + 2] = f32_mul(f32_add(a.z, b.z), 0.5f);
      v[i + 3] = f32_mul(f32_add(a.w, b.w), 0.5f);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
  const uint32_t sc = fp4_block_scale(amax);
  const float s = e4m3_mag(sc);
  uint32_t w0 = 0, w1 = 0;
  if (s > 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) w0 |= fp4_code(v[i], s) << (4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) w1 |= fp4_code(v[8 + i], s) << (4 * i);
  }
  *reinterpret_cast<uint2*>(nib + entry * CSA2_NIB_BYTES + blk * 8) = make_uint2(w0, w1);
  scale[entry * CSA2_SCALE_BYTES + blk] = (uint8_t)sc;

  // ---- indexer key: 4 lanes x 16 channels
  if (kin == nullptr) return;
  float kv[16];
  float kmax = 0.0f;
  if (blk < 4) {
    const float* q0 = kin + entry * ratio * ld_k + blk * 16;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a = q0[i];
      kv[i] = (ratio == 1) ? a : f32_mul(f32_add(a, q0[ld_k + i]), 0.5f);
      kmax = fmaxf(kmax, __builtin_fabsf(kv[i]));
    }
  }
  // amax over the 4 lanes of this entry (lanes 0..3 of the 32-lane group)
  kmax = fmaxf(kmax, quad_xor1(kmax));
  kmax = fmaxf(kmax, quad_xor2(kmax));
  if (blk >= 4) return;
  const float ks = f32_div(kmax, 448.0f);
  uint32_t c[4] = {0, 0, 0, 0};
  if (ks > 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i >> 2] |= e4m3_from_f32(f32_div(kv[i], ks)) << (8 * (i & 3));
  }
  *reinterpret_cast<uint4*>(k8 + entry * CSA2_D_INDEX + blk * 16) = make_uint4(c[0], c[1], c[2], c[3]);
  if (blk == 0) kscale[entry] = ks;
}

// Per-head indexer keys: 16 lanes per entry (256 values, 16 per lane), so
// a workgroup encodes 16 entries; the scale is the amax over all 16 lanes.
__global__ __launch_bounds__(256) void k_quantize_head_keys(const float* __restrict__ kin, int64_t ld_k,
                                                             int32_t ratio, int64_t n_entries,
                                                             uint8_t* __restrict__ k8,
                                                             float* __restrict__ kscale) {
  const int64_t entry = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  if (entry >= n_entries) return;  // whole 16-lane groups leave together
  float kv[16];
  float kmax = 0.0f;
  const float* q0 = kin + entry * ratio * ld_k + part * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float a = q0[i];
    kv[i] = (ratio == 1) ? a : f32_mul(f32_add(a, q0[ld_k + i]), 0.5f);
    kmax = fmaxf(kmax, __builtin_fabsf(kv[i]));
  }
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) kmax = fmaxf(kmax, __shfl_xor(kmax, d, 64));
  const float ks = f32_div(kmax, 448.0f);
  uint32_t c[4] = {0, 0, 0, 0};
  if (ks > 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i >> 2] |= e4m3_from_f32(f32_div(kv[i], ks)) << (8 * (i & 3));
  }
  *reinterpret_cast<uint4*>(k8 + entry * 4 * CSA2_D_INDEX + part * 16) = make_uint4(c[0], c[1], c[2], c[3]);
  if (part == 0) kscale[entry] = ks;
}

// Block keys: one thread per (block, 16-channel quarter); a quad encodes one
// block.  Block b holds entries 8b .. min(8b+8, n)-1 of its sequence.
__global__ __launch_bounds__(256) void k_block_keys(
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, int64_t k_stride,
    SeqArgs sa, uint8_t* __restrict__ bk8, float* __restrict__ bks, int64_t bk_stride) {
  const int seq = blockIdx.y;
  const int64_t block = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int quarter = threadIdx.x & 3;
  const int64_t n = sa.a[seq];
  const int64_t nb = (n + 7) / 8;
  const bool live = block < nb;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  int count = 0;
  if (live) {
    const uint8_t* kb = k8 + (seq * k_stride + block * 8) * CSA2_D_INDEX + quarter * 16;
    const float* sb = ks + seq * k_stride + block * 8;
    const int64_t rem = n - block * 8;
    count = rem < 8 ? (int)rem : 8;
    for (int j = 0; j < count; ++j) {          // position order
      uint4 raw = *reinterpret_cast<const uint4*>(kb + j * CSA2_D_INDEX);
      const float s = sb[j];
      uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float d = f32_mul(e4m3_value((w[i >> 2] >> (8 * (i & 3))) & 0xFFu), s);
        acc[i] = f32_add(acc[i], d);
      }
    }
  }
  float kmax = 0.0f;
  const float fc = (float)(count > 0 ? count : 1);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc[i] = f32_div(acc[i], fc);
    kmax = fmaxf(kmax, __builtin_fabsf(acc[i]));
  }
  kmax = fmaxf(kmax, quad_xor1(kmax));
  kmax = fmaxf(kmax, quad_xor2(kmax));
  if (!live) return;
  const float kss = f32_div(kmax, 448.0f);
  uint32_t c[4] = {0, 0, 0, 0};
  if (kss > 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i >> 2] |= e4m3_from_f32(f32_div(acc[i], kss)) << (8 * (i & 3));
  }
  *reinterpret_cast<uint4*>(bk8 + (seq * bk_stride + block) * CSA2_D_INDEX + quarter * 16) =
      make_uint4(c[0], c[1], c[2], c[3]);
  if (quarter == 0) bks[seq * bk_stride + block] = kss;
}

// The write side of a decode step: one 64-thread workgroup per sequence.
// The encoding arithmetic is k_quantize's and k_block_keys' (same helpers,
// same binary32 order), so appended tokens give the bytes the bulk encoders
// give for the whole history.
__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__global__ __launch_bounds__(64) void k_append(AppendPass p) {
  const int s = blockIdx.x, t = threadIdx.x;  // lane t: latent channels 8t..8t+7, key channel t
  const int64_t pos = p.seq.a[s];
  const float* xr = p.x + (int64_t)s * CSA2_D_LATENT;
  const float* kr = p.k_in + (int64_t)s * CSA2_D_INDEX;
  float* pend = p.pending ? p.pending + (int64_t)s * (CSA2_D_LATENT + CSA2_D_INDEX) : nullptr;
  const bool hold = p.ratio == 2 && (pos & 1) == 0;  // an even token waits for its pair
  const bool paired = p.ratio == 2 && !hold;
  const int64_t e = p.ratio == 1 ? pos : pos >> 1;
  const int64_t blk = e >> 3;
  const int count = (int)(e - 8 * blk) + 1;           // entries of the block, the new one included
  const bool blocks = p.bk8 != nullptr && !hold;

  // every global load first, so their latencies overlap
  const float4 xa = *reinterpret_cast<const float4*>(xr + 8 * t);
  const float4 xb = *reinterpret_cast<const float4*>(xr + 8 * t + 4);
  const float kin = kr[t];
  float4 pa = make_float4(0.f, 0.f, 0.f, 0.f), pb = pa;
  float kpend = 0.0f;
  if (paired) {
    pa = *reinterpret_cast<const float4*>(pend + 8 * t);
    pb = *reinterpret_cast<const float4*>(pend + 8 * t + 4);
    kpend = pend[CSA2_D_LATENT + t];
  }
  // the cache entries: contiguous, or one page of a pool (the block's eight
  // entries lie in the new entry's page: pages hold whole blocks); paged
  // accesses go through descriptors over the pool
  const bool paged = p.pm.pages != nullptr;
  const uint32_t lim = paged ? (uint32_t)p.pm.pool : (uint32_t)CSA2_MAX_ENTRIES;
  const int64_t ent = paged ? (int64_t)paged_entry_at(p.pm, s, e) : (int64_t)s * p.stride + e;
  const int64_t base = paged ? 0 : (int64_t)s * p.stride;  // descriptor start, in entries
  const uint32_t rel = (uint32_t)(ent - base);             // the new entry, from there
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.k8 + base * CSA2_D_INDEX), 0, (int)(lim * CSA2_D_INDEX), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.kscale + base), 0, (int)(lim * 4), kRawBufferWord3);
  uint32_t prev[7];
  float prev_s[7];
  {
    const uint32_t e0 = rel - (uint32_t)(e - 8 * blk);  // the block's first entry
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      const bool ok = blocks && j + 1 < count;
      prev[j] = ok ? __builtin_amdgcn_raw_buffer_load_b8(rk, (int)((e0 + j) * CSA2_D_INDEX) + t, 0, 0) : 0u;
      prev_s[j] = ok ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rks, (int)((e0 + j) * 4), 0, 0)) : 0.0f;
    }
  }

  // window ring: bf16 of channels 8t .. 8t+7 (nearest, ties to even)
  const float f[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
  if (p.swa) {
    const int64_t row = pos % p.swa_ring;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = __float_as_uint(f[2 * i]), hi = __float_as_uint(f[2 * i + 1]);
      lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
      hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
      w[i] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(p.swa + ((int64_t)s * p.swa_stride + row) * CSA2_D_LATENT + 8 * t) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (hold) {
    *reinterpret_cast<float4*>(pend + 8 * t) = xa;
    *reinterpret_cast<float4*>(pend + 8 * t + 4) = xb;
    pend[CSA2_D_LATENT + t] = kin;
    return;
  }

  // ---- main latent: 16-channel block b on lanes 2b (channels 16b..16b+7)
  // and 2b+1 (the next 8); the entry is the token (ratio 1) or the pair
  // mean (ratio 2)
  float v[8];
  const float pv[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = paired ? f32_mul(f32_add(pv[i], f[i]), 0.5f) : f[i];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
  amax = fmaxf(amax, quad_xor1(amax));  // both lanes of the block
  const uint32_t sc = fp4_block_scale(amax);
  const float sv = e4m3_mag(sc);
  uint32_t w8 = 0;
  if (sv > 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) w8 |= fp4_code(v[i], sv) << (4 * i);
  }
  const __amdgpu_buffer_rsrc_t rn = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.nib + base * CSA2_NIB_BYTES), 0, (int)(lim * CSA2_NIB_BYTES), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.scale + base * CSA2_SCALE_BYTES), 0, (int)(lim * CSA2_SCALE_BYTES), kRawBufferWord3);
  __builtin_amdgcn_raw_buffer_store_b32(w8, rn, (int)(rel * CSA2_NIB_BYTES) + t * 4, 0, 0);
  if ((t & 1) == 0) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, rsc, (int)(rel * CSA2_SCALE_BYTES) + (t >> 1), 0, 0);

  // ---- indexer key: channel t
  const float kv = paired ? f32_mul(f32_add(kpend, kin), 0.5f) : kin;
  const float ks = f32_div(wave_max64(__builtin_fabsf(kv)), 448.0f);
  const uint32_t code = ks > 0.0f ? e4m3_from_f32(f32_div(kv, ks)) : 0u;
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code, rk, (int)(rel * CSA2_D_INDEX) + t, 0, 0);
  if (t == 0) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ks), rks, (int)(rel * 4), 0, 0);

  // ---- block key of the new entry's block, channel t: its earlier entries
  // in position order, then the new key
  if (!blocks) return;
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    if (j + 1 >= count) break;
    acc = f32_add(acc, f32_mul(e4m3_value(prev[j]), prev_s[j]));
  }
  acc = f32_add(acc, f32_mul(e4m3_value(code), ks));
  acc = f32_div(acc, (float)count);
  const float bs = f32_div(wave_max64(__builtin_fabsf(acc)), 448.0f);
  p.bk8[((int64_t)s * p.bk_stride + blk) * CSA2_D_INDEX + t] = (uint8_t)(bs > 0.0f ? e4m3_from_f32(f32_div(acc, bs)) : 0u);
  if (t == 0) p.bks[(int64_t)s * p.bk_stride + blk] = bs;
}

hipError_t launch_append(const AppendPass& p, int32_t batch, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const int h = prof_begin(CSA2_K_APPEND, stream);
  hipLaunchKernelGGL(k_append, dim3((unsigned)batch), dim3(64), 0, stream, p);
  prof_end(h, stream);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* x, int64_t n_entries, int64_t ld_x, int32_t ratio,
                           uint8_t* nib, uint8_t* scale, const float* kin, int64_t ld_k,
                           uint8_t* k8, float* kscale, hipStream_t stream) {
  if (n_entries == 0) return hipSuccess;
  const int64_t grid = (n_entries + 7) / 8;
  const int h = prof_begin(CSA2_K_QUANTIZE, stream);
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)grid), dim3(256), 0, stream, x, ld_x, ratio,
                     n_entries, nib, scale, kin, ld_k, k8, kscale);
  prof_end(h, stream);
  return hipGetLastError();
}

hipError_t launch_quantize_head_keys(const float* kin, int64_t n_entries, int64_t ld_k, int32_t ratio, uint8_t* k8,
                                     float* kscale, hipStream_t stream) {
  if (n_entries == 0) return hipSuccess;
  const int h = prof_begin(CSA2_K_QUANTIZE, stream);
  hipLaunchKernelGGL(k_quantize_head_keys, dim3((unsigned)((n_entries + 15) / 16)), dim3(256), 0, stream, kin, ld_k,
                     ratio, n_entries, k8, kscale);
  prof_end(h, stream);
  return hipGetLastError();
}

hipError_t launch_block_keys(const uint8_t* k8, const float* ks, int64_t k_stride,
                             const int64_t* n_entries, int32_t batch, uint8_t* bk8, float* bks,
                             int64_t bk_stride, hipStream_t stream) {
  for (int32_t s0 = 0; s0 < batch; s0 += kMaxSeqPerLaunch) {
    const int32_t nb = batch - s0 < kMaxSeqPerLaunch ? batch - s0 : kMaxSeqPerLaunch;
    SeqArgs sa = {};
    int64_t max_blocks = 0;
    for (int32_t i = 0; i < nb; ++i) {
      sa.a[i] = n_entries[s0 + i];
      const int64_t b = (n_entries[s0 + i] + 7) / 8;
      max_blocks = b > max_blocks ? b : max_blocks;
    }
    if (max_blocks == 0) continue;
    dim3 grid((unsigned)((max_blocks + 63) / 64), (unsigned)nb);
    const int h = prof_begin(CSA2_K_BLOCK_KEYS, stream);
    hipLaunchKernelGGL(k_block_keys, grid, dim3(256), 0, stream, k8 + s0 * k_stride * CSA2_D_INDEX,
                       ks + s0 * k_stride, k_stride, sa, bk8 + s0 * bk_stride * CSA2_D_INDEX,
                       bks + s0 * bk_stride, bk_stride);
    prof_end(h, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace csa2
