// Shared device helpers of libcsa2: number-format codecs, DPP lane exchange,
// order-preserving score keys, and launch helpers.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa2.h"

namespace csa2 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Buffer descriptor word 3 for untyped (raw) buffer access on gfx9 parts;
// the cache-policy bit of nontemporal raw buffer loads.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kLoadNonTemporal = 2;
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kD = CSA2_D_LATENT;
constexpr int kDI = CSA2_D_INDEX;
constexpr int kHI = CSA2_H_INDEX;
constexpr int kH = CSA2_H_ATTN;

// ---------------------------------------------------------------- binary32
// One rounding per operation.  The pragma keeps these from being fused into
// an FMA with a neighbouring operation after inlining (HIP contracts a*b+c
// by default, and the library's __fmul_rn/__fadd_rn are plain operators).
__device__ __forceinline__ float f32_mul(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ float f32_add(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}
// IEEE division, correctly rounded (no fast-math in this library).
__device__ __forceinline__ float f32_div(float a, float b) { return a / b; }

// ---------------------------------------------------------------- E4M3 / E2M1
// E4M3 ("E4M3FN", OCP MX): bias 7, subnormals m * 2^-9, max 448, NaN 0x7F/0xFF.
// Value of a non-negative code 0..126, exactly, built from its bits.
__device__ __forceinline__ float e4m3_mag(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;        // m * 2^-9, exact
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  float v = e4m3_mag(c & 0x7Fu);
  return (c & 0x80u) ? -v : v;
}

// Round a binary32 value to E4M3: nearest, ties to even, saturating at 448,
// sign kept for values rounding to zero.  Integer bit manipulation only.
__device__ __forceinline__ uint32_t e4m3_from_f32(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {                // |x| >= 448
    code = 0x7Eu;
  } else if (a >= 0x3C800000u) {         // |x| >= 2^-6: normal E4M3 range
    uint32_t exp = (a >> 23) - 120u;     // E4M3 exponent field 1..15
    uint32_t man = a & 0x7FFFFFu;
    uint32_t keep = man >> 20, rest = man & 0xFFFFFu;
    uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
    code = (exp << 3) + keep + up;       // a mantissa carry moves into the exponent
    if (code > 0x7Eu) code = 0x7Eu;
  } else {                               // subnormal: integer multiple of 2^-9
    float n = __builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scaling, RNE
    code = (uint32_t)n;                  // 0..8; 8 is the smallest normal 0x08
  }
  return code | sign;
}

// E4M3 scale of an FP4 block: the code nearest amax/6 (real quotient), ties to
// even, saturating.  Decided with exact products 6*v, never by dividing.
__device__ __forceinline__ uint32_t fp4_block_scale(float amax) {
  if (!(amax > 0.0f)) return 0u;
  if (amax >= 2688.0f) return 0x7Eu;     // amax/6 >= 448
  // largest code c in [0,126] with 6*value(c) <= amax (value(0) = 0 always fits)
  uint32_t lo = 0, hi = 126;
  while (lo < hi) {
    uint32_t mid = (lo + hi + 1) >> 1;
    if (6.0f * e4m3_mag(mid) <= amax) lo = mid; else hi = mid - 1;
  }
  if (lo == 126u) return lo;
  // midpoint of value(lo) and value(lo+1) is exact (few significant bits)
  float mid2 = e4m3_mag(lo) + e4m3_mag(lo + 1u);  // twice the midpoint, exact
  float t = 3.0f * mid2;                            // 6 * midpoint, exact
  if (amax > t) return lo + 1u;
  if (amax == t) return (lo & 1u) ? lo + 1u : lo;
  return lo;
}

// E2M1 code of x for scale value s > 0: nearest of {0,.5,1,1.5,2,3,4,6}*s,
// ties to the even code, saturating; the sign bit follows x.  Every threshold
// t*s is exact in binary32.
__device__ __forceinline__ uint32_t fp4_code(float x, float s) {
  float a = __builtin_fabsf(x);
  uint32_t c = (a > 0.25f * s) + (a >= 0.75f * s) + (a > 1.25f * s) + (a >= 1.75f * s) +
               (a > 2.5f * s) + (a >= 3.5f * s) + (a > 5.0f * s);
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

// ---------------------------------------------------------------- score keys
// Order-preserving map of a binary32 score to uint32 (larger score, larger
// key).  -0 is folded into +0 first so equal scores give equal keys.
__device__ __forceinline__ uint32_t score_key(float s) {
  s = s + 0.0f;
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit selection key: score first, then the lower position wins ties.
__device__ __forceinline__ uint64_t select_key(uint32_t skey, uint32_t pos) {
  return ((uint64_t)skey << 32) | (uint64_t)(0xFFFFFFFFu - pos);
}
__device__ __forceinline__ uint32_t select_key_pos(uint64_t key) {
  return 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu);
}

// ---------------------------------------------------------------- lanes
// Quad exchange through DPP (quad_perm), no LDS round trip.
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS
// round trips): steps of 1, 2, 4 and 8 lanes inside each row of 16, then the
// totals of lanes 15 and 31 are broadcast into the rows above them.
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Largest uint32 of the wave, in every lane (DPP steps as in wave_incl_add;
// a lane without a source keeps its own value: 0 is the identity of max).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false));  // row_shr:1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false));  // row_shr:2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false));  // row_shr:4
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false));  // row_shr:8
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));  // row_bcast:15
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// One step of a 64-bit max (kMax) or min scan; lanes without a source keep
// their own value (the identity is fed in as the old value).
template <bool kMax, int kCtrl, int kRowMask>
__device__ __forceinline__ uint64_t dpp_step64(uint64_t x) {
  const int id = kMax ? 0 : -1;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(id, (int)(uint32_t)x, kCtrl, kRowMask, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(id, (int)(uint32_t)(x >> 32), kCtrl, kRowMask, 0xF, false);
  const uint64_t y = ((uint64_t)hi << 32) | lo;
  return kMax ? (y > x ? y : x) : (y < x ? y : x);
}

// Largest (kMax) or smallest 64-bit value of the wave, in every lane.
template <bool kMax>
__device__ __forceinline__ uint64_t wave_reduce64(uint64_t x) {
  x = dpp_step64<kMax, 0x111, 0xF>(x);
  x = dpp_step64<kMax, 0x112, 0xF>(x);
  x = dpp_step64<kMax, 0x114, 0xF>(x);
  x = dpp_step64<kMax, 0x118, 0xF>(x);
  x = dpp_step64<kMax, 0x142, 0xA>(x);
  x = dpp_step64<kMax, 0x143, 0xC>(x);
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), 63) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 63);
}

// x[lane] op x[lane ^ 16] and x[lane] op x[lane ^ 32] for a commutative op,
// through the lane swaps of gfx950 (v_permlane16_swap / v_permlane32_swap:
// VALU, no LDS round trip).  With both operands the same register, the two
// results of a swap are x[lane] and x[lane ^ 16] (or ^ 32) in some order.
// Every lane of the wave must be active.
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Histogram increment of `bin` by the calling lanes.  When every calling lane
// of the wave hits the same bin (keys sharing their high bits, the common case
// in top-k refinement) one lane adds the whole count: without it the LDS
// atomics of the wave serialise on one address.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin) {
  const unsigned long long act = __ballot(1);
  const int first = __ffsll((long long)act) - 1;
  const uint32_t ref = (uint32_t)__shfl((int)bin, first, 64);
  const unsigned long long same = __ballot(bin == ref);
  if (same == act) {
    if ((int)(threadIdx.x & 63) == first) atomicAdd(hist + ref, (uint32_t)__popcll(act));
  } else {
    atomicAdd(hist + bin, 1u);
  }
}

// Number of workgroups per XCD group: consecutive workgroup ids are spread
// round-robin over the 8 XCDs; these helpers remap a linear id so that the
// workgroups of one row land on one XCD (one L2).
constexpr int kXcds = 8;

}  // namespace csa2
