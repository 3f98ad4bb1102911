// Workgroup-wide selection helpers shared by the decode and prefill top-k.
#pragma once

#include "common.hpp"

namespace csa2 {

// Inclusive prefix sum over the NW waves of a workgroup: a DPP scan inside
// each wave, one LDS exchange of the wave totals.
template <int NW>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_add(v);
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    before += i < wave ? wsum[i] : 0u;
    all += wsum[i];
  }
  total = all;
  __syncthreads();
  return before + x;
}

__device__ __forceinline__ uint32_t block_incl_scan_256(uint32_t v, uint32_t* wsum, uint32_t& total) {
  return block_incl_scan<4>(v, wsum, total);
}

// Exact k-th largest of the unique non-zero 64-bit keys held in registers
// (kPer per thread, 256 threads, zeros for empty slots; at least two keys).
// All keys lie between the smallest and the largest, so they share the bits
// above the highest bit where those two differ: the radix starts there, with
// 11-bit steps, and ends as soon as the chosen bucket is taken whole.
// Returns the k-th key, or the lower edge of a bucket that holds exactly the
// keys from the top down to the k-th; either way the keys >= the result are
// the k largest.  `bins` is 2048 words of LDS.
template <int kPer>
__device__ uint64_t block_kth_regs(const uint64_t (&key)[kPer], uint32_t want, uint32_t* bins, uint32_t* wsum,
                                   uint32_t* sh) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  __shared__ uint64_t mm[2][4];
  // smallest and largest key
  uint64_t lo = ~0ull, hi = 0ull;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (key[i] != 0ull && key[i] < lo) lo = key[i];
    if (key[i] > hi) hi = key[i];
  }
  lo = wave_reduce64<false>(lo);
  hi = wave_reduce64<true>(hi);
  if (lane == 0) { mm[0][wave] = lo; mm[1][wave] = hi; }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    lo = mm[0][w] < lo ? mm[0][w] : lo;
    hi = mm[1][w] > hi ? mm[1][w] : hi;
  }
  int top = 64 - __clzll((long long)(lo ^ hi));  // bits [top - 1, 0] are undecided
  uint64_t pmask = top >= 64 ? 0ull : ~((1ull << top) - 1ull);
  uint64_t prefix = lo & pmask;
  uint32_t need = want;
#pragma unroll 1
  while (top > 0) {
    const int width = top < 11 ? top : 11;
    const int shift = top - width;
    const uint32_t nb = 1u << width;
    for (uint32_t i = t; i < 2048; i += 256) bins[i] = 0;
    if (t == 0) sh[0] = 0xFFFFFFFFu;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (key[i] != 0ull && (key[i] & pmask) == prefix) atomicAdd(&bins[(uint32_t)(key[i] >> shift) & (nb - 1)], 1u);
    __syncthreads();
    // thread t owns bins 8t .. 8t+7
    uint32_t hb[8], local = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hb[j] = bins[8 * t + j];
      local += hb[j];
    }
    uint32_t total;
    const uint32_t incl = block_incl_scan_256(local, wsum, total);
    uint32_t run = total - incl;  // keys in bins above 8t + 7
    if (run < need && run + local >= need) {
      for (int j = 7; j >= 0; --j) {
        if (run + hb[j] >= need) { sh[0] = 8 * t + j; sh[1] = need - run; sh[2] = hb[j]; break; }
        run += hb[j];
      }
    }
    __syncthreads();
    const uint32_t digit = sh[0], nneed = sh[1], count = sh[2];
    __syncthreads();
    prefix |= (uint64_t)digit << shift;
    pmask |= (uint64_t)(nb - 1) << shift;
    need = nneed;
    top = shift;
    if (need == count) break;  // the whole bucket is taken
  }
  return prefix;
}

// Smallest non-zero key at or above `edge` over the workgroup (256 threads);
// ~0 when there is none.  Turns the bucket edge of block_kth_regs into the
// k-th key itself.
template <int kPer>
__device__ uint64_t block_min_at_least(const uint64_t (&key)[kPer], uint64_t edge) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ uint64_t wmin[4];
  uint64_t m = ~0ull;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (key[i] != 0ull && key[i] >= edge && key[i] < m) m = key[i];
  m = wave_reduce64<false>(m);
  if (lane == 0) wmin[wave] = m;
  __syncthreads();
  m = ~0ull;
#pragma unroll
  for (int w = 0; w < 4; ++w) m = wmin[w] < m ? wmin[w] : m;
  __syncthreads();
  return m;
}

}  // namespace csa2
