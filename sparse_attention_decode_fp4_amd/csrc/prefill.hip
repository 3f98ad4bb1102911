// Indexer of a prefill chunk: many query rows scored against the same keys.
//
// Here the indexer scoring is a real dense contraction (query rows x 4 heads
// against every visible key), so it runs on fp8 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales).  The score and the
// selection rule are those of the decode indexer (a reading, see index.hip).
//
// Per-row top-k without materialising the score matrix, in four kernels:
//   sample     MFMA scores of every row against a strided sample of at most
//              2,048 keys of its row tile;
//   threshold  per row, T0 = the k_s-th largest sample score, with k_s sized
//              so that about 2.5 k keys of the full row reach T0;
//   filter     MFMA scores of every visible (row, key) pair; pairs scoring at
//              least T0 are appended to the row's candidate list, one segment
//              per (row, key range): their scores are staged in LDS and, after
//              every four A tiles, appended one per lane and round, each slot
//              from an LDS atomic on its row's count; the grid is sized to
//              fill the device in one round;
//   select     if the list holds at least min(k, visible) candidates and did
//              not overflow, it contains the whole top k.  MFMA scores are
//              not binary32-exact (measured error up to ~2.5e-5 of the sum
//              of |products|), so they settle only keys clearly above or
//              below the MFMA k-th score; keys within 2^-8 of it are rescored
//              on VALU (the decode scan's arithmetic) and ranked exactly.
//              Winners are sorted by position.  If the list cannot hold the
//              answer (overflow, too few keys, or the 2^-8 band reaches below
//              the sampled threshold) the row is recomputed exactly on its own
//              (VALU scoring, radix steps over recomputed keys): slow, exact,
//              and reached only when the sample misleads.
#include <atomic>

#include "kernels.hpp"
#include "select.hpp"

namespace csa2 {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kPfStage = 256;   // keys staged in LDS per step

// max(x, 0) as one integer max on the bits (negative floats, -0 included,
// are negative integers), without the NaN canonicalisation of fmaxf.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }
constexpr uint32_t kUnitScales = 0x7F7F7F7Fu;  // E8M0 127 = 1.0 in every byte

__device__ __forceinline__ int64_t pf_visible(const PrefillPass& p, int seq, int64_t qi) {
  const int64_t pos = p.seq.a[seq] + qi;
  int64_t v = (pos + 1) / p.ratio;
  const int64_t ne = p.seq.b[seq];
  v = v < ne ? v : ne;
  return v < 0 ? 0 : v;
}

// Samples of a row tile: S = min(V, kPfSample) keys j(t) = t*V/S, V being the
// visible count of the tile's first query (the smallest of the tile).
__device__ __forceinline__ int64_t pf_sample_key(int64_t t, int64_t V, int64_t S) {
  return S == V ? t : (t * V) / kPfSample;  // S == kPfSample whenever strided
}

__device__ __forceinline__ float tv_at(const float4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float key_to_score(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

// ------------------------------------------------------------------ MFMA pass
// Workgroup: 256 query rows of one sequence (wave w: rows 64w..64w+63 as
// eight A tiles of 8 queries x 4 heads) against a range of keys staged in LDS.
template <bool kFilter, bool kHasW>
__global__ __launch_bounds__(256) void k_prefill_mfma(PrefillPass p) {
  const int split = blockIdx.x % p.esplit;
  const int tile = blockIdx.x / p.esplit;
  const int seq = tile / p.tiles_per_seq;
  const int64_t q0 = (int64_t)(tile % p.tiles_per_seq) * kPfRows;
  const int nq_tile = (int)((p.n_q - q0) < kPfRows ? (p.n_q - q0) : kPfRows);
  const int64_t row0 = (int64_t)seq * p.n_q + q0;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, half = lane >> 5;

  const int64_t v_first = pf_visible(p, seq, q0);
  const int64_t v_last = pf_visible(p, seq, q0 + nq_tile - 1);
  // key range of this workgroup
  int64_t n_keys, k_begin, k_end;
  if (kFilter) {
    n_keys = v_last;
  } else {
    n_keys = v_first < kPfSample ? v_first : kPfSample;
  }
  {
    const int64_t per = ((n_keys + p.esplit - 1) / p.esplit + 31) / 32 * 32;
    k_begin = split * per;
    k_end = k_begin + per < n_keys ? k_begin + per : n_keys;
  }
  if (k_begin >= k_end) {
    if (kFilter)
      for (int i = t; i < nq_tile; i += 256) p.count[(row0 + i) * kPfSplits + split] = 0;
    return;
  }

  __shared__ __attribute__((aligned(16))) uint8_t stage[2][kPfStage * kDI];
  __shared__ float stage_ks[2][kPfStage];
  __shared__ int64_t vis_row[kPfRows];
  __shared__ __attribute__((aligned(16))) float w_row[kHasW ? kPfRows * kHI : 4];
  // row thresholds (filter), each group of 8 rows stored as [even rows,
  // odd rows], so a lane's four rows 8a + 2i + half are one 16-byte read
  __shared__ __attribute__((aligned(16))) float thr[kFilter ? kPfRows : 4];
  // filter: the scores of a quarter of a key block's pairs (A tiles a0,
  // a0 + 1) per wave, [wave][4 (a mod 2) + i][lane], and the candidate count
  // of each row (8 KB + 1 KB: three workgroups still fit on a CU)
  __shared__ float sst[kFilter ? 4 * 8 * 64 : 4];
  __shared__ uint32_t lcnt[kFilter ? kPfRows : 4];

  for (int i = t; i < kPfRows; i += 256) vis_row[i] = i < nq_tile ? pf_visible(p, seq, q0 + i) : 0;
  if (kFilter)
    for (int i = t; i < kPfRows; i += 256) {
      thr[(i & ~7) + 4 * (i & 1) + ((i & 7) >> 1)] = i < nq_tile ? p.thresh[row0 + i] : INFINITY;
    }
  if (kHasW)
    for (int i = t; i < kPfRows * kHI; i += 256)
      w_row[i] = (i / kHI) < nq_tile ? p.idx_w[(row0 + i / kHI) * kHI + (i % kHI)] : 0.0f;

  // A operands: tile a = queries 64w + 8a .. +8, row m = 4*query + head,
  // lane holds 32 consecutive channels 32*half .. of row l32
  v8i_t A[8];
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int ql = 64 * wave + 8 * a + (l32 >> 2);
    const int h = l32 & 3;
    uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
    if (ql < nq_tile) {
      const uint8_t* src = p.idx_q + ((row0 + ql) * kHI + h) * kDI + 32 * half;
      lo = *reinterpret_cast<const uint4*>(src);
      hi = *reinterpret_cast<const uint4*>(src + 16);
    }
    A[a] = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  const int seq_keys = 0;
  (void)seq_keys;
  const uint8_t* kb = p.k8 + (int64_t)seq * p.k_stride * kDI;
  const float* sb = p.kscale + (int64_t)seq * p.k_stride;

  auto key_of = [&](int64_t slot) -> int64_t {
    return kFilter ? slot : pf_sample_key(slot, v_first, n_keys);
  };
  // cooperative staging: thread t brings key (base + t)
  auto stage_load = [&](int buf, int64_t base) {
    const int64_t slot = base + t;
    uint4 v[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
    float ksv = 0.0f;
    if (slot < k_end) {
      const int64_t key = key_of(slot);
      const uint4* src = reinterpret_cast<const uint4*>(kb + key * kDI);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = src[i];
      ksv = sb[key];
    }
    uint4* dst = reinterpret_cast<uint4*>(&stage[buf][t * kDI]);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = v[i];
    stage_ks[buf][t] = ksv;
  };

  if (kFilter) lcnt[64 * wave + lane] = 0u;  // (a wave counts only its own rows: no barrier)
  float* const sst_w = sst + (kFilter ? 8 * 64 * wave : 0);
  int buf = 0;
  stage_load(0, k_begin);
  for (int64_t base = k_begin; base < k_end; base += kPfStage) {
    __syncthreads();  // stage[buf] complete; stage[buf^1] free
    if (base + kPfStage < k_end) stage_load(buf ^ 1, base + kPfStage);
    const int n_here = (int)(k_end - base < kPfStage ? k_end - base : kPfStage);
    for (int bt = 0; bt < n_here; bt += 32) {
      const uint8_t* brow = &stage[buf][(bt + l32) * kDI + 32 * half];
      const uint4 b0 = *reinterpret_cast<const uint4*>(brow);
      const uint4 b1 = *reinterpret_cast<const uint4*>(brow + 16);
      const v8i_t B = v8i_t{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      const float ksn = stage_ks[buf][bt + l32];
      const int64_t slot = base + bt + l32;
      const bool slot_ok = (bt + l32) < n_here;
      const bool all_visible = kFilter ? (base + bt + 32 <= v_first) : true;
      uint32_t hm = 0u;  // filter: bit 4 (a mod 2) + i: the pair of row 8 a + 2 i + half reached its threshold
      // head weights and thresholds of A tile a's rows (LDS), read one tile
      // ahead of their use
      auto load_wt = [&](int a, float4 (&wv)[4], float4& tv) {
        if (kHasW)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            wv[i] = *reinterpret_cast<const float4*>(&w_row[(64 * wave + 8 * a + 2 * i + half) * kHI]);
        if (kFilter) tv = *reinterpret_cast<const float4*>(&thr[64 * wave + 8 * a + 4 * half]);
      };
      // epilogue of A tile a: ReLU-sum of the 4 heads, times the key scale;
      // filter: append the pairs at or above the row threshold
      auto epilogue = [&](const v16f_t& acc, int a, const float4 (&wv)[4], const float4& tv) {
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float r0 = relu(acc[4 * i]), r1 = relu(acc[4 * i + 1]);
          const float r2 = relu(acc[4 * i + 2]), r3 = relu(acc[4 * i + 3]);
          float sum;
          if (kHasW) {
            sum = wv[i].x * r0 + wv[i].y * r1 + wv[i].z * r2 + wv[i].w * r3;
          } else {
            sum = (r0 + r1) + (r2 + r3);
          }
          sc[i] = ksn * sum;
        }
        // every lane computes its scores before any per-lane branch: the
        // MFMA reads all lanes' operands, so it must not be sunk into one
        asm volatile("" ::"v"(sc[0]), "v"(sc[1]), "v"(sc[2]), "v"(sc[3]));
        if (kFilter) {
          // pairs at or above their row's threshold: their scores go to the
          // wave's staging area and their bits to hm, and the appends wait
          // for the flush after every odd A tile.  The causal-edge test
          // (check_vis) runs only where the key block reaches past some
          // row's visible keys (a uniform branch)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            bool h = slot_ok && sc[i] >= tv_at(tv, i);
            if (!all_visible) h = h && slot < vis_row[64 * wave + 8 * a + 2 * i + half];
            sst_w[(4 * (a & 1) + i) * 64 + lane] = sc[i];
            hm |= (h ? 1u : 0u) << (4 * (a & 1) + i);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ql = 64 * wave + 8 * a + 2 * i + half;
            if (slot_ok && ql < nq_tile) p.sample[(row0 + ql) * kPfSample + slot] = sc[i];
          }
        }
      };
      // software pipeline: the MFMA of tile a + 1 is issued before the
      // epilogue of tile a, so it runs under it.  The empty asm takes the
      // result as an operand at the issue point, which keeps the compiler
      // from sinking the MFMA past the epilogue's branch to its own use (the
      // asm emits nothing, so nothing waits for the result there)
      // Appends of the staged pairs of A tiles a0, a0 + 1: one pair per lane
      // and round, its slot from an LDS atomic on its row's count (a round
      // per hit of the lane with the most, about 1.25 on average, in place
      // of a branch per (A tile, row pair) with any hit in the wave)
      auto flush = [&](int a0) {
        while (__builtin_amdgcn_ballot_w64(hm != 0u)) {
          if (hm != 0u) {
            const int b = __builtin_ctz(hm);
            hm &= hm - 1u;
            // the staged score and the slot come back in one LDS round trip:
            // the store is unconditional (a slot past the segment goes to
            // its last entry: the row's count then exceeds the segment, and
            // the select recomputes such a row without reading its list),
            // so the score's load is not sunk behind the atomic's return
            const float scb = sst_w[b * 64 + lane];
            const int rl = 64 * wave + 8 * (a0 + (b >> 2)) + 2 * (b & 3) + half;
            const uint32_t off = atomicAdd(&lcnt[rl], 1u);
            const uint32_t at = off < (uint32_t)kPfSeg ? off : (uint32_t)kPfSeg - 1u;
            uint32_t* dst = reinterpret_cast<uint32_t*>(p.list + ((row0 + rl) * kPfSplits + split) * kPfSeg + at);
            *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)slot, __float_as_uint(scb));  // raw (position, score bits)
          }
        }
      };
      v16f_t acc[2];
      float4 wv[2][4], tv[2];
      acc[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[0], B, v16f_t{}, 0, 0, 0, kUnitScales, 0,
                                                              kUnitScales);
      if (kFilter) asm volatile("" : "+v"(acc[0]));
      if (kFilter) load_wt(0, wv[0], tv[0]);
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        if (a + 1 < 8) {
          acc[(a + 1) & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[a + 1], B, v16f_t{}, 0, 0, 0,
                                                                            kUnitScales, 0, kUnitScales);
          if (kFilter) {
            asm volatile("" : "+v"(acc[(a + 1) & 1]));
            load_wt(a + 1, wv[(a + 1) & 1], tv[(a + 1) & 1]);
          }
        }
        if (!kFilter) load_wt(a, wv[a & 1], tv[a & 1]);  // the sample pass: no pipeline
        epilogue(acc[a & 1], a, wv[a & 1], tv[a & 1]);
        if (kFilter && (a & 1) == 1) flush(a - 1);
      }
    }
    buf ^= 1;
  }
  if (kFilter && 64 * wave + lane < nq_tile) p.count[(row0 + 64 * wave + lane) * kPfSplits + split] = lcnt[64 * wave + lane];
}

// ------------------------------------------------------------------ threshold
// One wave per row: T0 = the lower edge of the 16-bit key bucket that holds
// the k_s-th largest of the row's samples (two 8-bit radix steps over
// order-preserving keys held in registers).  Rounding T0 down that way (by
// at most 2^-7 of its value) only widens the candidate list, and the select
// checks its near-tie band against the T0 it was filtered with.
__global__ __launch_bounds__(256) void k_prefill_threshold(PrefillPass p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  __shared__ uint32_t hist[4][256];
  if (row >= p.rows) return;
  const int seq = (int)(row / p.n_q);
  const int64_t qi = row - (int64_t)seq * p.n_q;
  const int64_t q0 = qi / kPfRows * kPfRows;
  const int64_t V = pf_visible(p, seq, q0);
  const int64_t S = V < kPfSample ? V : kPfSample;
  const int64_t vis = pf_visible(p, seq, qi);
  const uint32_t k = (uint32_t)p.k;
  if (vis <= (int64_t)k || S == 0) {  // every visible key is a winner, or no sample
    if (lane == 0) p.thresh[row] = -INFINITY;
    return;
  }
  uint32_t ks;
  if (S == vis) {
    ks = k;
  } else {
    const double want = 2.5 * (double)k * (double)S / (double)vis + 4.0;
    ks = want >= (double)S ? (uint32_t)S : (uint32_t)want;
  }
  if (ks >= (uint32_t)S) {  // the sample is too small to bound the row
    if (lane == 0) p.thresh[row] = -INFINITY;
    return;
  }
  uint32_t keys[kPfSample / 64];
#pragma unroll
  for (int j = 0; j < kPfSample / 64; ++j) {
    const int64_t s = (int64_t)j * 64 + lane;
    keys[j] = s < S ? score_key(p.sample[row * kPfSample + s]) : 0u;
  }
  uint32_t prefix = 0, need = ks;
  for (int shift = 24; shift >= 16; shift -= 8) {
    for (int i = lane; i < 256; i += 64) hist[wave][i] = 0;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    const uint32_t hmask = shift == 24 ? 0u : (~0u << (shift + 8));
#pragma unroll
    for (int j = 0; j < kPfSample / 64; ++j) {
      const int64_t s = (int64_t)j * 64 + lane;
      if (s < S && (keys[j] & hmask) == prefix) hist_add(hist[wave], (keys[j] >> shift) & 255u);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t c0 = hist[wave][4 * lane], c1 = hist[wave][4 * lane + 1];
    const uint32_t c2 = hist[wave][4 * lane + 2], c3 = hist[wave][4 * lane + 3];
    const uint32_t mine = c0 + c1 + c2 + c3;
    const uint32_t incl = wave_incl_add(mine);
    uint32_t ab = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl;  // keys in digits above the lane's
    const uint32_t cs[4] = {c0, c1, c2, c3};
    uint32_t found = 0xFFFFFFFFu, nneed = 0;
    for (int j = 3; j >= 0; --j) {
      if (ab < need && ab + cs[j] >= need) { found = 4 * lane + j; nneed = need - ab; }
      ab += cs[j];
    }
    // exactly one lane found the digit
    const unsigned long long ball = __ballot(found != 0xFFFFFFFFu);
    const int src = __ffsll(ball) - 1;
    const uint32_t digit = __shfl(found, src, 64);
    need = __shfl(nneed, src, 64);
    prefix |= digit << shift;
    __builtin_amdgcn_wave_barrier();
  }
  if (lane == 0) p.thresh[row] = key_to_score(prefix);
}

// ------------------------------------------------------------------ select

// Exact score of key `pos` for a row whose query (16 channels per lane, 4
// heads) sits in q; a lane quad scores one key.  Mirrors the decode scan.
__device__ __forceinline__ float pf_quad_score(const half2_t (&q)[kHI][8], const float (&w)[kHI],
                                               const uint8_t* kb, const float* sb, int64_t pos, bool valid,
                                               int quarter) {
  u32x4_t raw = u32x4_t{0, 0, 0, 0};
  float ks = 0.0f;
  if (valid) {
    raw = *reinterpret_cast<const u32x4_t*>(kb + pos * kDI + quarter * 16);
    ks = sb[pos];
  }
  float d[kHI] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[j], 1.0f, false);
    const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[j], 1.0f, true);
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
  return ks * acc;
}

__global__ __launch_bounds__(256) void k_prefill_select(PrefillPass p) {
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int seq = (int)(row / p.n_q);
  const int64_t qi = row - (int64_t)seq * p.n_q;
  const int64_t vis = pf_visible(p, seq, qi);
  const uint32_t k = (uint32_t)p.k;
  const uint32_t need_all = vis < (int64_t)k ? (uint32_t)vis : k;
  int32_t* out = p.out + row * p.out_stride;

  // 49 KB in all, so three workgroups share a CU: the k-th key's histogram
  // and the near-tie band take turns in one array (the histogram is done
  // with before the band is written, and the band's exact keys move to lc
  // before the histogram serves the band's own k-th)
  constexpr uint32_t kPfBand = 2048;  // near-tie band keys, at most (else the exact recompute)
  __shared__ uint64_t lc[kPfCap];  // candidates; after the band is settled, the position bitmap
  __shared__ uint32_t win[CSA2_MAX_K];
  __shared__ uint32_t bt_h[kPfBand];
  uint32_t* const bt = bt_h;
  uint32_t* const h2048 = bt_h;
  __shared__ uint32_t h256[256];
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t sh3[3];
  __shared__ uint64_t sh_kth;
  __shared__ uint32_t sh_need;
  __shared__ uint32_t seg_start[kPfSplits + 1];

  // exact k-th largest over n keys from `get`, by 8-bit radix steps (the
  // exact-recompute path only)
  auto radix_kth = [&](auto get, uint32_t n, uint32_t want) -> uint64_t {
    if (t == 0) { sh_kth = 0; sh_need = want; }
    for (int shift = 56; shift >= 0; shift -= 8) {
      h256[t] = 0;
      __syncthreads();
      const uint64_t prefix = sh_kth;
      const uint64_t hmask = (shift == 56) ? 0ull : (~0ull << (shift + 8));
      get(n, [&](uint32_t g, uint64_t key) {
        (void)g;
        if ((key & hmask) == prefix) atomicAdd(&h256[(uint32_t)(key >> shift) & 255u], 1u);
      });
      __syncthreads();
      const uint32_t c = h256[t];
      uint32_t tot;
      const uint32_t incl = block_incl_scan_256(c, wsum, tot);
      const uint32_t above = tot - incl;  // keys in digits above t
      const uint32_t nd = sh_need;
      __syncthreads();
      if (above < nd && above + c >= nd) {
        sh_need = nd - above;
        sh_kth = prefix | ((uint64_t)t << shift);
      }
      __syncthreads();
    }
    return sh_kth;
  };

  // the row's query as packed f16 (16 channels of each head per lane of a
  // quad) for exact rescoring on VALU
  const int quarter = t & 3;
  half2_t q[kHI][8];
  {
    const uint8_t* qp = p.idx_q + row * (kHI * kDI) + quarter * 16;
#pragma unroll
    for (int h = 0; h < kHI; ++h) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qp + h * kDI);
      const uint32_t ws4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        q[h][2 * j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws4[j], 1.0f, false);
        q[h][2 * j + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws4[j], 1.0f, true);
      }
    }
  }
  float w[kHI];
#pragma unroll
  for (int h = 0; h < kHI; ++h) w[h] = p.idx_w ? p.idx_w[row * kHI + h] : 1.0f;
  const uint8_t* kb = p.k8 + (int64_t)seq * p.k_stride * kDI;
  const float* sb = p.kscale + (int64_t)seq * p.k_stride;

  // segment counts and every segment slot in one round trip: thread t takes
  // slots 32 (t % 4) .. +32 of segment t / 4 (kPfSplits = 64 segments)
  const int sgi = t >> 2;
  const uint32_t seg = sgi < p.esplit ? p.count[row * kPfSplits + sgi] : 0u;
  uint64_t sv[kPfSeg / 4];
  if (sgi < p.esplit) {
    const uint64_t* src = p.list + (row * kPfSplits + sgi) * kPfSeg + 32 * (t & 3);
#pragma unroll
    for (int i = 0; i < kPfSeg / 4; i += 2) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + i);
      // entries are (position, score bits) as the filter wrote them
      sv[i] = select_key(score_key(__uint_as_float(v.y)), v.x);
      sv[i + 1] = select_key(score_key(__uint_as_float(v.w)), v.z);
    }
  }
  const bool seg_over = __syncthreads_or((t & 3) == 0 && seg > (uint32_t)kPfSeg);
  uint32_t cnt;
  const uint32_t mine = (t & 3) == 0 ? seg : 0u;
  const uint32_t seg_off = block_incl_scan_256(mine, wsum, cnt) - mine;
  // a row with every visible key listed (vis <= k) must list no more than k
  bool fast = !seg_over && cnt >= need_all && cnt <= (uint32_t)kPfCap && (vis > (int64_t)k || cnt <= k);
  uint32_t n_win = 0;
  if (fast) {
    if ((t & 3) == 0 && sgi < p.esplit) seg_start[sgi] = seg_off;
    if (t == 0) seg_start[p.esplit] = cnt;
    __syncthreads();
    if (sgi < p.esplit) {
      const uint32_t base = seg_start[sgi], n = seg_start[sgi + 1] - base;
#pragma unroll
      for (int i = 0; i < kPfSeg / 4; ++i) {
        const uint32_t slot = 32 * (t & 3) + i;
        if (slot < n) lc[base + slot] = sv[i];
      }
    }
    __syncthreads();
    constexpr int kPer = kPfCap / 256;
    uint64_t key[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const uint32_t g = t + 256 * i;
      key[i] = g < cnt ? lc[g] : 0ull;  // 0 is below every candidate key
    }
    if (t == 0) sh_need = 0;
    if (vis <= (int64_t)k) {  // threshold -inf: the list is every visible key
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (key[i]) win[atomicAdd(&sh_need, 1u)] = select_key_pos(key[i]);
      __syncthreads();
      n_win = sh_need;
    } else {
      // MFMA scores are not binary32-exact (error up to ~2.5e-5 of the sum
      // of |products|): they settle only the clear winners and losers.  Keys
      // within 2^-8 of the MFMA k-th score are rescored exactly on VALU.
      const uint64_t kth_m = block_min_at_least<kPer>(key, block_kth_regs<kPer>(key, k, h2048, wsum, sh3));
      const float sk = key_to_score((uint32_t)(kth_m >> 32));
      const float mg = fabsf(sk) * 0.00390625f;
      const uint32_t lo_key = score_key(sk - mg), hi_key = score_key(sk + mg);
      // keys below the list's threshold are unknown: the band must sit above it
      if (!(sk - mg >= p.thresh[row])) fast = false;
      uint32_t oa = 0, ob = 0, n_band = 0;
      if (fast) {
        // clear winners to win[], band members to bt[]: counts packed as
        // (winners << 16) | band in one scan
        uint32_t na = 0, nb = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const uint32_t s32 = (uint32_t)(key[i] >> 32);
          na += (key[i] != 0ull && s32 > hi_key) ? 1u : 0u;
          nb += (key[i] != 0ull && s32 >= lo_key && s32 <= hi_key) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t packed = (na << 16) | nb;
        const uint32_t off = block_incl_scan_256(packed, wsum, tot) - packed;
        oa = off >> 16;
        ob = off & 0xFFFFu;
        n_win = tot >> 16;
        n_band = tot & 0xFFFFu;
        // every clear winner ranks above the k-th key, so n_win < k <= n_win + n_band
        if (n_win >= k || n_win + n_band < k || n_band > kPfBand) fast = false;
      }
      if (fast) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const uint32_t s32 = (uint32_t)(key[i] >> 32);
          if (key[i] == 0ull) continue;
          if (s32 > hi_key) win[oa++] = select_key_pos(key[i]);
          else if (s32 >= lo_key) bt[ob++] = select_key_pos(key[i]);
        }
        __syncthreads();
        const uint32_t need = k - n_win;
        // exact keys of the band, a lane quad per key
        for (uint32_t base = 0; base < n_band; base += 64) {
          const uint32_t g = base + (t >> 2);
          const bool valid = g < n_band;
          const uint32_t pos = valid ? bt[g] : 0u;
          const float sx = pf_quad_score(q, w, kb, sb, pos, valid, quarter);
          if (valid && quarter == 0) lc[g] = select_key(score_key(sx), pos);  // lc reused for exact keys
        }
        __syncthreads();
        uint64_t bkey[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const uint32_t g = t + 256 * i;
          bkey[i] = g < n_band ? lc[g] : 0ull;
        }
        uint64_t kth_x = 1ull;  // every band key when the band is no larger than what is missing
        if (n_band > need) kth_x = block_kth_regs<kPer>(bkey, need, h2048, wsum, sh3);
        if (t == 0) sh_need = n_win;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          if (bkey[i] != 0ull && bkey[i] >= kth_x) win[atomicAdd(&sh_need, 1u)] = select_key_pos(bkey[i]);
        __syncthreads();
        n_win = sh_need;
      }
    }
  }
  if (fast) {
    if (vis <= (int64_t)kPfBitmapItems) {
      // winners ascending by position through a bitmap (aliasing lc)
      uint32_t* bitmap = reinterpret_cast<uint32_t*>(lc);
      const uint32_t nwords = (uint32_t)((vis + 31) / 32);
      for (uint32_t i = t; i < nwords; i += 256) bitmap[i] = 0u;
      __syncthreads();
      for (uint32_t j = t; j < n_win; j += 256)
        if (win[j] < (uint32_t)vis) atomicOr(&bitmap[win[j] >> 5], 1u << (win[j] & 31u));
      __syncthreads();
      // thread t owns words wpt t .. wpt t + wpt - 1
      constexpr int kMaxWpt = kPfBitmapItems / 32 / 256;
      const uint32_t wpt = (nwords + 255) / 256;
      uint32_t wb[kMaxWpt], cnt_t = 0;
#pragma unroll
      for (int j = 0; j < kMaxWpt; ++j) {
        const uint32_t wi = wpt * t + j;
        wb[j] = (j < (int)wpt && wi < nwords) ? bitmap[wi] : 0u;
        cnt_t += __builtin_popcount(wb[j]);
      }
      uint32_t tot;
      uint32_t o = block_incl_scan_256(cnt_t, wsum, tot) - cnt_t;
      n_win = tot;
#pragma unroll
      for (int j = 0; j < kMaxWpt; ++j) {
        uint32_t bits = wb[j];
        while (bits) {
          const int b = __ffs(bits) - 1;
          out[o++] = (int32_t)((wpt * t + j) * 32 + b);
          bits &= bits - 1;
        }
      }
      for (uint32_t j = n_win + t; j < k; j += 256) out[j] = -1;
    } else {
      // winners ascending by position (bitonic sort, padded to a power of two)
      uint32_t n2 = 1;
      while (n2 < n_win) n2 <<= 1;
      __syncthreads();
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
      for (uint32_t j = t; j < k; j += 256) out[j] = j < n_win ? (int32_t)win[j] : -1;
    }
  } else {
    // ---- exact recompute of this row (rare): radix steps over recomputed keys
    if (t == 0) atomicAdd(p.fallbacks, 1u);
    const uint32_t nv = (uint32_t)vis;
    // visit every visible key: a lane quad per key, 64 keys per step
    auto visit = [&](uint32_t n, auto&& f) {
      for (uint32_t base = 0; base < n; base += 64) {
        const uint32_t pos = base + (t >> 2);
        const bool valid = pos < n;
        const float sx = pf_quad_score(q, w, kb, sb, pos, valid, quarter);
        if (valid && quarter == 0) f(pos, select_key(score_key(sx), pos));
      }
    };
    uint64_t kth = 0;
    if (nv > k) kth = radix_kth(visit, nv, k);
    // winners in position order: each step of 64 keys keeps its order
    uint32_t written = 0;
    for (uint32_t base = 0; base < nv; base += 64) {
      const uint32_t pos = base + (t >> 2);
      const bool valid = pos < nv;
      const float sx = pf_quad_score(q, w, kb, sb, pos, valid, quarter);
      const bool f = valid && quarter == 0 && select_key(score_key(sx), pos) >= kth;
      uint32_t nr;
      const uint32_t o = block_incl_scan_256(f ? 1u : 0u, wsum, nr) - (f ? 1u : 0u);
      if (f && written + o < k) out[written + o] = (int32_t)pos;
      written += nr;
    }
    for (uint32_t j = written + t; j < k; j += 256) out[j] = -1;
  }
}

int prefill_filter_slots(bool has_w) {
  static std::atomic<int> cache[2][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1024;
  int v = cache[has_w][dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int per_cu = 0, n_cu = 0;
  const hipError_t e1 = has_w ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_prefill_mfma<true, true>, 256, 0)
                              : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_prefill_mfma<true, false>, 256, 0);
  const hipError_t e2 = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  v = (e1 == hipSuccess && e2 == hipSuccess && per_cu > 0 && n_cu > 0) ? per_cu * n_cu : 1024;
  cache[has_w][dev].store(v, std::memory_order_relaxed);
  return v;
}

hipError_t launch_prefill_index(const PrefillPass& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  const int tiles = p.batch * p.tiles_per_seq;
  const unsigned grid = (unsigned)(tiles * p.esplit);
  int h = prof_begin(CSA2_K_PREFILL_SAMPLE, stream);
  if (p.idx_w)
    hipLaunchKernelGGL((k_prefill_mfma<false, true>), dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((k_prefill_mfma<false, false>), dim3(grid), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_prefill_threshold, dim3((unsigned)((p.rows + 3) / 4)), dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_end(h, stream);
  h = prof_begin(CSA2_K_PREFILL_FILTER, stream);
  if (p.idx_w)
    hipLaunchKernelGGL((k_prefill_mfma<true, true>), dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((k_prefill_mfma<true, false>), dim3(grid), dim3(256), 0, stream, p);
  prof_end(h, stream);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  h = prof_begin(CSA2_K_PREFILL_SELECT, stream);
  hipLaunchKernelGGL(k_prefill_select, dim3((unsigned)p.rows), dim3(256), 0, stream, p);
  prof_end(h, stream);
  return hipGetLastError();
}

}  // namespace csa2
