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
// ~2^-16).  The layers of a call attend over the same entries, so a
// gathered tile serves a pair of layers: waves 0-1 score one, waves 2-3 the
// other, and every wave updates both layers' O (pair_step).  Three forms:
//   tiles  one tile per workgroup (few rows: decode);
//   pair   a workgroup walks `tiles_per_split` tiles of one row for a pair
//          of layers, one online softmax per layer (many rows: prefill
//          chunks; or a split of a row: multi-token decode);
//   walk   the same for a single layer.
// When a (layer, row) is split over several workgroups, a second kernel
// merges the partial softmaxes in split order, so results do not depend on
// scheduling.
#include "tile.hpp"

namespace csa2 {

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
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[i][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int last_sel = (tile_end < n_tile_idx ? tile_end : n_tile_idx) - 1;  // last selected-entry tile here
  EntryFetch f;
  int32_t pos_next = -1;
  if (tile_begin <= last_sel) {
    fetch_entry<true>(p, seq, tile_position(p, tile_begin, row), f);
    if (tile_begin + 1 <= last_sel) pos_next = tile_position(p, tile_begin + 1, row);
  }
  // the queries, loaded once for the workgroup and staged through E (free
  // again before the first tile goes in)
  stage_q<LG>(p, l0, nl, row, s, qb);
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    if (tile > tile_begin) __syncthreads();  // the previous tile's readers of E are done
    if (tile <= last_sel) {
      store_entry<true>(f, s);
      if (tile + 1 <= last_sel) {
        fetch_entry<true>(p, seq, pos_next, f);
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

// Pair form (many rows, one workgroup per row): workgroup (row, pair of
// layers) walks the row's tiles for two layers at once.  Waves 0-1 score
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

// Tile form (one tile per workgroup, partials merged afterwards): workgroup
// (row, j).  j < n_tile_idx * n_groups: selected-entry tile j / n_groups for
// layer pair j % n_groups (layers 2 g, 2 g + 1): the layers of a group
// attend over the same entries, so a tile is gathered and dequantised once
// for the pair, whose two layers are scored side by side (pair_step);
// otherwise a window tile of one layer (none when the select launch ran
// them: window_elsewhere).
__global__ __launch_bounds__(256) void k_attention_tiles_pair(AttnPass p) {
  const int n_tile_idx = (p.n_idx + kAttnSplit - 1) / kAttnSplit;
  const int n_win_tiles = p.n_tiles - n_tile_idx;
  const int n_groups = (p.n_layers + 1) / 2;
  const int n_sel = n_tile_idx * n_groups;
  const int per_row = n_sel + (p.window_elsewhere ? 0 : p.n_layers * n_win_tiles);
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
  __shared__ __attribute__((aligned(16))) PairLds s;
  if (j < n_sel) {
    const int tile = j / n_groups, l0 = 2 * (j % n_groups);
    const int nl = p.n_layers - l0 < 2 ? p.n_layers - l0 : 2;
    const float sc2 = p.softmax_scale * 1.4426950408889634f;  // logits in the log2 domain
    // the positions and the queries go out together; the entries follow as
    // soon as the positions are in
    const int32_t pos = tile_position(p, tile, row);
    uint4 qb[16];
    EntryFetch f;
    fetch_entry<false>(p, seq, pos, f);
    stage_q_pair(p, l0, nl, row, s, qb);
    store_entry<false>(f, s.t);
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};
    f32x4_t o[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) o[i][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    pair_step(s, qb, nl == 2 ? 3 : 1, sc2, m_run, l_run, o);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i >= nl) break;  // uniform
      write_partial(p, (l0 + i) * p.rows + row, tile, m_run[i], l_run[i], o[i]);
    }
  } else {
    const int jj = j - n_sel;
    window_tile(p, row, jj / n_win_tiles, jj % n_win_tiles, s.t);
  }
}

// Workgroup (pair of layers, row, split): with one split the whole row and
// its outputs; with several, tiles tiles_per_split split .. of the row's
// tile list (selected-entry tiles, then window tiles, each window tile
// index standing for that window tile of both layers) and a partial
// softmax per layer for the merge.
__global__ __launch_bounds__(256, 2) void k_attention_pair(AttnPass p) {
  const int n_pairs = (p.n_layers + 1) / 2;
  const int units = n_pairs * p.rows;
  int unit, split;
  {
    const int lin = blockIdx.x;
    if (units >= kXcds && p.max_splits > 1) {  // the splits of a unit share one XCD
      const int xcd = lin & (kXcds - 1), w = lin >> 3;
      unit = xcd + kXcds * (w / p.max_splits);
      split = w % p.max_splits;
    } else if (units >= kXcds) {
      // each XCD takes a contiguous range of units, so the queries resident
      // on it together are consecutive tokens whose windows overlap in all
      // but one row, and the rows come from its L2
      const int xcd = lin & (kXcds - 1), w = lin >> 3;
      unit = xcd * ((units + kXcds - 1) / kXcds) + w;
      split = 0;
    } else {
      unit = lin / p.max_splits;
      split = lin % p.max_splits;
    }
  }
  if (unit >= units) return;
  const int pair = unit / p.rows, row = unit - pair * p.rows;
  const int l0 = 2 * pair;
  const int nl = p.n_layers - l0 < 2 ? p.n_layers - l0 : 2;
  const int seq = row / p.n_q;
  int n_win;
  const int64_t t0 = window_start(p, row, n_win);
  const int n_tile_idx = (p.n_idx + kAttnSplit - 1) / kAttnSplit;
  const int tile_begin = split * p.tiles_per_split;
  int tile_end = tile_begin + p.tiles_per_split;
  tile_end = tile_end < p.n_tiles ? tile_end : p.n_tiles;
  const int sel_end = tile_end < n_tile_idx ? tile_end : n_tile_idx;  // selected-entry tiles here: tile_begin .. sel_end

  __shared__ __attribute__((aligned(16))) PairLds s;
  TileLds& st = s.t;  // the tile loads fill its E and row_ok
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const float sc2 = p.softmax_scale * 1.4426950408889634f;  // logits in the log2 domain
  uint4 qb[16];
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};
  f32x4_t o[2][8];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[j][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int both = nl == 2 ? 3 : 1;

  EntryFetch f;
  int32_t pos_next = -1;
  if (tile_begin < sel_end) {
    fetch_entry<true>(p, seq, tile_position(p, tile_begin, row), f);
    if (tile_begin + 1 < sel_end) pos_next = tile_position(p, tile_begin + 1, row);
  }
  stage_q_pair(p, l0, nl, row, s, qb);
  for (int tile = tile_begin; tile < sel_end; ++tile) {
    if (tile > tile_begin) __syncthreads();  // the previous tile's readers of E are done
    store_entry<true>(f, st);
    if (tile + 1 < sel_end) {
      fetch_entry<true>(p, seq, pos_next, f);
      if (tile + 2 < sel_end) pos_next = tile_position(p, tile + 2, row);
    }
    pair_step(s, qb, both, sc2, m_run, l_run, o);
  }
  const int win_begin = tile_begin > n_tile_idx ? tile_begin : n_tile_idx;
  for (int j = 0; j < nl; ++j) {
    for (int tile = win_begin; tile < tile_end; ++tile) {
      __syncthreads();  // the previous tile's readers of E are done
      load_window(p, p.layer[l0 + j], tile - n_tile_idx, seq, t0, n_win, st);
      pair_step(s, qb, 1 << j, sc2, m_run, l_run, o);
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j >= nl) break;
    if (p.max_splits > 1) {  // a partial softmax per layer, merged afterwards
      write_partial(p, (l0 + j) * p.rows + row, split, m_run[j], l_run[j], o[j]);
      continue;
    }
    // the whole row is here: write the output
    float l_out[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) l_out[r] = __shfl(l_run[j], 4 * g4 + r, 64);
    float* out = p.layer[l0 + j].out;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int ch = 128 * wave + 16 * nt + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float inv = l_out[r] > 0.0f ? 1.0f / l_out[r] : 0.0f;
        out[((int64_t)row * kH + 4 * g4 + r) * kD + ch] = o[j][nt][r] * inv;
      }
    }
  }
}

// Merge of the split partial softmaxes, in split order.  A kernel of its
// own: the kernel boundary orders the partial writes before these reads on
// every XCD, which in-kernel device-scope fences would do by writing back
// the whole L2.  Workgroup (unit, channel quarter): thread t sums channel
// 128 quarter + t / 2, heads 8 (t % 2) .. +8 (16 contiguous bytes of each
// partial), with per-head weights l_s exp2(m_s - M) / L from the (m, l) of
// every split.  The (m, l) loads go out first and the partial loads of up to
// 16 splits behind them, so the weights are worked out while the partials
// are in flight.  A split's weight carries its up-scale for the quarter.
constexpr int kMaxMergeSplits = 64;
constexpr int kMergeBatch = 16;
// Workgroups run on the XCD that wrote the unit's partials (their lines are
// still in its L2): kMergeByRow, the tile form with 8 or more rows (row r's
// tiles on XCD r mod 8); kMergeByUnit, the walk form with 8 or more units
// (unit u's splits on XCD u mod 8); kMergeLinear otherwise.
enum MergeMap : int32_t { kMergeLinear = 0, kMergeByRow = 1, kMergeByUnit = 2 };
__global__ __launch_bounds__(256) void k_attention_merge(AttnPass p, int32_t map) {
  int unit, quarter;
  if (map == kMergeLinear) {
    unit = blockIdx.x >> 2;
    quarter = blockIdx.x & 3;
  } else {
    const int xcd = blockIdx.x & (kXcds - 1), w = blockIdx.x >> 3, k = w >> 2;
    quarter = w & 3;
    if (map == kMergeByRow) {
      const int rpx = (p.rows + kXcds - 1) / kXcds;  // rows per XCD, at most
      const int layer = k / rpx, row = xcd + kXcds * (k % rpx);
      if (layer >= p.n_layers || row >= p.rows) return;
      unit = layer * p.rows + row;
    } else {
      unit = xcd + kXcds * k;
      if (unit >= p.n_layers * p.rows) return;
    }
  }
  const int layer = unit / p.rows, row = unit - layer * p.rows;
  const int t = threadIdx.x;
  const int ch = 128 * quarter + (t >> 1), h0 = 8 * (t & 1);
  const int ns = p.max_splits;
  const float* pb = p.partial + (int64_t)unit * ns * kPartFloats;
  __shared__ float wgt[kMaxMergeSplits][kH];
  __shared__ float lsh[kMaxMergeSplits][kH];
  // every load is an unconditional buffer load over the unit's partials: a
  // split past the last reads zeros without touching memory, so no branch
  // holds a load back
  const __amdgpu_buffer_rsrc_t rp =
      __builtin_amdgcn_make_buffer_rsrc((void*)pb, 0, ns * kPartFloats * 4, kRawBufferWord3);
  // (split, head) (i / 16, i % 16) for i = t + 256 j: its m and l
  // and the up-scale of this workgroup's channel quarter
  constexpr int kMl = kMaxMergeSplits * kH / 256;
  float mv[kMl], lv[kMl], uv[kMl];
#pragma unroll
  for (int j = 0; j < kMl; ++j) {
    const int i = t + 256 * j;
    const int off = ((i / kH) * kPartFloats + kPartOWords + i % kH) * 4;
    mv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, off, 0, 0));
    lv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, off + kH * 4, 0, 0));
    uv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, off + (2 + quarter) * kH * 4, 0, 0));
  }
  u32x4_t v[kMergeBatch];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rp, (s0 + u) * kPartFloats * 4 + (ch * kH + h0) * 2, 0, 0);
  };
  float acc[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) acc[h] = 0.0f;
  auto accumulate = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      if (s0 + u >= ns) break;
      const uint32_t wd[4] = {v[u][0], v[u][1], v[u][2], v[u][3]};
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const half2_t pr = __builtin_bit_cast(half2_t, wd[h >> 1]);
        acc[h] += wgt[s0 + u][h0 + h] * (float)pr[h & 1];
      }
    }
  };
  load_batch(0);
  if (ns <= 256 / kH) {
    // thread t is (split t / 16, head t % 16), its m and l in mv[0], lv[0]:
    // the per-head max and sum over the splits are shuffles across the
    // wave's four splits and an LDS exchange between the waves
    __shared__ float red_m[4][kH], red_l[4][kH];
    const int lane = t & 63, wave = t >> 6, s_t = t / kH, h_t = t % kH;
    const bool live = s_t < ns;
    const float m = live ? mv[0] : -INFINITY;
    float M = max_xor32(max_xor16(m));
    if (lane < kH) red_m[wave][lane] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red_m[0][h_t], red_m[1][h_t]), fmaxf(red_m[2][h_t], red_m[3][h_t]));
    const float w = m == -INFINITY ? 0.0f : exp2f(m - M) * lv[0];
    float L = sum_xor32(sum_xor16(w));
    if (lane < kH) red_l[wave][lane] = L;
    __syncthreads();
    L = (red_l[0][h_t] + red_l[1][h_t]) + (red_l[2][h_t] + red_l[3][h_t]);
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if (live) wgt[s_t][h_t] = w * inv * uv[0];
  } else {
    __shared__ float ush[kMaxMergeSplits][kH];
#pragma unroll
    for (int j = 0; j < kMl; ++j) {
      const int i = t + 256 * j;
      if (i < ns * kH) {
        wgt[i / kH][i % kH] = mv[j];
        lsh[i / kH][i % kH] = lv[j];
        ush[i / kH][i % kH] = uv[j];
      }
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
      for (int s = 0; s < ns; ++s) wgt[s][t] = wgt[s][t] * inv * ush[s][t];
    }
  }
  __syncthreads();
  accumulate(0);
  for (int s0 = kMergeBatch; s0 < ns; s0 += kMergeBatch) {
    load_batch(s0);
    accumulate(s0);
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
  if (p.tiles_per_split == 1 && p.max_splits == p.n_tiles) {  // (the tile form)
    // one tile per workgroup: a selected-entry tile serves a pair of layers
    // (gathering a tile twice is cheap next to running four layers in one
    // workgroup), scored side by side
    constexpr int LG = 2;
    const int n_groups = (p.n_layers + LG - 1) / LG;
    const int per_row = n_tile_idx * n_groups + (p.window_elsewhere ? 0 : p.n_layers * (p.n_tiles - n_tile_idx));
    const int grows = p.rows >= kXcds ? (p.rows + kXcds - 1) / kXcds * kXcds : p.rows;
    hipLaunchKernelGGL(k_attention_tiles_pair, dim3((unsigned)(grows * per_row)), dim3(256), 0, stream, p);
  } else if (p.n_layers >= 2) {
    // two or more layers: the pair form
    const int punits = (p.n_layers + 1) / 2 * p.rows;
    const int pg = punits >= kXcds ? (punits + kXcds - 1) / kXcds * kXcds : punits;
    hipLaunchKernelGGL(k_attention_pair, dim3((unsigned)(pg * p.max_splits)), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(k_attention<kWalkLG>, dim3((unsigned)(gu * p.max_splits)), dim3(256), 0, stream, p);
  }
  prof_end(h, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_splits == 1) return e;
  if (p.max_splits > kMaxMergeSplits) return hipErrorInvalidValue;
  h = prof_begin(CSA2_K_ATTENTION_MERGE, stream);
  const bool tiles = p.tiles_per_split == 1 && p.max_splits == p.n_tiles;
  const int32_t map = tiles ? (p.rows >= kXcds ? kMergeByRow : kMergeLinear) : (units >= kXcds ? kMergeByUnit : kMergeLinear);
  const int mgrid = map == kMergeByRow ? kXcds * 4 * p.n_layers * ((p.rows + kXcds - 1) / kXcds)
                    : map == kMergeByUnit ? kXcds * 4 * ((units + kXcds - 1) / kXcds)
                                          : 4 * units;
  hipLaunchKernelGGL(k_attention_merge, dim3((unsigned)mgrid), dim3(256), 0, stream, p, map);
  prof_end(h, stream);
  return hipGetLastError();
}

}  // namespace csa2
