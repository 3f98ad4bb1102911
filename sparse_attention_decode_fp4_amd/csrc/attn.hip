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

// Tile form (one tile per workgroup, partials merged afterwards): workgroup
// (row, j).  j < n_tile_idx * n_groups: selected-entry tile j / n_groups for
// layer pair j % n_groups (layers 2 g, 2 g + 1): the layers of a group
// attend over the same entries, so a tile is gathered and dequantised once
// for the pair, whose two layers are scored side by side (pair_step);
// otherwise a window tile of one layer.  (A decode group's index pass runs
// all of these in its select launch instead: k_index_select_attend.)
__global__ __launch_bounds__(256) void k_attention_tiles_pair(AttnPass p) {
  const int n_tile_idx = (p.n_idx + kAttnSplit - 1) / kAttnSplit;
  const int n_win_tiles = p.n_tiles - n_tile_idx;
  const int n_groups = (p.n_layers + 1) / 2;
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
  const bool tiles_here = !(p.tiles_elsewhere && p.tiles_per_split == 1 && p.max_splits == p.n_tiles);
  int h = tiles_here ? prof_begin(CSA2_K_ATTENTION, stream) : -1;
  const int n_tile_idx = (p.n_idx + kAttnSplit - 1) / kAttnSplit;
  if (p.tiles_per_split == 1 && p.max_splits == p.n_tiles) {  // (the tile form)
    // one tile per workgroup: a selected-entry tile serves a pair of layers
    // (gathering a tile twice is cheap next to running four layers in one
    // workgroup), scored side by side
    constexpr int LG = 2;
    const int n_groups = (p.n_layers + LG - 1) / LG;
    const int per_row = n_tile_idx * n_groups + p.n_layers * (p.n_tiles - n_tile_idx);
    const int grows = p.rows >= kXcds ? (p.rows + kXcds - 1) / kXcds * kXcds : p.rows;
    if (tiles_here)
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
