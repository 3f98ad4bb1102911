// Internal interface between the host dispatch (api.cpp) and the HIP kernels.
#pragma once

#include "common.hpp"

namespace csa2 {

// Per-sequence scalars travel as kernel arguments (no host-to-device copy, so
// a stream capture records them); a launch covers at most this many sequences.
constexpr int kMaxSeqPerLaunch = 64;
struct SeqArgs {
  int64_t a[kMaxSeqPerLaunch];
  int64_t b[kMaxSeqPerLaunch];
};

// Paged caches: with `pages` set, position j of sequence s is entry
// pages[s * stride + (j >> lg)] * 2^lg + (j mod 2^lg) of the pool the cache
// pointers address (pages of 2^lg entries, 2^lg >= 128); otherwise sequence
// s starts `stride` entries of its own pass after sequence s - 1.  Paged
// accesses go through buffer descriptors over the pool's `pool` entries, so
// an entry past the pool (a bad page index) reads zeros and is not written.
struct PageMap {
  const int32_t* pages;  // device [sequences][stride] or null
  int64_t stride;        // page-table entries between sequences
  int64_t pool;          // entries in the pool (<= CSA2_MAX_ENTRIES)
  int32_t lg;            // log2 of the entries per page
};

// Descriptor over sequence `seq`'s row of the page table: an index past the
// row reads 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_row(const PageMap& m, int seq) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)(m.pages + (int64_t)seq * m.stride), 0, (int)(m.stride * 4),
                                           kRawBufferWord3);
}

// Pool entry of position `pos` given its page's table value, clamped to the
// pool size (which every paged descriptor treats as out of range).
__device__ __forceinline__ uint32_t paged_entry(const PageMap& m, uint32_t page, int64_t pos) {
  const int64_t e = ((int64_t)page << m.lg) | (pos & (((int64_t)1 << m.lg) - 1));
  return e < m.pool && e >= 0 ? (uint32_t)e : (uint32_t)m.pool;
}

// Pool entry of position `pos` of sequence `seq` (one page-table load).
__device__ __forceinline__ uint32_t paged_entry_at(const PageMap& m, int seq, int64_t pos) {
  const uint32_t page = __builtin_amdgcn_raw_buffer_load_b32(page_row(m, seq), (int)((pos >> m.lg) * 4), 0, 0);
  return paged_entry(m, page, pos);
}

// Items scored per workgroup of the indexer scan (a chunk), at most.
constexpr int kScanChunk = 2048;
// Items per scan chunk of a row with n_items items and top-k: the largest
// power of two in [128, kScanChunk] that keeps the expected number of the
// row's winners in one chunk, k * size / n_items, at most kChunkWinners (16
// for k above 1,024).  A row then has at most max(ceil(n / 2048), k / 8 + 1)
// chunks.
__host__ __device__ constexpr int chunk_winners(int k) { return k > 1024 ? 16 : 8; }
__host__ __device__ inline int64_t scan_chunk_items(int64_t n_items, int k) {
  int64_t c = kScanChunk;
  while (c > 128 && (int64_t)k * c > (int64_t)chunk_winners(k) * n_items) c >>= 1;
  return c;
}
// Chunks of a row of n_items items cut into chunks of csize (a power of two).
__host__ __device__ inline int64_t scan_chunk_count(int64_t n_items, int64_t csize) {
  int lg = 0;
  while (((int64_t)1 << lg) < csize) ++lg;
  return (n_items + csize - 1) >> lg;
}
// Chunks per row a workspace must hold for rows of up to max_items items.
inline int64_t scan_max_chunks(int64_t max_items) {
  const int64_t a = (max_items + kScanChunk - 1) / kScanChunk;
  return a > CSA2_MAX_K / 8 + 1 ? a : CSA2_MAX_K / 8 + 1;
}
constexpr int kSeg = 128;
constexpr int kMaxChunks = 4096;
constexpr int kMaxPool = CSA2_N_BLOCKS * CSA2_BLOCK;  // 16,384 positions

// Where the items of an indexer pass come from.
enum ItemSource : int32_t {
  kItemsDirect = 0,  // item i is position i (entry or block id)
  kItemsBlocks = 1,  // item i is position 8*blocks[i/8] + i%8 (hierarchical pool)
  kItemsList = 2,    // item i is position list[i], -1 = empty (candidate pool)
};

// One indexer pass over `rows` query rows (row = seq * n_q + i).
struct IndexPass {
  int32_t rows, n_q, ratio, k;
  int32_t source;
  int32_t key_heads;           // 1: one 64-byte key per entry shared by the heads; 4: per-head keys (256 B)
  // 0: items are positions (or list / block entries); 1: items are blocks
  // scored by their block keys; 2: items are blocks scored by the largest
  // score of their visible positions, read from block_max (a block-max pass)
  int32_t block_level;
  SeqArgs seq;                 // a = q_pos0, b = n_entries (per sequence)
  const uint8_t* idx_q;        // [rows][4][64]
  const float* idx_w;          // [rows][4] or null
  const uint8_t* k8;           // per sequence at + seq*k_stride*64
  const float* kscale;
  int64_t k_stride;
  const int32_t* list;         // kItemsList: [rows][list_len]
  int32_t list_len;
  const int32_t* blocks;       // kItemsBlocks: [rows][CSA2_MAX_K] selected block ids
  const int32_t* nsel;         // kItemsBlocks: [rows] number of selected blocks
  int64_t max_items;           // items per row the grid covers
  // workspace
  uint32_t* fallbacks;         // rows that took the exact recompute (a counter)
  // per (row, chunk): the chunk's two candidate bands (see the scan), as
  // {n0 | ntot << 16, band-0 edge key, band-1 edge key (0: nothing dropped),
  //  largest key scale of the chunk}
  u32x4_t* chunk_info;         // [rows][max_chunks]
  uint64_t* seg_list;          // [rows][max_chunks][kSeg] (score key << 32 | ~item)
  int32_t max_chunks;
  int32_t mfma_scores;         // scores come from fp8 MFMA (queries sharing a scan)
  // block_level 0 with block_max set: the scan also writes each block's
  // largest score key there, and the select the row's largest key scale to
  // row_ksm; a block-max pass reads both
  uint32_t* block_max;         // [rows][block_max_stride]
  int64_t block_max_stride;
  uint32_t* row_ksm;           // [rows] float bits
  // output: either positions (out, -1 padded to k) or block ids + count
  int32_t* out;                // [rows][out_stride]
  int32_t out_stride;
  int32_t* out_count;          // [rows] or null
  int32_t* out_pool;           // optional: pool positions of the kept blocks
  int32_t pool_stride;
  PageMap pm;                  // paged k8 / kscale (direct items over entries only)
};

// Kernel classes of the optional timing records (csa2_profile_*).
int prof_begin(int32_t kernel, hipStream_t stream);
void prof_end(int handle, hipStream_t stream);
void prof_suspend(bool on);  // while on, this thread's launches are not timed

// One decode step's appends: sequence s writes its token at position
// seq.a[s] (see csa2_append).
struct AppendPass {
  int32_t ratio;
  SeqArgs seq;                  // a = position of the new token
  const float* x;               // [batch][512]
  const float* k_in;            // [batch][64]
  uint8_t* nib;
  uint8_t* scale;
  uint8_t* k8;
  float* kscale;
  int64_t stride;
  uint8_t* bk8;                 // or null
  float* bks;
  int64_t bk_stride;
  float* pending;               // ratio 2: [batch][576]
  uint16_t* swa;                // or null
  int64_t swa_stride, swa_ring;
  PageMap pm;                   // paged nib / scale / k8 / kscale
};
hipError_t launch_append(const AppendPass& p, int32_t batch, hipStream_t stream);

hipError_t launch_quantize(const float* x, int64_t n_entries, int64_t ld_x, int32_t ratio,
                           uint8_t* nib, uint8_t* scale, const float* kin, int64_t ld_k,
                           uint8_t* k8, float* kscale, hipStream_t stream);
hipError_t launch_quantize_head_keys(const float* kin, int64_t n_entries, int64_t ld_k, int32_t ratio, uint8_t* k8,
                                     float* kscale, hipStream_t stream);
hipError_t launch_block_keys(const uint8_t* k8, const float* ks, int64_t k_stride,
                             const int64_t* n_entries, int32_t batch, uint8_t* bk8, float* bks,
                             int64_t bk_stride, hipStream_t stream);
struct AttnPass;
// `attn`, if given, is the tile-form attention pass of the group the index
// pass serves: the select launch may run all of its tiles
// (k_index_select_attend), and *attended then says whether it did (only the
// merge is left).
hipError_t launch_index_pass(const IndexPass& p, hipStream_t stream, const AttnPass* attn = nullptr,
                             bool* attended = nullptr);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t stream);

// Attention over the candidates of each row for one or more layers that
// share the KV and the index lists.
struct AttnLayer {
  const uint16_t* q;    // [rows][16][512]
  const uint16_t* swa;  // per sequence at + seq*swa_stride*512
  float* out;           // [rows][16][512]
};
constexpr int kMaxAttnLayers = 8;
constexpr int kAttnSplit = 64;  // candidates per workgroup
// A partial softmax, in 4-byte words: O / l as [512 channels][16 heads] fp16
// (normalised, so every value is a convex combination of value rows), then
// m[16] and l[16] as float32, then up[4][16]: the fp16 values of channel
// quarter c (channels 128 c .. 128 c + 127) of head h are O / l times
// 1 / up[c][h], a power of two (1 unless the quarter's largest magnitude is
// 2^15 or more, as window rows of large values give), so fp16 holds every
// value in range.
constexpr int kPartOWords = kD * kH / 2;
constexpr int kPartUp = kPartOWords + 2 * kH;
constexpr int kPartFloats = kPartUp + 4 * kH;
struct AttnPass {
  int32_t rows, n_q, n_idx, n_layers;
  SeqArgs seq;                  // a = q_pos0, b = swa_pos0
  const uint8_t* nib;
  const uint8_t* scale;
  int64_t kv_stride;
  const int32_t* idx;           // [rows][n_idx]
  int64_t swa_stride;
  float softmax_scale;
  AttnLayer layer[kMaxAttnLayers];
  int32_t n_tiles;              // candidate tiles of kAttnSplit rows per (layer, row)
  int32_t tiles_per_split;      // tiles one workgroup walks (online softmax)
  int32_t max_splits;           // ceil(n_tiles / tiles_per_split)
  int64_t swa_ring;             // 0: linear window rows from seq.b; > 0: token t at row t mod swa_ring
  int32_t tiles_elsewhere;      // tile form: every tile ran in the select launch; only the merge is left
  PageMap pm;                   // paged nib / scale
  // workspace (used when max_splits > 1)
  float* partial;               // [n_layers*rows][max_splits][kPartFloats]
};
hipError_t launch_attention(const AttnPass& p, hipStream_t stream);

// Prefill chunk indexer (fp8 MFMA): used for FLAT indexing of calls with at
// least kPrefillMinQ queries per sequence.
constexpr int kPrefillMinQ = 32;
constexpr int kPfRows = 256;      // query rows per workgroup
constexpr int kPfSample = 2048;   // sampled keys per row tile
constexpr int kPfCap = 4096;      // candidates a row's selection holds in LDS
constexpr int kPfSplits = 64;     // key ranges (filter workgroups) per row tile, at most
constexpr int kPfSeg = 128;       // candidates kept per (row, key range)
constexpr int kPfBitmapItems = 1 << 18;  // rows with at most this many visible keys order winners by bitmap
struct PrefillPass {
  int32_t rows, n_q, ratio, k, batch;
  int32_t tiles_per_seq, esplit;
  SeqArgs seq;                   // a = q_pos0, b = n_entries
  const uint8_t* idx_q;          // [rows][4][64]
  const float* idx_w;            // [rows][4] or null
  const uint8_t* k8;
  const float* kscale;
  int64_t k_stride;
  // workspace
  float* sample;                 // [rows][kPfSample]
  float* thresh;                 // [rows]
  uint32_t* fallbacks;           // rows that took the exact recompute (a counter)
  uint32_t* count;               // [rows][kPfSplits] candidates per segment
  uint64_t* list;                // [rows][kPfSplits][kPfSeg] (position, score bits) pairs
  int32_t* out;                  // [rows][out_stride]
  int32_t out_stride;
};
hipError_t launch_prefill_index(const PrefillPass& p, hipStream_t stream);
// Filter workgroups resident on the current device at once (CUs x
// workgroups per CU for the filter variant with or without head weights);
// the key split of a prefill chunk is sized to fill them in one round.
int prefill_filter_slots(bool has_w);

}  // namespace csa2
