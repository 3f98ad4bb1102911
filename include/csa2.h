/*
 * libcsa2: the CSA2 compressed-sparse-attention step with an FP4 KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * The step, as five public news pages about DeepSeek-V4.1-Flash describe it:
 *   - the main KV cache holds one latent per position as E2M1 values with one
 *     E4M3 scale per 16 channels and no global scale (ai-wave.ru, "DeepSeek
 *     V4.1-Flash: 1M context, FP4 KV cache and an attention-reuse
 *     architecture", fourth paragraph; agentnet.co.il, "DeepSeek launches
 *     V4.1-Flash ...", section "Quantization and deployment");
 *   - an indexer scores the positions and keeps 512 of them, directly or
 *     through a hierarchical pool of at most 2,048 blocks of 8 positions
 *     (agentnet.co.il, section "CSA2: compression along the layer axis");
 *   - attention runs over the kept entries plus a 128-token sliding window
 *     (ai-wave.ru, second paragraph);
 *   - every layer has a fixed mode: Full, Reindex or Reuse (agentnet.co.il,
 *     section "CSA2: compression along the layer axis").
 *
 * Conventions for every call:
 *   - Pointers documented as "device" point to GPU memory the caller owns;
 *     pointers documented as "host" point to host memory read during the
 *     call only.  The library never allocates or frees caller memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; the library never synchronises.
 *   - Every argument is validated before anything is enqueued.  On an error
 *     nothing is launched, no output is written, and a non-zero status is
 *     returned; csa2_last_error() then gives a message (thread-local).
 *   - Scratch memory comes from a caller-provided workspace of at least
 *     csa2_workspace_bytes() bytes, 256-byte aligned.  Calls that share a
 *     workspace must be ordered on one stream.
 *   - Non-finite inputs are outside the contract.
 *   - Results are deterministic: partial results are combined in a fixed
 *     order, independent of scheduling.
 *   - Layout: bf16 tensors are passed as uint16_t bit patterns.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 4

/* Model constants the kernels are built for. */
#define CSA2_D_LATENT 512   /* channels of one main-KV latent (key = value)        */
#define CSA2_SCALE_GROUP 16 /* channels sharing one E4M3 scale                     */
#define CSA2_NIB_BYTES 256  /* packed E2M1 bytes per entry                          */
#define CSA2_SCALE_BYTES 32 /* E4M3 scale bytes per entry                           */
#define CSA2_D_INDEX 64     /* channels of the fp8 indexer key / query per head     */
#define CSA2_H_INDEX 4      /* indexer heads                                        */
#define CSA2_H_ATTN 16      /* attention heads                                      */
#define CSA2_TOP_K 512      /* entries kept per query                               */
#define CSA2_SWA 128        /* sliding-window length in tokens                      */
#define CSA2_BLOCK 8        /* positions per hierarchical block                     */
#define CSA2_N_BLOCKS 2048  /* blocks kept by the hierarchical indexer              */
#define CSA2_MAX_K 2048     /* largest k accepted by csa2_index_topk                */
#define CSA2_MAX_ENTRIES 8388607 /* cache entries per sequence, at most (2^23 - 1)  */

/* Status codes. */
#define CSA2_OK 0
#define CSA2_ERR_ARG 1         /* a null, misaligned or inconsistent argument       */
#define CSA2_ERR_UNSUPPORTED 2 /* a size or mode the kernels are not built for      */
#define CSA2_ERR_STATE 3       /* Reindex/Reuse with no Full layer in the state     */
#define CSA2_ERR_WORKSPACE 4   /* workspace missing or too small                    */
#define CSA2_ERR_HIP 5         /* a HIP launch failed; see csa2_last_error()        */

/* Indexer kinds. */
#define CSA2_INDEX_FLAT 0 /* score every visible position                           */
#define CSA2_INDEX_HIER 1 /* blocks first, then positions inside the kept blocks    */
#define CSA2_INDEX_POOL 2 /* score only a given candidate pool                      */
#define CSA2_INDEX_FLAT_POOL 3 /* FLAT, and a pool of the blocks its scores rank highest */

/* Layer modes. */
#define CSA2_MODE_FULL 0
#define CSA2_MODE_REINDEX 1
#define CSA2_MODE_REUSE 2

/* Version of this interface (CSA2_ABI_VERSION); no side effects. */
int csa2_abi_version(void);

/* Message of the last failed call on this thread ("" if none); owned by the
 * library, valid until the next call on this thread. */
const char* csa2_last_error(void);

/* sizeof() of the argument structs, for bindings to check their layouts:
 * 0 index_args, 1 attn_args, 2 kv, 3 layer, 4 group_state, 5 group_args,
 * 6 append_args, 7 pages; 0 for anything else. */
size_t csa2_struct_size(int32_t which);

/*
 * Encode tokens into cache entries (the FP4 main-KV encoder, and optionally
 * the fp8 indexer key).
 *
 * Entry j is built from tokens ratio*j .. ratio*j+ratio-1; at ratio 2 it is
 * their float32 mean fp32(fp32(a+b)*0.5) (globalfeed.ai, "DeepSeek-V4.1-Flash
 * released ...", section "What changed in the architecture", gives ratio 2
 * for the encoder layers; the mean is a reading).
 *
 * Main KV (ai-wave.ru fourth paragraph; agentnet.co.il section "Quantization
 * and deployment"): per 16-channel block, scale S = E4M3 nearest to amax/6
 * (ties to even, saturating at 448); each element code = E2M1 nearest to x/S
 * (ties to even, saturating at 6, sign bit = sign of x); S == 0 gives code 0.
 * Byte i of an entry's 256 bytes holds channel 2i (low nibble) and channel
 * 2i+1 (high nibble); scale j covers channels 16j..16j+15.
 *
 * Indexer key (a reading; agentnet.co.il section "CSA2: compression along the
 * layer axis" says Full layers project an indexer K): ks = fp32(amax/448),
 * code = E4M3 nearest to fp32(k/ks) (ties to even, saturating); amax == 0
 * gives ks = 0 and codes 0.
 *
 *   x      device float32 [n_tok][ld_x], 16-byte aligned, ld_x a multiple of 4
 *          and >= 512; the first 512 columns are used
 *   n_tok  tokens (>= 0, a multiple of ratio); 0 enqueues nothing
 *   ratio  1 or 2
 *   nib    device uint8 [n_tok/ratio][256], 16-byte aligned   (out)
 *   scale  device uint8 [n_tok/ratio][32]    (out)
 *   k_in   device float32 [n_tok][ld_k] or NULL (then k8/kscale are ignored)
 *   k8     device uint8 [n_tok/ratio][64], 16-byte aligned    (out)
 *   kscale device float32 [n_tok/ratio]      (out)
 * Errors: CSA2_ERR_ARG for null pointers, bad leading dimensions, bad ratio,
 * n_tok not a multiple of ratio, or misaligned pointers.
 */
int csa2_quantize_kv(const float* x, int64_t n_tok, int64_t ld_x, int32_t ratio,
                     uint8_t* nib, uint8_t* scale,
                     const float* k_in, int64_t ld_k, uint8_t* k8, float* kscale,
                     void* stream);

/*
 * Block keys of the hierarchical indexer (agentnet.co.il, section "CSA2:
 * compression along the layer axis": blocks of 8 positions).  A reading:
 * block b of a sequence is the float32 mean of the dequantised keys
 * fp32(e4m3(code) * ks) of its entries 8b..8b+7 (fewer for a trailing partial
 * block), summed in position order and divided by their count, then encoded
 * like an indexer key.
 *
 *   k8, kscale   device: sequence s starts at k8 + s*k_stride*64 and
 *                kscale + s*k_stride
 *   batch        sequences (>= 0); n_entries[s] (host int64 [batch]) entries each
 *   bk8, bkscale device out: sequence s at bk8 + s*bk_stride*64 and
 *                bkscale + s*bk_stride; ceil(n_entries[s]/8) blocks each
 * Errors: CSA2_ERR_ARG for null pointers, negative sizes, strides smaller
 * than the data they hold.
 */
int csa2_build_block_keys(const uint8_t* k8, const float* kscale, int32_t batch,
                          const int64_t* n_entries, int64_t k_stride,
                          uint8_t* bk8, float* bkscale, int64_t bk_stride,
                          void* stream);

/*
 * Per-head indexer keys (the other reading of the key layout: each of the 4
 * indexer heads has its own 64-channel key).  One
 * entry's key is quantised as one 256-value vector, with the rule of
 * csa2_quantize_kv's key: ks = fp32(amax / 448) over all four heads, codes
 * E4M3(fp32(k / ks)) (round to nearest even, saturating); at ratio 2 the
 * pair mean is taken first.  Head h of entry e is at k8 + e*256 + h*64.
 * Scores then dot head h's query with head h's key:
 *   s = ks * sum_h w_h * max(0, q_h . k_h).
 *   k_in    device float32 [n_tok][ld_k], ld_k >= 256 (4 heads x 64 channels)
 *   k8      device [n_tok / ratio][256] (out);  kscale  device float32 [n_tok / ratio] (out)
 * Errors: CSA2_ERR_ARG for null or misaligned pointers, a bad ratio or
 * ld_k, or n_tok not a multiple of ratio.
 */
int csa2_quantize_head_keys(const float* k_in, int64_t n_tok, int64_t ld_k, int32_t ratio,
                            uint8_t* k8, float* kscale, void* stream);

/*
 * Paged caches (for serving: a pool of fixed-size pages and a page table per
 * sequence, so sequences grow without a fixed stride).  With table set,
 * position j of sequence s is pool entry
 *   table[s*table_stride + j/page_size] * page_size + j % page_size
 * of nib/scale/k8/kscale (each laid out as one [pool_entries] array), and
 * the per-sequence strides of those arrays are not read.  Block keys (HIER)
 * stay per-sequence arrays.  Paged caches serve the decode path: FLAT
 * indexing with n_q < 32 (csa2_index_topk, csa2_run_group), attention and
 * csa2_append; HIER, POOL and prefill-sized calls return
 * CSA2_ERR_UNSUPPORTED with a table.  Results are those of the same cache
 * laid out contiguously, bit for bit.
 *   table         device int32 [batch][table_stride]: page indices; the
 *                 caller guarantees one for every page a sequence's entries
 *                 (and an append's new entry) fall in.  Indices are not
 *                 checked on the host; an entry they place at or past
 *                 pool_entries reads as zeros and is not written
 *   table_stride  entries between sequences' table rows (>= the pages of the
 *                 longest sequence; <= 65,536)
 *   page_size     entries per page: a power of two, 128 .. 65,536
 *   pool_entries  entries in the pool, 1 .. CSA2_MAX_ENTRIES
 * A zero table means a contiguous cache (the other fields are then unused).
 */
typedef struct csa2_pages {
  const int32_t* table;
  int64_t table_stride;
  int64_t pool_entries;
  int32_t page_size;
} csa2_pages;

/*
 * Indexer + top-k (agentnet.co.il, section "CSA2: compression along the
 * layer axis": a Full layer picks 512 fresh positions; Reindex ranks with its
 * own indexer Q; the hierarchical indexer builds a pool of 2,048 blocks of 8).
 *
 * Score (a reading, the pages give no formula):
 *   s_p = ks_p * sum_h w_h * max(0, q_h . k_p),   h = 0..3, 64 channels,
 * q_h and k_p being E4M3 code values.  Scores are computed in float32 on the
 * GPU.  With n_q < 32, keys whose float32 scores lie within the float32
 * error bound of the k-th are rescored exactly (float64: every product of
 * E4M3 codes and every partial sum of 64 is exact there) and ranked on those
 * exact scores, so the selected set is the one the exact scores give; with
 * n_q >= 32 a band around the MFMA k-th score is rescored in float32.
 * Selection: score descending, then position ascending; the min(k, n)
 * winners are written in ascending position order, padded with -1.
 *
 * Visibility: query i of sequence s is at token position q_pos0[s] + i and
 * sees entries j < min(n_entries[s], (pos + 1) / ratio).
 *
 * FLAT scores every visible entry.  HIER scores the visible blocks (block
 * keys), keeps the top n_blocks blocks, and scores the visible positions of
 * those blocks; out_pool (optional) receives the kept positions in ascending
 * order, -1 padded.  POOL scores only the positions in cand, which must be
 * ascending with any -1 padding at the end.  FLAT_POOL is FLAT (the same
 * out_idx) that also keeps a pool, the other reading of the same section:
 * block b (positions 8b .. 8b+7) scores the largest score among its visible
 * positions, the top n_blocks blocks are kept (score descending, then lower
 * block; near-ties settled on exact scores as above), and out_pool
 * (required) receives their visible positions as for HIER.  With n_q >= 32
 * (a prefill chunk) FLAT scoring runs on fp8 MFMA; HIER, POOL and FLAT_POOL
 * then return CSA2_ERR_UNSUPPORTED.
 */
typedef struct csa2_index_args {
  int32_t kind;              /* CSA2_INDEX_*                                          */
  int32_t batch;             /* sequences, >= 1                                       */
  int32_t n_q;               /* queries per sequence, >= 1                            */
  int32_t ratio;             /* 1 or 2                                                */
  const int64_t* q_pos0;     /* host [batch] token position of each sequence's query 0 */
  const int64_t* n_entries;  /* host [batch] entries present per sequence             */
  const uint8_t* idx_q;      /* device [batch][n_q][4][64] E4M3 codes                 */
  const float* idx_w;        /* device [batch][n_q][4] or NULL (all weights 1)        */
  const uint8_t* k8;         /* device, sequence s at k8 + s*k_stride*64              */
  const float* kscale;       /* device, sequence s at kscale + s*k_stride             */
  int64_t k_stride;          /* entries between sequences                             */
  const uint8_t* bk8;        /* HIER: device block codes, sequence s at + s*bk_stride*64 */
  const float* bkscale;      /* HIER: device block scales                             */
  int64_t bk_stride;         /* HIER: blocks between sequences                        */
  const int32_t* cand;       /* POOL: device [batch][n_q][n_cand] positions, -1 = none */
  int32_t n_cand;            /* POOL: candidates per query, 1..16384                  */
  int32_t k;                 /* entries kept per query, 1..CSA2_MAX_K (512 normally)  */
  int32_t n_blocks;          /* HIER, FLAT_POOL: blocks kept, 1..CSA2_MAX_K (2048 normally) */
  int32_t* out_idx;          /* device [batch][n_q][k] (out)                          */
  int32_t* out_pool;         /* HIER, FLAT_POOL: device [batch][n_q][n_blocks*8] (out; optional for HIER) */
  csa2_pages pages;          /* paged k8/kscale (FLAT with n_q < 32), or all zero     */
  int32_t key_heads;         /* indexer-key layout: 0 or 1 shared key (64 B / entry),
                                4 per-head keys (256 B / entry, see
                                csa2_quantize_head_keys): FLAT, FLAT_POOL and POOL
                                with n_q < 32, contiguous caches                      */
} csa2_index_args;

int csa2_index_topk(const csa2_index_args* a, void* workspace, size_t ws_bytes, void* stream);

/*
 * Sparse + sliding-window attention (ai-wave.ru second paragraph: every layer
 * keeps a 128-token window; news.hamidun.com "... 890 bytes per token instead
 * of 3514", section "Three memory-saving mechanisms": layers read the shared
 * FP4 cache).  Readings: the latent is both key and value; the window is a
 * separate bf16 buffer of raw token rows; a query at token p sees the rows of
 * tokens max(0, p-127)..p and the selected entries in one softmax, without
 * removing overlaps.  For head h:
 *   out_h = sum_i softmax_i(scale * q_h . e_i) e_i
 * with e_i the dequantised entries (exact in bf16) and window rows; products
 * accumulate in float32.
 *
 *   q         device bf16 [batch][n_q][16][512]
 *   nib/scale device, sequence s at nib + s*kv_stride*256, scale + s*kv_stride*32
 *   idx       device int32 [batch][n_q][n_idx], -1 = unused; each must be
 *             < the entries present and < CSA2_MAX_ENTRIES (not checked on
 *             the device)
 *   swa       device bf16, sequence s at swa + s*swa_stride*512.  Linear
 *             (swa_ring = 0): row r holds token swa_pos0[s] + r, swa_rows rows
 *             present.  Ring (swa_ring > 0, as csa2_append writes it): token
 *             t is row t mod swa_ring; swa_pos0 and swa_rows are not read, and
 *             the caller guarantees the rows of every token a query sees hold
 *             that token (swa_ring >= n_q + 127 so they are distinct rows)
 *   out       device float32 [batch][n_q][16][512] (out)
 * Errors: CSA2_ERR_ARG when a window row a query needs is not in the buffer
 * (linear), or swa_ring is below n_q + 127 or not below 2^21 (ring).
 */
typedef struct csa2_attn_args {
  int32_t batch, n_q, n_idx;  /* n_idx 0..CSA2_MAX_K                                 */
  const int64_t* q_pos0;      /* host [batch]                                         */
  const uint16_t* q;
  const uint8_t* nib;
  const uint8_t* scale;
  int64_t kv_stride;          /* entries between sequences                            */
  const int32_t* idx;
  const uint16_t* swa;
  int64_t swa_stride;         /* rows between sequences                               */
  const int64_t* swa_pos0;    /* host [batch]                                         */
  int64_t swa_rows;           /* rows present per sequence                            */
  float softmax_scale;
  float* out;
  int64_t swa_ring;           /* 0: linear window rows; > 0: ring of this many rows   */
  csa2_pages pages;           /* paged nib/scale, or all zero                         */
} csa2_attn_args;

int csa2_sparse_swa_attn(const csa2_attn_args* a, void* workspace, size_t ws_bytes, void* stream);

/*
 * The static layer plan (agentnet.co.il, section "CSA2: compression along the
 * layer axis"; tgviewer.app sof_news24 "DeepSeek V4.1 Flash: new architecture
 * ...", section "Layers no longer store everything independently"):
 *   FULL    takes its own encoded KV (kv), indexes it with its own indexer Q,
 *           and records {kv, indices} in the state;
 *   REINDEX indexes the state's KV with its own indexer Q (the reading of two
 *           pages; a third says it keeps the indices) and records the indices;
 *   REUSE   attends with the state's KV and latest indices, no indexer.
 * Every layer then runs csa2_sparse_swa_attn with its own q and window rows.
 * The state persists across calls; Reindex/Reuse with no Full in the state
 * return CSA2_ERR_STATE.  With index_kind HIER the Full layer uses the
 * hierarchical indexer and stores its pool; with FLAT_POOL it indexes flat
 * and stores the pool of the blocks its token scores rank highest (both
 * need state.pool).  reindex_kind POOL makes Reindex rank only that pool; a
 * Full layer that stores no pool drops the state's earlier pool.
 */
typedef struct csa2_kv {
  const uint8_t* nib;      /* device, sequence s at + s*stride*256                    */
  const uint8_t* scale;    /* device, sequence s at + s*stride*32                     */
  const uint8_t* k8;       /* device, sequence s at + s*stride*64                     */
  const float* kscale;     /* device, sequence s at + s*stride                        */
  int64_t stride;          /* entries between sequences                               */
  const uint8_t* bk8;      /* device block keys (HIER), sequence s at + s*bk_stride*64 */
  const float* bkscale;
  int64_t bk_stride;       /* blocks between sequences                                */
  csa2_pages pages;        /* paged nib/scale/k8/kscale (stride unused), or all zero  */
  int32_t key_heads;       /* indexer-key layout, as csa2_index_args.key_heads        */
} csa2_kv;

typedef struct csa2_layer {
  int32_t mode;            /* CSA2_MODE_*                                             */
  const uint16_t* q;       /* device bf16 [batch][n_q][16][512]                       */
  const uint16_t* swa;     /* device bf16, layout as in csa2_attn_args               */
  const uint8_t* idx_q;    /* FULL/REINDEX: device [batch][n_q][4][64]                */
  const float* idx_w;      /* FULL/REINDEX: device [batch][n_q][4] or NULL            */
  const csa2_kv* kv;       /* FULL: host pointer to the layer's KV                    */
  float* out;              /* device float32 [batch][n_q][16][512] (out)              */
} csa2_layer;

typedef struct csa2_group_state {
  csa2_kv kv;              /* KV of the last Full layer                               */
  int32_t* indices;        /* caller-owned device [batch][n_q][512]                   */
  int32_t* pool;           /* caller-owned device [batch][n_q][n_blocks*8] or NULL    */
  int32_t has_full, has_indices, has_pool;
  int32_t batch, n_q;      /* shape the indices were made for                         */
} csa2_group_state;

typedef struct csa2_group_args {
  int32_t batch, n_q, ratio;
  int32_t index_kind;      /* CSA2_INDEX_FLAT, _HIER or _FLAT_POOL for Full layers    */
  int32_t reindex_kind;    /* CSA2_INDEX_FLAT or CSA2_INDEX_POOL for Reindex layers   */
  const int64_t* q_pos0;   /* host [batch]                                            */
  const int64_t* n_entries;/* host [batch]                                            */
  const int64_t* swa_pos0; /* host [batch]                                            */
  int64_t swa_stride, swa_rows;
  float softmax_scale;
  int32_t n_layers;
  const csa2_layer* layers;/* host [n_layers]                                         */
  int64_t swa_ring;        /* window layout of every layer, as in csa2_attn_args      */
} csa2_group_args;

int csa2_run_group(const csa2_group_args* a, csa2_group_state* state,
                   void* workspace, size_t ws_bytes, void* stream);

/*
 * csa2_run_group for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, hosts that forbid hipMalloc.  It
 * takes no workspace and allocates nothing; it works in a scratch array of
 * CSA2_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs
 * on, from the first call on that device until the process ends.  Arguments,
 * state, outputs and errors are those of csa2_run_group, and so are the
 * results, bit for bit.  The call uses the scratch of the current device
 * (the stream must belong to it).  All calls on one device share that
 * device's scratch, which keeps the last call's contents: calls that may
 * overlap on one device (other streams, other threads) race, and the caller
 * must order them.  Nothing in the scratch has to start at zero (a call
 * writes everything it reads).  Calls are not timed by csa2_profile_*.
 * Size: decode steps of up to about 16 sequences x 131,072 entries with up
 * to four layers per Full/Reindex layer need about 15 MiB.  Errors: those of
 * csa2_run_group, and CSA2_ERR_UNSUPPORTED when the call needs more than
 * CSA2_NOALLOC_SCRATCH_BYTES (csa2_last_error() gives both figures).
 */
#define CSA2_NOALLOC_SCRATCH_BYTES (32u << 20)
int csa2_run_group_noalloc(const csa2_group_args* a, csa2_group_state* state, void* stream);

/*
 * The write side of one decode step: one new token per sequence goes into
 * the caches the read side uses.  The cache format is the one
 * csa2_quantize_kv writes (ai-wave.ru "DeepSeek V4.1-Flash: 1M context, FP4
 * KV cache ...", fourth paragraph); at ratio 2 two tokens make one entry
 * (globalfeed.ai "DeepSeek-V4.1-Flash released ...", section "What changed
 * in the architecture"; the pair mean is a reading); block keys cover 8
 * entries (agentnet.co.il "DeepSeek launches V4.1-Flash ...", section
 * "CSA2: compression along the layer axis"); the window keeps the last 128
 * tokens uncompressed (ai-wave.ru, second paragraph).  For sequence s and
 * its new token at position pos[s]:
 *   ratio 1   entry pos is encoded from x, k_in;
 *   ratio 2   an even pos is held in pending; an odd pos completes entry
 *             (pos-1)/2 from the pair mean fp32(fp32(held + new) * 0.5);
 *   blocks    with kv.bk8 set, the block holding a new entry is re-derived
 *             from its entries present (a trailing block averages those);
 *   window    with swa set, bf16(x) (round to nearest even) goes to row
 *             pos mod swa_ring.
 * Results equal csa2_quantize_kv / csa2_build_block_keys over the whole
 * token history, byte for byte, when tokens are appended in position order
 * (entries 8*(e/8) .. e-1 of a block must be in the cache before entry e).
 *   x          device float32 [batch][512], the new tokens' latents
 *   k_in       device float32 [batch][64], their indexer keys
 *   nib..kscale  device cache to write, laid out as csa2_kv (all four
 *              required); entry e of sequence s must be < stride and
 *              < CSA2_MAX_ENTRIES
 *   bk8, bkscale device block keys, as csa2_kv, or NULL
 *   pending    ratio 2: device float32 [batch][576] (latent, then key) that
 *              holds an even token until its pair arrives; caller-owned
 *   swa        device bf16 or NULL: sequence s's ring at swa + s*swa_stride*512
 *              (swa_stride >= swa_ring >= 128 when batch > 1)
 * Errors: CSA2_ERR_ARG for missing pointers, negative positions, entries
 * past stride, a ring under 128 rows; CSA2_ERR_UNSUPPORTED for entries at
 * or past CSA2_MAX_ENTRIES; CSA2_ERR_HIP for launch failures.
 */
typedef struct csa2_append_args {
  int32_t batch, ratio;       /* ratio 1 or 2                                         */
  const int64_t* pos;         /* host [batch]: position of each new token             */
  const float* x;
  const float* k_in;
  uint8_t* nib;               /* device, sequence s at + s*stride*256                 */
  uint8_t* scale;             /* device, sequence s at + s*stride*32                  */
  uint8_t* k8;                /* device, sequence s at + s*stride*64                  */
  float* kscale;              /* device, sequence s at + s*stride                     */
  int64_t stride;             /* entries between sequences                            */
  uint8_t* bk8;               /* device or NULL, sequence s at + s*bk_stride*64       */
  float* bkscale;
  int64_t bk_stride;          /* blocks between sequences                             */
  float* pending;
  uint16_t* swa;
  int64_t swa_stride;         /* rows between sequences                               */
  int64_t swa_ring;           /* ring rows per sequence (>= 128)                      */
  csa2_pages pages;           /* paged nib/scale/k8/kscale (stride unused), or all zero */
} csa2_append_args;

int csa2_append(const csa2_append_args* a, void* stream);

/*
 * Workspace bytes sufficient for any call with at most max_batch sequences,
 * max_n_q queries per sequence and max_entries entries per sequence
 * (returns 0 for invalid sizes).
 */
size_t csa2_workspace_bytes(int32_t max_batch, int32_t max_n_q, int64_t max_entries);

/*
 * Zero a workspace (optional: every call initialises what it reads; it also
 * resets csa2_workspace_fallbacks).
 *   workspace  device, 256-byte aligned;  ws_bytes  a multiple of 4
 */
int csa2_workspace_init(void* workspace, size_t ws_bytes, void* stream);

/*
 * Diagnostic: how many query rows, since the workspace was last zeroed by
 * csa2_workspace_init, had their top-k recomputed exactly over every item
 * because the candidate bands of the scan could not hold the answer (a scan
 * chunk holding more of the row's winners than its 128-slot segment, e.g.
 * when many keys score the same, or, for prefill-sized calls, the sampled
 * threshold or the MFMA band misled).  Results are exact either way; a
 * count above zero on a steady workload means the slow path is taken.
 *   workspace  device, the workspace the calls used;  count  host (out)
 * Waits for the stream.  Errors: CSA2_ERR_ARG / CSA2_ERR_WORKSPACE for bad
 * pointers, CSA2_ERR_HIP if the copy fails.
 */
int csa2_workspace_fallbacks(const void* workspace, uint32_t* count, void* stream);

/*
 * Optional kernel timing, for measurement tools (the pages say nothing about
 * it).  While enabled, each kernel the library launches is bracketed by two
 * HIP events recorded on the launch's own stream; csa2_profile_read waits for
 * the recorded events of one kernel class and returns their summed elapsed
 * milliseconds and count.  Process-wide; do not enable while a stream is
 * being captured into a graph.  Returns CSA2_ERR_ARG for null outputs and
 * CSA2_ERR_HIP if an event cannot be read.
 */
#define CSA2_K_QUANTIZE 0
#define CSA2_K_BLOCK_KEYS 1
#define CSA2_K_INDEX_SCAN 2
#define CSA2_K_INDEX_SAMPLE 3     /* kept for numbering: no decode launch records it     */
#define CSA2_K_INDEX_SELECT 4     /* in csa2_run_group decode calls, the select launch   */
                                  /* also runs the attention tiles (CSA2_K_ATTENTION then */
                                  /* records nothing; the merge keeps its own class)     */
#define CSA2_K_ATTENTION 5
#define CSA2_K_PREFILL_SAMPLE 6
#define CSA2_K_ATTENTION_MERGE 7
#define CSA2_K_PREFILL_FILTER 8
#define CSA2_K_PREFILL_SELECT 9
#define CSA2_K_APPEND 10
int csa2_profile_enable(int32_t on);
int csa2_profile_reset(void);
int csa2_profile_read(int32_t kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
