/*
 * csa2.h - C ABI of one Compressed Sparse Attention 2 (CSA2) layer step over
 * an FP4 (E2M1 + E8M0) global KV cache, for AMD Instinct MI355X (gfx950).
 *
 * What the step is.  CSA2 runs every layer in one of three static modes that
 * share one global KV cache and one sparse selection across layers
 * ("Unlocking Extreme Context Scaling with DeepSeek-V4.1-Flash", section
 * "Compressed Sparse Attention 2 (CSA2)"; the same three modes in
 * "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression",
 * Method):
 *   Full    - writes fresh main-KV and indexer-K entries, scores them and
 *             selects new Top-512 indices, then attends;
 *   Reindex - scores a new indexer query against the last Full layer's
 *             indexer-K and selects afresh, then attends over that layer's KV;
 *   Reuse   - attends with the main KV and Top-K indices of an earlier layer,
 *             skipping the indexer.
 * The main KV is stored in the E2M1 FP4 format ("DeepSeek-V4.1-Flash",
 * aiany.app item, "What Sets It Apart"), at about half the bytes of FP8
 * ("Unlocking Extreme Context Scaling ...", "Deployment and
 * Infrastructure"), and the global KV lives in HBM ("DeepSeek-V4.1-Flash",
 * researchpod.app episode summary).
 *
 * Formats fixed here (the pages name the formats but not their layout):
 *   main-KV row  : 512 latent values, one E8M0 scale per 32 consecutive
 *                  values; 272 bytes = 256 bytes of E2M1 codes (element 2i
 *                  in the low nibble of byte i, 2i+1 in the high nibble)
 *                  followed by 16 scale bytes (value 2^(byte-127)).
 *                  Encoding: scale = smallest 2^e with amax <= 6 * 2^e
 *                  (e clamped to [-127, 127], all-zero block -> byte 0);
 *                  code = round-to-nearest of x / 2^e on the E2M1 grid, ties
 *                  to the even code, sign bit copied from x.
 *   indexer-K row: 128 OCP E4M3FN bytes, round-to-nearest-even from bf16,
 *                  saturating at +-448, sign bit copied.
 *   indexer score: s_t = sum_h w_h * max(0, q_h . k_t), fp32 accumulation of
 *                  exact FP8 products; a zero score counts as +0.
 *   Top-K        : the first min(k, V) entries under (score descending,
 *                  index ascending), written in ascending index order,
 *                  slots beyond the count set to -1.
 *   attention    : K = V = the dequantised latent row shared by all heads;
 *                  O[h] = sum_j softmax_j(sm_scale * q_h . X_j) X_j over the
 *                  selected rows, fp32; LSE[h] = natural-log normaliser.
 *
 * Conventions for every entry point.
 *   - All data pointers are device pointers owned by the caller.  The library
 *     allocates no memory and keeps no state between calls except what the
 *     caller's workspace carries (see csa2_workspace_bytes).
 *   - Work is enqueued on the given HIP stream and is asynchronous.  Argument
 *     errors are found on the host before anything is enqueued and return a
 *     status; execution errors surface at the caller's next stream sync.
 *   - Device-resident values (seq_lens, q_vis, q_seq, page-table entries,
 *     slots, idx, cnt, pool) are trusted: the caller guarantees q_vis[i] <=
 *     seq_len(q_seq[i]) <= max_pages * page_size and that every page-table
 *     entry a query can reach lies in [0, num_pages).  The kernels still clamp
 *     q_vis to [0, max_vis], counts to [0, k], selected and pool indices to
 *     the page table's range and the page ids they read to [0, num_pages), so
 *     such values give wrong results rather than stray memory accesses;
 *     q_seq and slots are used as given.
 *   - Every pointer must be 16-byte aligned (w, q_seq, q_vis, cnt, lse,
 *     slots: 4-byte aligned suffices); a zero count (n == 0 or nq == 0)
 *     returns CSA2_OK and enqueues nothing.
 *   - Indices are logical entry positions inside a sequence (not physical
 *     slots), so a Reuse layer can hand them on unchanged.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_D_LATENT        512
#define CSA2_D_INDEX         128
#define CSA2_KV_ROW_BYTES    272
#define CSA2_IDXK_ROW_BYTES  128
#define CSA2_MAX_K           2048
#define CSA2_MAX_H_IDX       16
#define CSA2_MAX_H           128
#define CSA2_MIN_PAGE_SIZE   64

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misalignment      */
  CSA2_ERR_UNSUPPORTED = 2,   /* valid request this library does not serve */
  CSA2_ERR_WORKSPACE = 3,     /* ws_bytes below csa2_workspace_bytes(...)  */
  CSA2_ERR_HIP = 4            /* a HIP launch failed                        */
} csa2_status;

typedef enum { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2 } csa2_mode;

/* One Full layer's global cache (all pointers device memory, caller-owned).
 * Logical entry t of sequence s lives at page page_table[s*max_pages +
 * t/page_size], row t % page_size of that page. */
typedef struct {
  uint8_t*       kv;          /* [num_pages][page_size][272] main-KV rows     */
  uint8_t*       idx_k;       /* [num_pages][page_size][128] indexer-K rows   */
  const int32_t* page_table;  /* [num_seqs][max_pages]                        */
  const int32_t* seq_lens;    /* [num_seqs] valid entries (informational)     */
  int32_t num_pages;
  int32_t page_size;          /* power of two, >= CSA2_MIN_PAGE_SIZE          */
  int32_t num_seqs;
  int32_t max_pages;
  uint8_t*       idxk_bounds; /* nullable: block-level representation of the
                                 indexer-K for CSA2_STEP_PRUNE,
                                 [num_pages * page_size / 64][2][128] E4M3
                                 codes (see csa2_idxk_bounds_build)          */
} csa2_cache_view;

/* Block-level representation of the indexer-K, the summary the pruning of
 * CSA2_STEP_PRUNE reads.  The indexer the hierarchical indexer is informed by
 * scores token-level entries and prunes them by block-level representations
 * ("DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression",
 * Related Work); the pages define no summary, the reading here: a block is
 * CSA2_PRUNE_BLOCK consecutive physical rows (so a block never straddles a
 * page), its representation 256 bytes, the E4M3 code of each dimension's
 * largest value over the block's rows followed by that of its smallest.
 * csa2_idxk_bounds_build recomputes blocks first_block .. first_block +
 * n_blocks - 1 from c->idx_k (after bulk writes; csa2_layer_step refreshes
 * the blocks of the rows it appends itself whenever c->idxk_bounds is set).
 * Rows of a block that were never written count with whatever bytes they
 * hold, which only widens the bounds.  Errors: CSA2_ERR_INVALID_ARG for a
 * null or misaligned idxk_bounds (16 bytes), a bad cache or a block range
 * outside the cache; CSA2_ERR_HIP if the launch fails. */
#define CSA2_PRUNE_BLOCK 64
csa2_status csa2_idxk_bounds_build(const csa2_cache_view* c, int32_t first_block, int32_t n_blocks,
                                   hipStream_t s);

/* Quantize-on-append ("DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
 * Compression", Method: FP4 global KV with an inference system built to
 * serve the format).  Encodes n bf16 rows and writes them at physical slots
 * slots[i] = page * page_size + row:
 *   kv_rows   [n][512] bf16 bit patterns -> c->kv    (272-byte FP4 rows)
 *   idxk_rows [n][128] bf16 bit patterns -> c->idx_k (128-byte E4M3 rows)
 * Slots must be distinct within one call.  The caller updates seq_lens and
 * the page table.  Output bytes are deterministic. */
csa2_status csa2_append_quant_fp4(const csa2_cache_view* c, const int32_t* slots,
                                  const uint16_t* kv_rows, const uint16_t* idxk_rows,
                                  int32_t n, hipStream_t s);

/* Bytes of workspace a layer_step call of this shape needs.  Layout: three
 * per-query u32 arrays [nq] first (candidate counters, the dense indexer's
 * thresholds, its full-rescore counters), padded to 256 bytes; then (Full
 * and Reindex) per-query candidate indices [nq][round_up(max_vis + 2, 64)]
 * i32, their score keys of the same shape, the per-query scan's chunk key
 * floors [nq][ceil(max_vis / 2048)] u32, the CSA2_STEP_PRUNE block masks of
 * the same shape (bit i of word c: block 32c + i of the query's visible
 * range holds no Top-k entry) and the scan's largest score key of every
 * 64-entry block [nq][ceil(max_vis / 2048)][32] u32, that region being at
 * least nq * 8 KB so a CSA2_STEP_POOL layer can score its pool there.
 * csa2_index_topk accepts a workspace sized by this call for the same shape;
 * attention needs none.  Only the first round_up(nq * 12, 256) bytes carry
 * state: every call leaves them zeroed for the next one, so zero the whole
 * workspace once after allocating it (csa2_workspace_init does this); the
 * rest is written before it is read within each call.  Calls that share one
 * workspace must not run concurrently. */
size_t csa2_workspace_bytes(csa2_mode mode, int32_t nq, int32_t max_vis,
                            int32_t h_idx, int32_t h, int32_t k);

/* Zero-fills ws_bytes of workspace on stream s (a fill kernel, no memset
 * node, so it may be captured in a graph). */
csa2_status csa2_workspace_init(void* ws, size_t ws_bytes, hipStream_t s);

/* Indexer scoring + Top-K ("Unlocking Extreme Context Scaling ...", section
 * CSA2: Full and Reindex modes score indexer queries against the cached
 * indexer-K and select Top-512).  For query i of sequence q_seq[i], entries
 * 0..q_vis[i]-1 are scored with
 *   q_idx [nq][h_idx][128] E4M3 bytes, w [nq][h_idx] fp32,
 * and out_idx [nq][k] int32 receives the selection in ascending index order
 * (-1 padded), out_cnt [nq] the count min(k, q_vis[i]).
 * max_vis is a host upper bound on q_vis (sizes the grid and workspace).
 * 1 <= h_idx <= 16, 1 <= k <= CSA2_MAX_K. */
csa2_status csa2_index_topk(const csa2_cache_view* c, const uint8_t* q_idx, const float* w,
                            const int32_t* q_seq, const int32_t* q_vis,
                            int32_t nq, int32_t h_idx, int32_t k, int32_t max_vis,
                            int32_t* out_idx, int32_t* out_cnt,
                            void* ws, size_t ws_bytes, hipStream_t s);

/* Dense form of csa2_index_topk for a prefill chunk, where every query
 * belongs to one sequence (q_seq[i] == q_seq[0] for all i; a device value,
 * trusted like q_vis).  The scoring then runs as one FP8 matrix product
 * [nq * h_idx x 128] x [128 x max_vis] under the causal mask t < q_vis[i],
 * prefill being the computationally expensive phase ("DeepSeek-V4.1-Flash"
 * research-podcast summary, abstract).  Arguments, outputs, workspace and
 * errors are those of csa2_index_topk, and the scores - so the selection -
 * are bit-identical to it. */
csa2_status csa2_prefill_index_topk(const csa2_cache_view* c, const uint8_t* q_idx, const float* w,
                                    const int32_t* q_seq, const int32_t* q_vis,
                                    int32_t nq, int32_t h_idx, int32_t k, int32_t max_vis,
                                    int32_t* out_idx, int32_t* out_cnt,
                                    void* ws, size_t ws_bytes, hipStream_t s);

/* Sparse attention over the selected rows.  Every CSA2 mode ends here: Full
 * and Reindex attend over the Top-512 entries they just selected, Reuse over
 * the main KV and indices of an earlier layer ("Unlocking Extreme Context
 * Scaling with DeepSeek-V4.1-Flash", section "Compressed Sparse Attention 2
 * (CSA2)"); the cost is set by the selection, not by the context length
 * ("DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression",
 * Introduction: near-constant single-token decode FLOPs from 4K to 1M).
 * Keys and values are the same dequantised 512-wide latent row, shared by all
 * heads (the reading stated at the top of this header).
 *   q   [nq][h][512] bf16 bit patterns, q_seq [nq],
 *   idx [nq][k] selected entry indices (first cnt[i] valid), cnt [nq]
 *   (a count outside [0, k] is taken as the nearest bound),
 *   out [nq][h][512] fp32, lse [nq][h] fp32 (nullable).
 * 1 <= h <= 128; sm_scale > 0 and finite.  The attention needs no
 * workspace: ws may be NULL (a non-NULL ws must be 16-byte aligned and is
 * left untouched).  Selected indices are clamped to the page table's range
 * and page ids to [0, num_pages) before any row is read.
 * Errors: CSA2_ERR_INVALID_ARG for bad sizes, a bad sm_scale, null or
 * misaligned pointers; CSA2_ERR_HIP if a launch fails. */
csa2_status csa2_sparse_attn(const csa2_cache_view* c, const uint16_t* q, const int32_t* q_seq,
                             const int32_t* idx, const int32_t* cnt,
                             int32_t nq, int32_t h, int32_t k, float sm_scale,
                             float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t s);

/* Per-kernel device timing of one call, for measurement.  For each kernel
 * class whose ring is set, the call's launches of that class record the
 * hipEvent pair start[count] / stop[count] and increment count, until count
 * reaches capacity.  The events are carried by the kernel dispatches
 * themselves (start when the class's first kernel of the launch begins, stop
 * when its last kernel ends), so no separate stream operations are added.
 * Everything is caller memory: the events (hipEventCreate), the rings and
 * this struct, which must stay valid until the call returns; the library
 * writes only the rings' count fields.  Calls that run concurrently must not
 * share a ring.  Classes: append, indexer scan (for the dense indexer:
 * threshold, candidates, full rescore and compaction), Top-K select,
 * attention, the dense indexer's matrix-product (candidate) kernel alone,
 * hierarchical indexer pool scoring and pool select. */
typedef struct {
  hipEvent_t* start;     /* [capacity] */
  hipEvent_t* stop;      /* [capacity] */
  int32_t     capacity;
  int32_t     count;     /* launches recorded so far */
} csa2_timing_ring;

#define CSA2_KCLASS_APPEND 0
#define CSA2_KCLASS_SCAN   1
#define CSA2_KCLASS_SELECT 2
#define CSA2_KCLASS_ATTN   3
#define CSA2_KCLASS_DENSE  4
#define CSA2_KCLASS_POOL_SCAN   5   /* hierarchical indexer: pool scoring */
#define CSA2_KCLASS_POOL_SELECT 6   /* hierarchical indexer: Top-k of the pool */
#define CSA2_NUM_KCLASSES  7

typedef struct csa2_timing {
  csa2_timing_ring* ring[CSA2_NUM_KCLASSES];   /* NULL: that class untimed */
} csa2_timing;

#define CSA2_DENSE_RESCORE_ALL (-1)

/* Arguments of one layer.  Fields a mode does not use must be NULL / 0. */
typedef struct {
  const csa2_cache_view* cache;  /* Full: its own cache (written);
                                    Reindex/Reuse: the source Full layer's   */
  const int32_t*  new_slots;     /* Full only: rows appended before scoring  */
  const uint16_t* new_kv;
  const uint16_t* new_idxk;
  int32_t         n_new;
  const uint8_t*  q_idx;         /* Full, Reindex */
  const float*    w;
  int32_t         h_idx;
  const uint16_t* q;             /* all modes */
  int32_t         h;
  float           sm_scale;
  const int32_t*  q_seq;
  const int32_t*  q_vis;
  int32_t         nq;
  int32_t         k;
  int32_t         max_vis;
  int32_t*        idx;           /* Full/Reindex: written; Reuse: read       */
  int32_t*        cnt;
  float*          out;
  float*          lse;           /* nullable */
  void*           ws;
  size_t          ws_bytes;
  uint32_t        flags;         /* CSA2_STEP_* bits, 0 by default            */
  int32_t*        pool;          /* CSA2_STEP_POOL: [nq][pool_k] candidate pool
                                    (Full: written; Reindex: read)           */
  int32_t*        pool_cnt;      /* [nq]                                      */
  int32_t         pool_k;        /* pool width P, k <= P <= CSA2_MAX_K        */
  int32_t         dense_cand_factor;  /* CSA2_STEP_DENSE_INDEX: expected
                                    candidates per query in units of k (the
                                    selection is exact for every value): 0 =
                                    default (4), 1..64 = that factor,
                                    CSA2_DENSE_RESCORE_ALL = every query with
                                    more than k visible entries is rescored in
                                    full; must be 0 without the flag          */
  struct csa2_timing* timing;    /* nullable: device timestamps of this call's
                                    kernels (see csa2_timing)                  */
  const int32_t*  seed;          /* CSA2_STEP_PRUNE: [nq][k] entry indices
                                    whose scores set each query's threshold
                                    (e.g. its previous Top-K row; may be idx
                                    itself, read before the layer writes it) */
  const int32_t*  seed_cnt;      /* CSA2_STEP_PRUNE: [nq] entries of each seed
                                    row to use (clamped to [0, k])            */
} csa2_step_args;

/* Full/Reindex: score as csa2_prefill_index_topk (all queries of the call
 * belong to the sequence q_seq[0], e.g. one prefill chunk). */
#define CSA2_STEP_DENSE_INDEX 1u
/* Hierarchical indexer (see csa2_pool_index_topk).  Full: the indexer keeps
 * its Top-pool_k as the pool (written to pool/pool_cnt, ascending) and the
 * layer's Top-k is then taken among the pool, which equals its plain Top-k.
 * Reindex: only the entries of pool (an earlier Full layer's) are scored.
 * Reuse: not allowed. */
#define CSA2_STEP_POOL 2u
/* Large batches of 64-head queries normally take the attention form that
 * gathers and dequantises each selected row once for all 64 heads of a query;
 * this flag keeps one workgroup per 16-head group instead.  Both forms give
 * identical bits (it exists to test and measure that). */
#define CSA2_STEP_ATTN_PER_HEAD_GROUP 4u
/* Block-level pruning of a Full or Reindex layer's per-query indexer (not
 * with CSA2_STEP_DENSE_INDEX or CSA2_STEP_POOL; needs cache->idxk_bounds).
 * Per query, the threshold T is the k-th largest score (the indexer's own
 * arithmetic) of the distinct entries of seed[i][0 .. seed_cnt[i]) that lie
 * in its visible range; with fewer than k of them nothing is pruned.  Every
 * 64-entry block whose bound lies below T (bound: sum over heads of
 * w_h * max(0, the largest (w_h >= 0) or smallest (w_h < 0) value q_h . k
 * takes in the block's per-dimension box), widened by 2^-14 of its summed
 * magnitudes against rounding) is never read.  At least k entries score
 * T or more, so no pruned entry belongs to the Top-k: the selection, and
 * everything after it, is the one without the flag, bit for bit. */
#define CSA2_STEP_PRUNE 8u

/* Hierarchical indexer: the indexer of a later (Reindex) layer scores only
 * the shared candidate pool an earlier indexer chose, and keeps its Top-k
 * among it ("DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
 * Compression", Method: the Hierarchical Sparse Indexer restricts the
 * indexers to a shared candidate pool selected by an earlier indexer).  The
 * pages do not say how large the pool is or how it is chosen; the reading
 * here: the earlier layer's own Top-P (csa2_index_topk with k = P), so pool
 * rows are ascending entry indices.  Per query: s_t as in csa2_index_topk for
 * the pool's first pool_cnt entries t only (bit-identical to the exhaustive
 * scan's s_t), then the first min(k, pool_cnt) of them under (score
 * descending, index ascending), written ascending to out_idx [nq][k], -1
 * padded; out_cnt [nq].
 *   pool [nq][p] int32 (first pool_cnt[q] valid, ascending, each < the
 *   sequence's visible length), 1 <= p <= CSA2_MAX_K, 1 <= k <= CSA2_MAX_K;
 *   other arguments as csa2_index_topk.  ws: at least
 *   csa2_pool_workspace_bytes(nq, p) bytes, 16-byte aligned, no initial state.
 * Errors: CSA2_ERR_INVALID_ARG for bad sizes or null/misaligned pointers,
 * CSA2_ERR_WORKSPACE for a short workspace, CSA2_ERR_HIP on launch failure;
 * nq = 0 enqueues nothing.  Pool values are trusted device data. */
csa2_status csa2_pool_index_topk(const csa2_cache_view* c, const uint8_t* q_idx, const float* w,
                                 const int32_t* q_seq, const int32_t* pool, const int32_t* pool_cnt,
                                 int32_t nq, int32_t h_idx, int32_t p, int32_t k,
                                 int32_t* out_idx, int32_t* out_cnt, void* ws, size_t ws_bytes, hipStream_t s);
size_t csa2_pool_workspace_bytes(int32_t nq, int32_t p);

/* One CSA2 layer in one of the three static modes of "Unlocking Extreme
 * Context Scaling with DeepSeek-V4.1-Flash", section "Compressed Sparse
 * Attention 2 (CSA2)" (the same modes in "DeepSeek-V4.1-Flash: Pushing the
 * Limits of KV Cache Compression", Method):
 *   Full    = append (if n_new > 0) -> index_topk -> sparse_attn
 *             (fresh entries, fresh scores and Top-k);
 *   Reindex = index_topk with the layer's own indexer query on the source
 *             Full layer's indexer-K -> sparse_attn over that layer's KV;
 *   Reuse   = sparse_attn with the given idx/cnt (an earlier layer's KV and
 *             indices; no indexing at all).
 * Every argument is checked on the host before anything is enqueued: the
 * checks of csa2_append_quant_fp4, csa2_index_topk (Full, Reindex) and
 * csa2_sparse_attn, unknown flags, fields the mode does not use that are not
 * NULL / 0, a workspace below csa2_workspace_bytes(mode, ...) for Full and
 * Reindex.  Returns the first failing status (nothing enqueued), else
 * CSA2_ERR_HIP if a launch fails, else CSA2_OK. */
csa2_status csa2_layer_step(csa2_mode mode, const csa2_step_args* a, hipStream_t s);

/* csa2_layer_step for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same layer step, with the workspace taken from a fixed array of
 * CSA2_STATIC_SCRATCH_BYTES bytes of device memory that the library holds on
 * each GPU it runs on until the process ends, instead of a->ws.  Allocates
 * nothing (no hipMalloc, hipFree or allocating library call).  a->ws must be
 * NULL and a->ws_bytes 0; every other field is as for csa2_layer_step, whose
 * results it gives bit for bit.  The stream must belong to the current
 * device; the first call on a device looks up that device's array.  Every
 * call clears the array's state-carrying head (the per-query histograms and
 * counters) before its kernels run, so a call never depends on an earlier
 * one.  All calls on one GPU share its array: calls that overlap in time on
 * one GPU race, so serialise them (one stream, or events).  Errors: those of
 * csa2_layer_step; CSA2_ERR_WORKSPACE when the shape needs more than
 * CSA2_STATIC_SCRATCH_BYTES (csa2_workspace_bytes(mode, ...) gives the need);
 * CSA2_ERR_INVALID_ARG for a non-NULL ws; CSA2_ERR_HIP if the array's address
 * cannot be found or a launch fails. */
#define CSA2_STATIC_SCRATCH_BYTES (64u << 20)
csa2_status csa2_layer_step_static(csa2_mode mode, const csa2_step_args* a, hipStream_t s);

/* A group of layers that share caches and indices, run as one call.  The
 * layers' results are exactly those of calling csa2_layer_step on each in
 * order on s (same kernels, same inputs); the group only overlaps work that
 * does not depend on each other.  The modes' composition is the one of
 * "Unlocking Extreme Context Scaling with DeepSeek-V4.1-Flash", section
 * "Compressed Sparse Attention 2 (CSA2)": Reindex and Reuse layers read an
 * earlier Full layer's cache, Reuse layers its indices; a Reuse layer skips
 * indexing altogether, so its attention can run beside the layers after it.
 *
 * Execution (ex): with ex == NULL or n_aux == 0 the layers run one after the
 * other on s.  Otherwise Full and Reindex layers still run whole on s in
 * layer order, and each Reuse layer runs on one of the caller's auxiliary
 * streams (round-robin) as soon as the select whose idx/cnt it reads is done,
 * beside the layers that follow it on s.  Layers that share a workspace, an
 * output, an idx/cnt buffer one of them writes, or a cache a later Full layer
 * appends to are ordered with events, so sharing buffers is always correct
 * but removes overlap: give concurrent layers their own workspaces.  All work
 * is ordered after what was enqueued on s before the call, and everything
 * enqueued on s afterwards runs after all of it (s waits for every auxiliary
 * stream used).
 *
 * Ownership: the caller creates the auxiliary streams (default priority,
 * same device, none equal to s) and at least csa2_group_events(n, n_aux)
 * events (flags without timing suffice); the call records and waits on them
 * and keeps no reference after it returns.  Calls that overlap in time must
 * not share events.  Errors: CSA2_ERR_INVALID_ARG for n outside
 * [0, CSA2_GROUP_MAX_LAYERS], null arrays, n_aux outside
 * [0, CSA2_GROUP_MAX_AUX], a null or repeated stream, too few or null
 * events; every layer is validated as by csa2_layer_step before anything is
 * enqueued, and the first failing layer's status is returned. */
#define CSA2_GROUP_MAX_LAYERS 64
#define CSA2_GROUP_MAX_AUX 4
typedef struct {
  hipStream_t aux[CSA2_GROUP_MAX_AUX];
  int32_t     n_aux;
  hipEvent_t* events;
  int32_t     n_events;
} csa2_group_exec;

/* Events a csa2_group_step call needs: 1 + 3 n_layers + n_aux; -1 for
 * arguments outside the limits above. */
int32_t csa2_group_events(int32_t n_layers, int32_t n_aux);

csa2_status csa2_group_step(int32_t n, const csa2_mode* modes, const csa2_step_args* layers, hipStream_t s,
                            const csa2_group_exec* ex);

/* Merge of the global (CSA2) branch with the local sliding-window branch of
 * the same queries and heads: the output and LSE of one softmax over the
 * union of the two branches' keys.  The pages place a global attention branch
 * over the full context beside local sliding-window attention ("DeepSeek-
 * V4.1-Flash: Pushing the Limits of KV Cache Compression"; the
 * research-podcast summary: global context decoupled from local
 * sliding-window attention) and give no combination formula; this is the
 * plainest reading.  Per row r (e.g. r = query * h + head):
 *   M = max(lse_a[r], lse_b[r]), w_x = e^(lse_x[r] - M),
 *   o[r][:] = (w_a o_a[r][:] + w_b o_b[r][:]) / (w_a + w_b),
 *   lse[r] = M + ln(w_a + w_b)   (natural log, like csa2_sparse_attn's LSE);
 * a branch with lse = -inf has no keys and counts for nothing; both empty
 * give o = 0, lse = -inf.
 * Layout: o_a, o_b, o [rows][dim] fp32 (16-byte aligned, dim a multiple of 4,
 * 4 <= dim), lse_a, lse_b, lse [rows] fp32 (lse nullable).  o may be o_a or
 * o_b (in place); lse must not be lse_a or lse_b.  All device memory owned
 * by the caller.  rows = 0 enqueues nothing.  Errors: CSA2_ERR_INVALID_ARG for
 * rows < 0, a bad dim, null or misaligned pointers, or lse aliasing an input
 * LSE; CSA2_ERR_HIP if the launch fails. */
csa2_status csa2_lse_merge(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                           int32_t rows, int32_t dim, float* o, float* lse, hipStream_t s);

/* FP4 fake quantisation for quantization-aware training: the global KV is
 * trained with FP4 ("DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
 * Compression").  Every 32-element block of x (consecutive in memory) is
 * encoded with exactly the main-KV rules of csa2_append_quant_fp4 (E8M0 scale
 * 2^e, the smallest with amax <= 6 * 2^e; E2M1 codes, round to nearest, ties
 * to the even code, sign kept) and decoded back: y = E2M1(code) * 2^e, in the
 * dtype of x (the values are exact in fp32 and bf16).  Backward: the
 * straight-through gradient is the identity, exact here because the scale
 * rule never clips, so no backward entry point is needed.
 * x, y: n values of dtype (CSA2_DTYPE_F32 or CSA2_DTYPE_BF16), device memory
 * owned by the caller, 16-byte aligned; y may be x (in place).  n must be a
 * non-negative multiple of 32; n = 0 enqueues nothing.  Errors:
 * CSA2_ERR_INVALID_ARG for a bad n or dtype, null or misaligned pointers;
 * CSA2_ERR_HIP if the launch fails. */
#define CSA2_DTYPE_F32  0
#define CSA2_DTYPE_BF16 1
csa2_status csa2_fake_quant_fp4(const void* x, void* y, int64_t n, int32_t dtype, hipStream_t s);

/* Static description of a status code. */
const char* csa2_status_string(csa2_status st);


#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
