// Internal launchers of the CSA2 kernels (not part of the C ABI).
#pragma once
#include <algorithm>
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

struct CacheArgs {
  uint8_t* kv;
  uint8_t* idx_k;
  const int32_t* page_table;
  int32_t max_pages;
  int32_t lg_page;       // log2(page_size)
  int32_t num_pages;
};

// Page id read from the page table, clamped to the cache's pages.
__device__ __forceinline__ int clamp_page(int page, const CacheArgs& c) {
  return min(max(page, 0), c.num_pages - 1);
}

// Physical row of logical entry t of a sequence (page-table row pt_row), with
// t clamped to the table's range and the page id to the cache's pages, so a
// bad index reads some row of the cache rather than stray memory.
__device__ __forceinline__ int64_t entry_row_clamped(const int32_t* __restrict__ pt_row, int t, const CacheArgs& c) {
  t = min(max(t, 0), (c.max_pages << c.lg_page) - 1);
  const int page = clamp_page(pt_row[t >> c.lg_page], c);
  return ((int64_t)page << c.lg_page) + (t & ((1 << c.lg_page) - 1));
}

// Workspace of the indexer (byte offsets):
//   [0, Z)      zero-state, three [nq] u32 arrays: candidate counters, the
//               dense indexer's thresholds (fp32 bits) and its full-rescore
//               counters; the final select kernel zeroes a query's three
//               words again.
//   [Z, ...)    candidate indices [nq][vstride] i32, their score keys
//               [nq][vstride] u32, then (per-query scan) the chunk key floors
//               [nq][fstride] u32, the pruned-block masks [nq][fstride] u32
//               and the block maximum keys [nq][fstride][32] u32; no initial
//               state needed.
struct IndexWs {
  uint32_t* cand_cnt;
  float* tau;            // dense indexer: the query's candidate threshold
  uint32_t* cnt2;        // dense indexer: candidates the full rescore added after cand_cnt
  int32_t* cand;
  uint32_t* ckey;        // score key of cand[i], stored beside it (the final select reads no scores)
  int64_t vstride;
  int32_t vis_cap;       // max_vis of the call: visible counts are clamped to it
  // Per-query scan: the key floor below which each 2,048-entry chunk kept no
  // candidate, [nq][fstride] u32 (a 22-bit key prefix; bit 0 set,
  // kFloorBlockMax, when the chunk stored its block maximum keys in bmax);
  // NULL for the dense indexer, whose candidates are exact above its
  // threshold.
  uint32_t* floor;
  int32_t fstride;
  // Block-level pruning: per (query, chunk) the mask of its 64-entry blocks
  // that cannot hold an entry of the Top-k, [nq][fstride] u32 (bit i: block
  // 32 * chunk + i); NULL when the call prunes nothing.  The query's
  // threshold is in tau.
  uint32_t* prune;
  // Per-query scan: per (query, chunk) the largest score key of each of its
  // 32 blocks of 64 entries, [nq][fstride][32] u32 (0 for a pruned block or
  // one past the visible range), written only by chunks whose candidates
  // crowd into one block (floor bit kFloorBlockMax), so the final select
  // rescores only blocks that can hold entries it lacks; NULL for the dense
  // indexer.
  uint32_t* bmax;
};

constexpr uint32_t kFloorBlockMax = 1u;      // chunk floor bit: block maximum keys stored
constexpr int kPruneBlockRows = 64;          // cache rows per block-level representation
constexpr int kPruneBoundBytes = 256;        // per block: 128 maximum codes, 128 minimum codes

// A query's visible count as the indexer kernels use it: clamped to [0, max_vis].
__device__ __forceinline__ int clamp_vis(int v, const IndexWs& ws) { return min(max(v, 0), ws.vis_cap); }

// Optional device timestamps of one launch class: `start` is taken when its
// first kernel starts, `stop` when its last kernel ends (recorded by the
// dispatch itself, so timing adds no separate stream operations).
struct KEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
  KEvents first() const { return {start, nullptr}; }
  KEvents last() const { return {nullptr, stop}; }
};

template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, hipStream_t s, const KEvents& ev, Args... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// A launch class that dispatches nothing still completes its events.
inline void record_empty(const KEvents& ev, hipStream_t s) {
  if (ev.start) (void)hipEventRecord(ev.start, s);
  if (ev.stop) (void)hipEventRecord(ev.stop, s);
}

constexpr int kHistBits = 11;                // first radix digit of the score key
constexpr int kHistBins = 1 << kHistBits;
constexpr int kScanChunk = 2048;             // entries per scan workgroup
constexpr int kSelectThreads = 1024;
constexpr int kTieCap = 4096;                // composite keys held in LDS by the select kernel (32 KB of LDS)
constexpr int kCollectSlice = 8192;          // entries per candidate-collect workgroup

int64_t index_vstride(int32_t max_vis);
size_t zero_state_bytes(int32_t nq);
size_t index_score_bytes(int32_t nq, int32_t max_vis);

hipError_t launch_append_quant(uint8_t* kv, uint8_t* idx_k, const int32_t* slots, const uint16_t* kv_rows,
                               const uint16_t* idxk_rows, int n, hipStream_t s, const KEvents& ev = {});
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

// Per-query scan: scores every visible entry and keeps, per 2,048-entry chunk,
// the entries at or above the chunk's local rank threshold as candidates
// (indices, score keys, their histogram, and the chunk's key floor); the final
// select then completes the exact Top-k (k is needed for the local rank).
// A layer step's quantize-on-append of at most kMaxFusedAppend rows can run
// inside the scan launch (its own workgroups write the rows; scan workgroups
// whose chunk holds one score it from the bf16 source).
struct AppendArgs {
  uint8_t* kv;
  uint8_t* idx_k;
  const int32_t* slots;
  const uint16_t* kv_rows;
  const uint16_t* idxk_rows;
  int n;
};
constexpr int kMaxFusedAppend = 64;
hipError_t launch_index_scan(const CacheArgs& c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                             const int32_t* q_vis, int nq, int h_idx, int k, int max_vis, const IndexWs& ws,
                             hipStream_t s, const KEvents& ev = {}, const AppendArgs* ap = nullptr);
// Inputs of the final select's repair of a chunk whose local threshold lies
// above the k-th key's bin (per-query scan only).
struct ScanArgs {
  CacheArgs c;
  const uint8_t* q_idx;
  const float* w;
  const int32_t* q_seq;
  int h_idx;
};

// Dense form for many queries of one sequence (q_seq[0]): leaves a candidate
// list (indices and score keys) per query for the final select, with scores
// bit-identical to the per-query scan.  ev covers the threshold, candidate
// and full-rescore kernels, ev_product the candidate (matrix-product) kernel
// alone.
// cand_factor: expected candidates per query in units of k (0 sends every
// query through the full rescore).
constexpr int kDefaultCandFactor = 4;
hipError_t launch_prefill_scan(const CacheArgs& c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                               const int32_t* q_vis, int nq, int h_idx, int k, int max_vis, const IndexWs& ws,
                               int cand_factor, hipStream_t s, const KEvents& ev = {},
                               const KEvents& ev_product = {});
// Block-level pruning: the bounds of the blocks holding the given slots
// (slots != NULL, n slots) or of blocks first_block .. first_block + n - 1;
// and per query the threshold of its seed and the mask of pruned blocks.
hipError_t launch_idxk_bounds(const uint8_t* idx_k, uint8_t* bounds, const int32_t* slots, int first_block,
                              int n, int64_t n_rows, hipStream_t s, const KEvents& ev = {});
hipError_t launch_prune_mask(const CacheArgs& c, const uint8_t* bounds, const uint8_t* q_idx, const float* w,
                             const int32_t* q_seq, const int32_t* q_vis, const int32_t* seed, const int32_t* seed_cnt,
                             int nq, int h_idx, int k, const IndexWs& ws, hipStream_t s, const KEvents& ev = {});
// The final select over a query's candidate list (the dense indexer's, or the
// per-query scan's, which sa and ws.floor let it repair).
hipError_t launch_topk_final(const IndexWs& ws, const ScanArgs& sa, const int32_t* q_vis, int nq, int k,
                             int32_t* out_idx, int32_t* out_cnt, hipStream_t s, const KEvents& ev = {});

// share_heads: large batches of 64-head queries take the form that gathers
// each selected row once for all 64 heads of a query (identical bits).
hipError_t launch_sparse_attn(const CacheArgs& c, const uint16_t* q, const int32_t* q_seq, const int32_t* idx,
                              const int32_t* cnt, int nq, int h, int k, float sm_scale, float* out, float* lse,
                              bool share_heads, hipStream_t s, const KEvents& ev = {});

// Hierarchical indexer: scores of each query's pool entries only (pool
// [nq][p] ascending entry indices, pool_cnt valid; scores [nq][round_up(p, 64)]
// fp32 in sc), then its Top-k among them.
size_t pool_score_bytes(int nq, int p);
hipError_t launch_pool_index(const CacheArgs& c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                             const int32_t* pool, const int32_t* pool_cnt, int nq, int h_idx, int p, int k,
                             int32_t* out_idx, int32_t* out_cnt, float* sc, hipStream_t s,
                             const KEvents& ev_scan = {}, const KEvents& ev_select = {});
// Branch merge: O and LSE of one softmax over the union of two key sets
// ([rows][dim] fp32 outputs, [rows] LSEs; dim a multiple of 4).
hipError_t launch_lse_merge(const float* oa, const float* la, const float* ob, const float* lb, int rows, int dim,
                            float* o, float* lse, hipStream_t s, const KEvents& ev = {});

// FP4 fake quantisation of n values (n a multiple of 32), fp32 or bf16.
hipError_t launch_fake_quant(const void* x, void* y, int64_t n, bool bf16, hipStream_t s, const KEvents& ev = {});

}  // namespace csa2
