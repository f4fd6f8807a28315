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
};

// Workspace of the indexer (byte offsets):
//   [0, Z)      zero-state: histograms [nq][2048] u32, then candidate
//               counters [nq] u32; the final select kernel leaves every row
//               it used zeroed again.
//   [Z, ...)    scores [nq][vstride] fp32, then candidate indices
//               [nq][vstride] i32, then (dense prefill indexer) candidate
//               masks, round_up(nq, 16) * vstride / 8 bytes; no initial
//               state needed.
struct IndexWs {
  uint32_t* hist;
  uint32_t* cand_cnt;
  float* scores;
  int32_t* cand;
  uint32_t* ckey;        // score key of cand[i], stored beside it (the final select reads no scores)
  uint64_t* mask;
  int64_t vstride;
};

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

hipError_t launch_index_scan(const CacheArgs& c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                             const int32_t* q_vis, int nq, int h_idx, int max_vis, const IndexWs& ws,
                             hipStream_t s, const KEvents& ev = {});

// Dense form for many queries of one sequence (q_seq[0]): leaves the same
// inputs for the final select (candidate list, candidate histogram, scores of
// the candidates), with scores bit-identical to the per-query scan.  ev covers
// the threshold, candidate, full-rescore and compaction kernels, ev_product
// the candidate (matrix-product) kernel alone.
hipError_t launch_prefill_scan(const CacheArgs& c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                               const int32_t* q_vis, int nq, int h_idx, int k, int max_vis, const IndexWs& ws,
                               hipStream_t s, const KEvents& ev = {}, const KEvents& ev_product = {});
// Expected candidates per query of the dense indexer, in units of k (0 sends
// every query through the full rescore).
extern int g_prefill_cand_factor;
// 1: large batches of 64-head queries take the attention form that shares
// each gathered row among the 64 heads.
extern int g_attn_share_heads;
// Launches of the final select alone (the dense indexer compacts its own candidates).
hipError_t launch_topk_final(const IndexWs& ws, const int32_t* q_vis, int nq, int k, int32_t* out_idx,
                             int32_t* out_cnt, hipStream_t s, const KEvents& ev = {});

hipError_t launch_topk_select(const IndexWs& ws, const int32_t* q_vis, int nq, int k, int max_vis,
                              int32_t* out_idx, int32_t* out_cnt, hipStream_t s, const KEvents& ev = {});

// Attention shares (small batches split their rows across workgroups):
// [nq * ceil(h/16)][nsplit][16][512] fp32 partial outputs, then
// [nq * ceil(h/16)][nsplit][32] fp32 (max, sum); no initial state needed.
int attn_nsplit(int nq, int h, int k);
size_t attn_part_bytes(int nq, int h, int k);

hipError_t launch_sparse_attn(const CacheArgs& c, const uint16_t* q, const int32_t* q_seq, const int32_t* idx,
                              const int32_t* cnt, int nq, int h, int k, float sm_scale, float* out, float* lse,
                              void* part, hipStream_t s, const KEvents& ev = {});

// Hierarchical indexer: scores of each query's pool entries only (pool
// [nq][p] ascending entry indices, pool_cnt valid; scores [nq][round_up(p, 64)]
// fp32 in sc), then its Top-k among them.
size_t pool_score_bytes(int nq, int p);
hipError_t launch_pool_index(const CacheArgs& c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                             const int32_t* pool, const int32_t* pool_cnt, int nq, int h_idx, int p, int k,
                             int32_t* out_idx, int32_t* out_cnt, float* sc, hipStream_t s,
                             const KEvents& ev_scan = {}, const KEvents& ev_select = {});
// Top-k of each query's pool from an exhaustive scan's score rows (score of
// entry t at scores[q * vstride + t]): no rescoring.
hipError_t launch_pool_select_by_entry(const int32_t* pool, const int32_t* pool_cnt, int nq, int p,
                                       const float* scores, int64_t vstride, int k, int32_t* out_idx,
                                       int32_t* out_cnt, hipStream_t s, const KEvents& ev = {});

// Branch merge: O and LSE of one softmax over the union of two key sets
// ([rows][dim] fp32 outputs, [rows] LSEs; dim a multiple of 4).
hipError_t launch_lse_merge(const float* oa, const float* la, const float* ob, const float* lb, int rows, int dim,
                            float* o, float* lse, hipStream_t s, const KEvents& ev = {});

// FP4 fake quantisation of n values (n a multiple of 32), fp32 or bf16.
hipError_t launch_fake_quant(const void* x, void* y, int64_t n, bool bf16, hipStream_t s, const KEvents& ev = {});

}  // namespace csa2
