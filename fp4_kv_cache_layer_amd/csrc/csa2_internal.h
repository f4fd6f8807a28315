// Internal launchers of the CSA2 kernels (not part of the C ABI).
#pragma once
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

// Workspace layout of the indexer: [hist: nq * 2048 u32][scores: nq * vstride f32]
struct IndexWs {
  uint32_t* hist;
  float* scores;
  int64_t vstride;
};

constexpr int kScanChunk = 2048;             // entries per scan workgroup
constexpr int kSelectThreads = 1024;
constexpr int kTieCap = 12288;               // composite keys held in LDS by the select kernel

int64_t index_vstride(int32_t max_vis);
size_t index_ws_bytes(int32_t nq, int32_t max_vis);
IndexWs index_ws_carve(void* ws, int32_t nq, int32_t max_vis);

hipError_t launch_append_quant(uint8_t* kv, uint8_t* idx_k, const int32_t* slots, const uint16_t* kv_rows,
                               const uint16_t* idxk_rows, int n, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

hipError_t launch_index_scan(const CacheArgs& c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                             const int32_t* q_vis, int nq, int h_idx, int max_vis, const IndexWs& ws,
                             hipStream_t s);

hipError_t launch_topk_select(const IndexWs& ws, const int32_t* q_vis, int nq, int k, int32_t* out_idx,
                              int32_t* out_cnt, hipStream_t s);

hipError_t launch_sparse_attn(const CacheArgs& c, const uint16_t* q, const int32_t* q_seq, const int32_t* idx,
                              const int32_t* cnt, int nq, int h, int k, float sm_scale, float* out, float* lse,
                              hipStream_t s);

}  // namespace csa2
