// Hierarchical indexer: a later (Reindex) indexer scores only the shared
// candidate pool an earlier indexer chose, and keeps its Top-K among the
// pool ("DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression",
// Method: the Hierarchical Sparse Indexer restricts later indexers to a
// shared candidate pool chosen by an earlier one).  The pool is the earlier
// layer's own Top-P (ascending entry indices), the reading stated in csa2.h.
//
// pool_scan_kernel: the decode scan's arithmetic on gathered rows.  A 16-entry
// tile is 16 pool entries: lane l loads 32 bytes of entry (l / 4)'s indexer-K
// row, the wave's LDS slot turns the tile into the V_MFMA_F32_16X16X128_F8F6F4
// operand (same layout, same product, same ReLU * w reduction as the scan), so
// a pool entry's score has the bits the exhaustive scan gives it.
//
// pool_select_kernel: one workgroup per query; the pool's (score, position)
// keys are sorted in LDS (bitonic, at most 2,048 keys), the first k positions
// are flagged, and the flagged pool entries are written in pool order, which
// is ascending entry order.
#include "csa2.h"
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kPoolWaves = 4;
constexpr int kPoolChunk = 256;               // pool entries per scan workgroup
constexpr int kPoolSelectThreads = 1024;

__global__ void __launch_bounds__(kPoolWaves * 64)
pool_scan_kernel(CacheArgs c, const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                 const int32_t* __restrict__ q_seq, const int32_t* __restrict__ pool,
                 const int32_t* __restrict__ pool_cnt, int nq, int h_idx, int p, int nchunks, float* __restrict__ sc,
                 int pstride) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[kPoolWaves][kFp8SlotBytes];
  const int q = blockIdx.x / nchunks;
  const int chunk = blockIdx.x - q * nchunks;
  const int n = min(pool_cnt[q], p);
  const int e0 = chunk * kPoolChunk;
  if (e0 >= n) return;                                   // uniform
  const int e1 = min(n, e0 + kPoolChunk);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
  intx8 a = {0, 0, 0, 0, 0, 0, 0, 0};
  if (r < h_idx) a = load_fp8_operand(q_idx + ((int64_t)q * h_idx + r) * kIndexDim, g);
  float wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wv[i] = (4 * g + i < h_idx) ? w[(int64_t)q * h_idx + 4 * g + i] : 0.0f;
  const int32_t* pt_row = c.page_table + (int64_t)q_seq[q] * c.max_pages;
  const int32_t* prow = pool + (int64_t)q * p;
  const int t_max = (c.max_pages << c.lg_page) - 1;     // keeps a bad pool entry inside the page table
  float* srow = sc + (int64_t)q * pstride;
  uint8_t* const slot = stage[wave];
  const int ntiles = (e1 - e0 + 15) >> 4;
  // tiles j = wave, wave + 4, ...: gather lane l's 32 bytes of entry l / 4
  auto load = [&](int j, intx8& lin) {
    const int pos = min(e0 + 16 * j + (lane >> 2), e1 - 1);
    const int64_t row = entry_row(pt_row, min(max(prow[pos], 0), t_max), c.lg_page);
    const uint8_t* src = c.idx_k + row * kIndexDim + 32 * (lane & 3);
    const intx4 lo = *reinterpret_cast<const intx4*>(src);
    const intx4 hi = *reinterpret_cast<const intx4*>(src + 16);
    lin = intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  intx8 cur, nxt;
  load(wave, cur);
  for (int j = wave; j < ntiles; j += kPoolWaves) {
    load(min(j + kPoolWaves, ntiles - 1), nxt);
    const intx8 b = fp8_tile_operand(slot, cur, lane);
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
    const float part = halves_sum(rows_pair_sum(relu_weighted(acc, wv)));   // every lane: entry r's score
    uint32_t u32 = __float_as_uint(part);
    if ((u32 << 1) == 0) u32 = 0;                         // -0 -> +0
    const int pos = min(e0 + 16 * j + r, pstride - 1);    // positions past the count are never read
    srow[pos] = __uint_as_float(u32);
    cur = nxt;
  }
}

// Top-k of one query's pool.  Keys (score key << 32) | ~position order as
// (score descending, position ascending) = (score descending, entry index
// ascending), the pool being ascending; padding keys are 0 (below every key).
__global__ void __launch_bounds__(kPoolSelectThreads)
pool_select_kernel(const int32_t* __restrict__ pool, const int32_t* __restrict__ pool_cnt, int p, const float* sc,
                   int pstride, int k, int32_t* __restrict__ out_idx, int32_t* __restrict__ out_cnt) {
  __shared__ uint64_t key[CSA2_MAX_K];
  __shared__ uint8_t flag[CSA2_MAX_K];
  __shared__ uint32_t wsum[kPoolSelectThreads / 64];
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = max(0, min(pool_cnt[q], p));
  const int kp = min(k, n);
  const int32_t* prow = pool + (int64_t)q * p;
  int32_t* orow = out_idx + (int64_t)q * k;
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (int i = tid; i < n2; i += kPoolSelectThreads) {
    key[i] = i < n ? ((uint64_t)score_key(sc[(int64_t)q * pstride + i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i)
                   : 0ull;
    flag[i] = 0;
  }
  lds_barrier();
  for (int size = 2; size <= n2; size <<= 1) {           // bitonic sort, descending
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n2 / 2; i += kPoolSelectThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t x = key[lo], y = key[hi];
        if ((x < y) == desc) { key[lo] = y; key[hi] = x; }
      }
      lds_barrier();
    }
  }
  for (int i = tid; i < kp; i += kPoolSelectThreads) flag[0xFFFFFFFFu - (uint32_t)key[i]] = 1;
  lds_barrier();
  // flagged positions in pool order: thread t owns positions [2t, 2t + 2)
  const int p0 = 2 * tid;
  const uint32_t mine = (p0 < n ? flag[p0] : 0) + (p0 + 1 < n ? flag[p0 + 1] : 0);
  uint32_t x = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  lds_barrier();
  uint32_t pos = x - mine;
  for (int i = 0; i < wave; ++i) pos += wsum[i];
  if (p0 < n && flag[p0]) orow[pos++] = prow[p0];
  if (p0 + 1 < n && flag[p0 + 1]) orow[pos] = prow[p0 + 1];
  for (int i = kp + tid; i < k; i += kPoolSelectThreads) orow[i] = -1;
  if (tid == 0) out_cnt[q] = kp;
}

size_t pool_score_bytes(int nq, int p) { return (size_t)nq * ((p + 63) / 64 * 64) * 4; }

hipError_t launch_pool_index(const CacheArgs& c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                             const int32_t* pool, const int32_t* pool_cnt, int nq, int h_idx, int p, int k,
                             int32_t* out_idx, int32_t* out_cnt, float* sc, hipStream_t s, const KEvents& ev_scan,
                             const KEvents& ev_select) {
  if (nq <= 0) {
    record_empty(ev_scan, s);
    record_empty(ev_select, s);
    return hipSuccess;
  }
  const int pstride = (p + 63) / 64 * 64;
  const int nchunks = (p + kPoolChunk - 1) / kPoolChunk;
  launch(pool_scan_kernel, dim3((unsigned)((int64_t)nq * nchunks)), dim3(kPoolWaves * 64), s, ev_scan, c, q_idx, w,
         q_seq, pool, pool_cnt, nq, h_idx, p, nchunks, sc, pstride);
  launch(pool_select_kernel, dim3((unsigned)nq), dim3(kPoolSelectThreads), s, ev_select, pool, pool_cnt, p,
         (const float*)sc, pstride, k, out_idx, out_cnt);
  return hipGetLastError();
}

}  // namespace csa2
