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
// pool_select_kernel: one workgroup per query, four pool positions per
// thread.  A most-significant-digit-first radix search over the 32-bit score
// keys (four 8-bit digits, histograms in LDS, digit search by a DPP wave
// prefix sum) finds the k-th largest key T and how many entries tied at T
// still fit; the entries above T and the first of those tied at T in pool
// order are selected, and a block-wide prefix count writes them in pool
// order, which is ascending entry order.  Every load is issued unconditionally
// (positions clamped) so they are all in flight at once.
#include "csa2.h"
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kPoolWaves = 4;
constexpr int kPoolChunk = 16 * kPoolWaves;   // pool entries per scan workgroup: one tile per wave
constexpr int kPoolSelThreads = 512;
constexpr int kPoolPer = CSA2_MAX_K / kPoolSelThreads;   // pool positions per select thread

__global__ void __launch_bounds__(kPoolWaves * 64)
pool_scan_kernel(CacheArgs c, const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                 const int32_t* __restrict__ q_seq, const int32_t* __restrict__ pool,
                 const int32_t* __restrict__ pool_cnt, int nq, int h_idx, int p, int nchunks, float* __restrict__ sc,
                 int pstride) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[kPoolWaves][kFp8SlotBytes];
  const int q = blockIdx.x / nchunks;
  const int chunk = blockIdx.x - q * nchunks;
  const int n = min(pool_cnt[q], p);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e0 = chunk * kPoolChunk + 16 * wave;          // this wave's tile
  if (e0 >= n) return;                                     // uniform per wave; no workgroup barrier follows
  const int e1 = min(n, e0 + 16);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, r = lane & 15;
  // the tile's rows first (pool index -> page -> row: three dependent loads)
  const int32_t* pt_row = c.page_table + (int64_t)q_seq[q] * c.max_pages;
  const int t = pool[(int64_t)q * p + min(e0 + (lane >> 2), e1 - 1)];
  const int64_t row = entry_row_clamped(pt_row, t, c);   // a bad pool entry stays inside the cache
  const uint8_t* src = c.idx_k + row * kIndexDim + 32 * (lane & 3);
  const intx4 lo = *reinterpret_cast<const intx4*>(src);
  const intx4 hi = *reinterpret_cast<const intx4*>(src + 16);
  intx8 a = {0, 0, 0, 0, 0, 0, 0, 0};
  if (r < h_idx) a = load_fp8_operand(q_idx + ((int64_t)q * h_idx + r) * kIndexDim, g);
  float wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wv[i] = (4 * g + i < h_idx) ? w[(int64_t)q * h_idx + 4 * g + i] : 0.0f;
  // gathered rows take the scan's operand path, so every score has its bits
  const intx8 b = fp8_tile_operand(stage[wave], intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, lane);
  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
  const float part = halves_sum(rows_pair_sum(relu_weighted(acc, wv)));   // every lane: entry r's score
  uint32_t u32 = __float_as_uint(part);
  if ((u32 << 1) == 0) u32 = 0;                           // -0 -> +0
  if (g == 0 && e0 + r < e1) sc[(int64_t)q * pstride + e0 + r] = __uint_as_float(u32);
}

// Exclusive prefix sum of v over the workgroup (kPoolSelThreads threads);
// part must hold one slot per wave and not be in use by another scan.
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t v, uint32_t* part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_sum(v);
  if (lane == 63) part[wave] = x;
  lds_barrier();
  uint32_t base = 0;
  for (int i = 0; i < wave; ++i) base += part[i];
  return base + x - v;
}

// Scores: sc[q * sstride + position] (the pool scan's output).
__global__ void __launch_bounds__(kPoolSelThreads)
pool_select_kernel(const int32_t* __restrict__ pool, const int32_t* __restrict__ pool_cnt, int p,
                   const float* __restrict__ sc, int64_t sstride, int k, int32_t* __restrict__ out_idx,
                   int32_t* __restrict__ out_cnt) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t res[2];
  __shared__ uint32_t part[2][kPoolSelThreads / 64];
  const int q = blockIdx.x, tid = threadIdx.x;
  const int n = max(0, min(pool_cnt[q], p));
  const int kp = min(k, n);
  const int32_t* prow = pool + (int64_t)q * p;
  const float* srow = sc + q * sstride;
  int32_t* orow = out_idx + (int64_t)q * k;
  uint32_t key[kPoolPer];
  int32_t ent[kPoolPer];
  if (n == 0) {
    for (int i = tid; i < k; i += kPoolSelThreads) orow[i] = -1;
    if (tid == 0) out_cnt[q] = 0;
    return;
  }
#pragma unroll
  for (int i = 0; i < kPoolPer; ++i) ent[i] = prow[min(kPoolPer * tid + i, n - 1)];
#pragma unroll
  for (int i = 0; i < kPoolPer; ++i) key[i] = score_key(srow[min(kPoolPer * tid + i, n - 1)]);
  auto valid = [&](int i) { return kPoolPer * tid + i < n; };
  // threshold T: the kp-th largest key; need: how many keys equal to T are taken
  uint32_t T = 0, need = 0;
  if (kp < n) {
    uint32_t prefix = 0;
    need = (uint32_t)kp;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
      const int sh = 24 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      lds_barrier();
#pragma unroll
      for (int i = 0; i < kPoolPer; ++i)
        if (valid(i) && (pass == 0 || (key[i] >> (sh + 8)) == prefix)) atomicAdd(&hist[(key[i] >> sh) & 255u], 1u);
      lds_barrier();
      if (tid < 64) {
        // lane l: digits 255 - 4l - i, i = 0..3 (descending); the lane whose
        // range holds the need-th largest key resolves the digit
        uint32_t c[4], mine = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) { c[i] = hist[255 - 4 * tid - i]; mine += c[i]; }
        const uint32_t x = wave_incl_sum(mine);
        uint32_t run = x - mine;
        if (run < need && need <= x) {
          bool done = false;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (!done && need <= run + c[i]) {
              res[0] = 255u - 4u * tid - i;
              res[1] = run;
              done = true;
            }
            run += c[i];
          }
        }
      }
      lds_barrier();
      prefix = (prefix << 8) | res[0];
      need -= res[1];
    }
    T = prefix;
  }
  uint32_t eq = 0;
#pragma unroll
  for (int i = 0; i < kPoolPer; ++i) eq += (valid(i) && key[i] == T) ? 1u : 0u;
  uint32_t rank = block_excl_sum(eq, part[0]);             // tied keys before this thread's, in pool order
  uint32_t take = 0;
  bool sel[kPoolPer];
#pragma unroll
  for (int i = 0; i < kPoolPer; ++i) {
    const bool tie = valid(i) && key[i] == T;
    sel[i] = valid(i) && (kp == n || key[i] > T || (tie && rank < need));
    rank += tie ? 1u : 0u;
    take += sel[i] ? 1u : 0u;
  }
  uint32_t pos = block_excl_sum(take, part[1]);
#pragma unroll
  for (int i = 0; i < kPoolPer; ++i)
    if (sel[i] && pos < (uint32_t)k) orow[pos++] = ent[i];
  for (int i = kp + tid; i < k; i += kPoolSelThreads) orow[i] = -1;
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
  launch(pool_select_kernel, dim3((unsigned)nq), dim3(kPoolSelThreads), s, ev_select, pool, pool_cnt, p,
         (const float*)sc, (int64_t)pstride, k, out_idx, out_cnt);
  return hipGetLastError();
}

}  // namespace csa2
