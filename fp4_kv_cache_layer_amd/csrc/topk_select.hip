// Top-K select: for each query, the first min(k, V) entries under the order
// (score descending, index ascending), written in ascending index order.
//
// Top-512 selection per query is the CSA2 Full/Reindex output ("Unlocking
// Extreme Context Scaling with DeepSeek-V4.1-Flash", section "Compressed
// Sparse Attention 2 (CSA2)"); the tie rule (lower index first) is the
// reading stated in csa2.h.
//
// Every entry gets the unique 64-bit key C = (orderable score << 32) |
// (0xFFFFFFFF - index), so "score descending, index ascending" is "C
// descending" and no two entries tie.  One 1024-thread workgroup per query:
//   1. the scan already histogrammed the top 11 bits of C; a block scan over
//      that histogram fixes the 11-bit prefix P that holds the k-th key;
//   2. while more than kTieCap keys share the prefix (only for heavily tied
//      inputs), one more pass over the scores histograms the next digit;
//   3. one pass over the scores takes every entry whose prefix is above P and
//      parks the entries equal to P in LDS;
//   4. radix refinement of the parked keys in LDS finishes the selection;
//   5. a bitonic sort puts the chosen indices in ascending order.
// The histogram rows the scan filled are zeroed here, ready for the next call.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {

__device__ __forceinline__ uint64_t composite(float s, int t) {
  return ((uint64_t)score_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
}

constexpr int CSA2_SEL_CAP = 2048;

struct SelShared {
  uint32_t h[kHistBins];
  int32_t sel[CSA2_SEL_CAP];
  uint64_t tie[kTieCap];
  uint32_t wave_tot[kSelectThreads / 64];
  int32_t dstar;
  uint32_t above;
  int32_t selcnt;
  int32_t tiecnt;
};

// Given hist[0..nb) in LDS (nb <= 2048) and need >= 1, finds the largest digit
// d* whose suffix count reaches need; returns d* and the count strictly above.
__device__ void find_digit(SelShared& S, int nb, uint32_t need, int& dstar, uint32_t& above) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // thread tid covers descending positions 2*tid, 2*tid+1 -> digits nb-1-2tid, nb-2-2tid
  const int d0 = nb - 1 - 2 * tid, d1 = nb - 2 - 2 * tid;
  const uint32_t v0 = d0 >= 0 ? S.h[d0] : 0u;
  const uint32_t v1 = d1 >= 0 ? S.h[d1] : 0u;
  uint32_t x = v0 + v1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) S.wave_tot[wave] = x;
  __syncthreads();
  uint32_t off = 0;
  for (int i = 0; i < wave; ++i) off += S.wave_tot[i];
  const uint32_t incl = x + off, excl = incl - v0 - v1;
  if (d0 >= 0 && excl < need && need <= excl + v0) { S.dstar = d0; S.above = excl; }
  if (d1 >= 0 && excl + v0 < need && need <= excl + v0 + v1) { S.dstar = d1; S.above = excl + v0; }
  __syncthreads();
  dstar = S.dstar;
  above = S.above;
  __syncthreads();
}

}  // namespace

__global__ void __launch_bounds__(kSelectThreads)
topk_select_kernel(IndexWs ws, const int32_t* __restrict__ q_vis, int k,
                   int32_t* __restrict__ out_idx, int32_t* __restrict__ out_cnt) {
  __shared__ SelShared S;
  const int q = blockIdx.x, tid = threadIdx.x;
  const int V = q_vis[q];
  uint32_t* gh = ws.hist + (int64_t)q * kHistBins;
  const float* sc = ws.scores + (int64_t)q * ws.vstride;
  int32_t* oi = out_idx + (int64_t)q * k;

  if (V <= k) {                                       // everything visible is selected
    for (int i = tid; i < kHistBins; i += kSelectThreads) gh[i] = 0;
    for (int i = tid; i < k; i += kSelectThreads) oi[i] = i < V ? i : -1;
    if (tid == 0) out_cnt[q] = V;
    return;
  }
  for (int i = tid; i < kHistBins; i += kSelectThreads) { S.h[i] = gh[i]; gh[i] = 0; }
  if (tid == 0) { S.selcnt = 0; S.tiecnt = 0; }
  __syncthreads();

  uint32_t need = (uint32_t)k;
  int nbits = kHistBits;
  int dstar;
  uint32_t above;
  find_digit(S, kHistBins, need, dstar, above);
  uint64_t P = (uint64_t)dstar;
  need -= above;
  uint32_t cnt_eq = S.h[dstar];
  __syncthreads();

  // 2. global refinement while the prefix class is too large for LDS
  while (cnt_eq > (uint32_t)kTieCap) {
    const int d = min(kHistBits, 64 - nbits);
    for (int i = tid; i < (1 << d); i += kSelectThreads) S.h[i] = 0;
    __syncthreads();
    for (int t = tid; t < V; t += kSelectThreads) {
      const uint64_t C = composite(sc[t], t);
      if ((C >> (64 - nbits)) == P) atomicAdd(&S.h[(uint32_t)(C >> (64 - nbits - d)) & ((1u << d) - 1)], 1u);
    }
    __syncthreads();
    find_digit(S, 1 << d, need, dstar, above);
    need -= above;
    P = (P << d) | (uint64_t)dstar;
    nbits += d;
    cnt_eq = S.h[dstar];
    __syncthreads();
  }

  // 3. collect: prefix above P -> selected; prefix equal to P -> parked
  for (int t = tid; t < V; t += kSelectThreads) {
    const uint64_t C = composite(sc[t], t);
    const uint64_t pre = C >> (64 - nbits);
    if (pre > P) {
      const int pos = atomicAdd(&S.selcnt, 1);
      if (pos < CSA2_SEL_CAP) S.sel[pos] = t;
    } else if (pre == P) {
      const int pos = atomicAdd(&S.tiecnt, 1);
      if (pos < kTieCap) S.tie[pos] = C;
    }
  }
  __syncthreads();
  const int ntie = min(S.tiecnt, kTieCap);

  // 4. refine the parked keys (dropped entries become 0, never a valid key)
  while (need > 0) {
    if (cnt_eq == need) {
      for (int i = tid; i < ntie; i += kSelectThreads) {
        const uint64_t C = S.tie[i];
        if (C) {
          const int pos = atomicAdd(&S.selcnt, 1);
          if (pos < CSA2_SEL_CAP) S.sel[pos] = (int32_t)(0xFFFFFFFFu - (uint32_t)C);
        }
      }
      __syncthreads();
      break;
    }
    const int d = min(kHistBits, 64 - nbits);
    if (d <= 0) break;
    const int sh = 64 - nbits - d;
    for (int i = tid; i < (1 << d); i += kSelectThreads) S.h[i] = 0;
    __syncthreads();
    for (int i = tid; i < ntie; i += kSelectThreads) {
      const uint64_t C = S.tie[i];
      if (C) atomicAdd(&S.h[(uint32_t)(C >> sh) & ((1u << d) - 1)], 1u);
    }
    __syncthreads();
    find_digit(S, 1 << d, need, dstar, above);
    for (int i = tid; i < ntie; i += kSelectThreads) {
      const uint64_t C = S.tie[i];
      if (!C) continue;
      const int dig = (int)((uint32_t)(C >> sh) & ((1u << d) - 1));
      if (dig > dstar) {
        const int pos = atomicAdd(&S.selcnt, 1);
        if (pos < CSA2_SEL_CAP) S.sel[pos] = (int32_t)(0xFFFFFFFFu - (uint32_t)C);
        S.tie[i] = 0;
      } else if (dig < dstar) {
        S.tie[i] = 0;
      }
    }
    need -= above;
    nbits += d;
    P = (P << d) | (uint64_t)dstar;
    cnt_eq = S.h[dstar];
    __syncthreads();
  }

  // 5. ascending order: bitonic sort of k indices padded to a power of two
  int n2 = 1;
  while (n2 < k) n2 <<= 1;
  for (int i = tid; i < n2; i += kSelectThreads)
    if (i >= min(k, S.selcnt)) S.sel[i] = 0x7FFFFFFF;
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n2 / 2; i += kSelectThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const int32_t a = S.sel[lo], b = S.sel[hi];
        if ((a > b) == up) { S.sel[lo] = b; S.sel[hi] = a; }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += kSelectThreads) oi[i] = S.sel[i];
  if (tid == 0) out_cnt[q] = k;
}

hipError_t launch_topk_select(const IndexWs& ws, const int32_t* q_vis, int nq, int k, int32_t* out_idx,
                              int32_t* out_cnt, hipStream_t s) {
  hipLaunchKernelGGL(topk_select_kernel, dim3(nq), dim3(kSelectThreads), 0, s, ws, q_vis, k, out_idx, out_cnt);
  return hipGetLastError();
}

}  // namespace csa2
