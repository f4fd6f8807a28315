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
// descending" and no two entries tie.  The indexer scan has already
// histogrammed the top 11 bits of every key; a block scan over that histogram
// fixes the 11-bit prefix P holding the k-th key.  Then:
//
//  collect (one workgroup per 8K-entry slice of a query, so the score pass is
//          spread over the whole chip): every entry whose score reaches the
//          lowest score of prefix P is appended to an LDS list, which is
//          copied to the query's candidate list after one global atomic
//          reserves its place;
//  final   (one workgroup per query): candidates above P are selected, those
//          equal to P are parked in LDS and refined digit by digit (heavily
//          tied inputs first refine over the candidate list in global memory),
//          the chosen indices are marked in an LDS bitmap over the context
//          and written in index order by a block-wide prefix count (a bitonic
//          sort when the context is too long for the bitmap).  It leaves the
//          query's histogram row and candidate counter zeroed for the next call.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {

constexpr int kSelCap = 2048;
constexpr int kCollectThreads = 256;

// Lowest float whose orderable key is >= key (scores are canonical: no -0, no NaN).
__device__ __forceinline__ float key_floor_float(uint32_t key) {
  if (key == 0) return -INFINITY;
  const uint32_t bits = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(bits);
}

// Search over a descending-ordered histogram h[0..nb) (nb <= 2048): the
// largest digit d* whose suffix count reaches need (1 <= need <= total), and
// the count strictly above it, written to result[0..1].  One wave does the
// search; the workgroup barrier at the end publishes the result.  Callers
// have h complete (a barrier) first.
__device__ void find_digit(const uint32_t* h, int nb, uint32_t need, uint32_t* result) {
  if ((threadIdx.x >> 6) == 0) {
    const int lane = threadIdx.x & 63;
    if (nb == kHistBins) {
      // Lane l sums the digits [base, base + 32), base = nb - 32 (l + 1)
      // (descending positions 32l .. 32l+31), reading its eight 16-byte
      // pieces in a lane-rotated order so the wave's reads spread over the
      // banks; a wave scan finds the lane L whose range holds d*.  Then lanes
      // 0..31 take one digit each of L's range, descending, and a second scan
      // finds d* itself.
      const int base = nb - 32 * (lane + 1);
      uint32_t mine = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint4 w = *reinterpret_cast<const uint4*>(h + base + 4 * ((j + lane) & 7));
        mine += (w.x + w.y) + (w.z + w.w);
      }
      const uint32_t x = wave_incl_sum(mine);
      const uint64_t hm = __builtin_amdgcn_ballot_w64(x - mine < need && need <= x);
      const int L = __builtin_ctzll(hm);
      const uint32_t run0 = __builtin_amdgcn_readlane(x - mine, L);
      const int dig = nb - 1 - 32 * L - lane;                 // lanes 0..31: L's digits, descending
      const uint32_t hv = h[lane < 32 ? dig : 0];
      const uint32_t c = lane < 32 ? hv : 0u;
      const uint32_t y = wave_incl_sum(c) + run0;
      const uint64_t dm = __builtin_amdgcn_ballot_w64(lane < 32 && need <= y && y - c < need);
      const int L2 = __builtin_ctzll(dm);
      const uint32_t above = __builtin_amdgcn_readlane(y - c, L2);
      if (lane == 0) {
        result[0] = (uint32_t)(nb - 1 - 32 * L - L2);
        result[1] = above;
      }
    } else {
      const int per = (nb + 63) >> 6;
      const int p0 = min(nb, lane * per), p1 = min(nb, p0 + per);
      uint32_t mine = 0;
      for (int p = p0; p < p1; ++p) mine += h[nb - 1 - p];
      const uint32_t x = wave_incl_sum(mine);
      const uint32_t excl = x - mine;
      if (excl < need && need <= x) {
        uint32_t run = excl;
        for (int p = p0; p < p1; ++p) {
          const uint32_t c = h[nb - 1 - p];
          if (need <= run + c) { result[0] = (uint32_t)(nb - 1 - p); result[1] = run; break; }
          run += c;
        }
      }
    }
  }
  lds_barrier();
}

// Appends value for every lane where flag holds, one atomic per wave.
template <typename T>
__device__ __forceinline__ void wave_append(bool flag, T value, int* counter, T* list, int cap) {
  const uint64_t m = __builtin_amdgcn_ballot_w64(flag);
  if (m == 0) return;
  const int lane = threadIdx.x & 63;
  const int leader = __builtin_ctzll(m);
  int base = 0;
  if (lane == leader) base = atomicAdd(counter, __builtin_popcountll(m));
  base = __builtin_amdgcn_readlane(base, leader);
  const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
  if (flag && pos < cap) list[pos] = value;
}

}  // namespace

// ---------------------------------------------------------------------------
// collect
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kCollectThreads)
topk_collect_kernel(IndexWs ws, const int32_t* __restrict__ q_vis, int k, int nslices) {
  __shared__ __attribute__((aligned(16))) uint32_t h[kHistBins];
  __shared__ int32_t list[kCollectSlice];             // this slice's candidates
  __shared__ uint32_t klist[kCollectSlice];           // and their score keys
  __shared__ uint32_t res[2];
  __shared__ int count, base;
  const int q = blockIdx.x / nslices;
  const int slice = blockIdx.x - q * nslices;
  const int V = clamp_vis(q_vis[q], ws);
  const int t0 = slice * kCollectSlice;
  if (V <= k || t0 >= V) return;                      // uniform
  const int tid = threadIdx.x;
  const int t1 = min(V, t0 + kCollectSlice);
  // the histogram row first, then the slice's scores (indices clamped, entries past t1 ignored)
  const uint32_t* gh = ws.hist + (int64_t)q * kHistBins;
  for (int i = tid; i < kHistBins; i += kCollectThreads) h[i] = gh[i];
  constexpr int kPer = kCollectSlice / (4 * kCollectThreads);   // float4 loads per thread
  const float4* sc4 = reinterpret_cast<const float4*>(ws.scores + (int64_t)q * ws.vstride + t0);
  const int nvec = (t1 - t0 + 3) >> 2;
  float4 v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) v[u] = sc4[min(u * kCollectThreads + tid, nvec - 1)];
  if (tid == 0) count = 0;
  lds_barrier();
  find_digit(h, kHistBins, (uint32_t)k, res);
  const float floor_s = key_floor_float(res[0] << (32 - kHistBits));
  // count this thread's candidates, one scan and one reservation per wave,
  // then write them in order
  uint32_t mine = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int vi = u * kCollectThreads + tid;
    const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) mine += (t0 + 4 * vi + c < t1 && e[c] >= floor_s) ? 1u : 0u;
  }
  const int lane = tid & 63;
  const uint32_t x = wave_incl_sum(mine);
  int wbase = 0;
  if (lane == 63 && x) wbase = atomicAdd(&count, (int)x);
  int pos = __shfl(wbase, 63) + (int)(x - mine);
  if (mine) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int vi = u * kCollectThreads + tid;
      const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int t = t0 + 4 * vi + c;
        if (t < t1 && e[c] >= floor_s) {                  // at most kCollectSlice entries in all
          list[pos] = t;
          klist[pos++] = score_key(e[c]);
        }
      }
    }
  }
  lds_barrier();
  // one global reservation per workgroup, then a coalesced copy of the list
  const int n = count;
  if (n == 0) return;
  if (tid == 0) base = atomicAdd(&ws.cand_cnt[q], (uint32_t)n);
  lds_barrier();
  int32_t* cand = ws.cand + (int64_t)q * ws.vstride + base;
  uint32_t* ckey = ws.ckey + (int64_t)q * ws.vstride + base;
  for (int i = tid; i < n; i += kCollectThreads) {
    cand[i] = list[i];
    ckey[i] = klist[i];
  }
}

// ---------------------------------------------------------------------------
// final
// ---------------------------------------------------------------------------
namespace {

struct SelShared {
  alignas(16) uint32_t h[kHistBins];
  int32_t sel[kSelCap];
  uint64_t tie[kTieCap];                        // parked keys; reused as the output bitmap
  uint32_t scratch[kSelectThreads / 64];
  uint32_t res[2];
  int32_t selcnt;
  int32_t tiecnt;
};

}  // namespace

__global__ void __launch_bounds__(kSelectThreads)
topk_final_kernel(IndexWs ws, const int32_t* __restrict__ q_vis, int k,
                  int32_t* __restrict__ out_idx, int32_t* __restrict__ out_cnt) {
  __shared__ SelShared S;
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = clamp_vis(q_vis[q], ws);
  uint32_t* gh = ws.hist + (int64_t)q * kHistBins;
  const int32_t* cand = ws.cand + (int64_t)q * ws.vstride;
  const uint32_t* ckey = ws.ckey + (int64_t)q * ws.vstride;
  int32_t* oi = out_idx + (int64_t)q * k;

  if (V <= k) {                                       // everything visible is selected
    for (int i = tid; i < kHistBins; i += kSelectThreads) gh[i] = 0;
    for (int i = tid; i < k; i += kSelectThreads) oi[i] = i < V ? i : -1;
    if (tid == 0) { out_cnt[q] = V; ws.cand_cnt[q] = 0; }
    return;
  }
  const int ncand = ws.cand_cnt[q];
  for (int i = tid; i < kHistBins; i += kSelectThreads) { S.h[i] = gh[i]; gh[i] = 0; }
  if (tid == 0) { S.selcnt = 0; S.tiecnt = 0; }
  lds_barrier();

  uint32_t need = (uint32_t)k;
  int nbits = kHistBits;
  find_digit(S.h, kHistBins, need, S.res);
  int dstar = (int)S.res[0];
  uint64_t P = (uint64_t)dstar;
  need -= S.res[1];
  uint32_t cnt_eq = S.h[dstar];
  lds_barrier();

  // heavily tied inputs: refine the prefix over the candidate list until its class fits in LDS
  while (cnt_eq > (uint32_t)kTieCap) {
    const int d = min(kHistBits, 64 - nbits);
    for (int i = tid; i < (1 << d); i += kSelectThreads) S.h[i] = 0;
    lds_barrier();
    for (int i = tid; i < ncand; i += kSelectThreads) {
      const int t = cand[i];
      const uint64_t C = ((uint64_t)ckey[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
      if ((C >> (64 - nbits)) == P) atomicAdd(&S.h[(uint32_t)(C >> (64 - nbits - d)) & ((1u << d) - 1)], 1u);
    }
    lds_barrier();
    find_digit(S.h, 1 << d, need, S.res);
    dstar = (int)S.res[0];
    need -= S.res[1];
    P = (P << d) | (uint64_t)dstar;
    nbits += d;
    cnt_eq = S.h[dstar];
    lds_barrier();
  }

  // candidates: prefix above P -> selected; prefix equal to P -> parked.
  // Batches of kCandBatch per thread: all their indices and keys are in
  // flight together.
  constexpr int kCandBatch = 4;
  for (int i0 = 0; i0 < ncand; i0 += kCandBatch * kSelectThreads) {
    int t[kCandBatch];
    uint32_t kv[kCandBatch];
#pragma unroll
    for (int b = 0; b < kCandBatch; ++b) {
      const int i = min(i0 + b * kSelectThreads + tid, ncand - 1);
      t[b] = cand[i];
      kv[b] = ckey[i];
    }
#pragma unroll
    for (int b = 0; b < kCandBatch; ++b) {
      const bool valid = i0 + b * kSelectThreads + tid < ncand;
      const uint64_t C = ((uint64_t)kv[b] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t[b]);
      const uint64_t pre = C >> (64 - nbits);
      wave_append<int32_t>(valid && pre > P, t[b], &S.selcnt, S.sel, kSelCap);
      wave_append<uint64_t>(valid && pre == P, C, &S.tiecnt, S.tie, kTieCap);
    }
  }
  lds_barrier();
  const int ntie = min(S.tiecnt, kTieCap);

  // refine the parked keys (dropped entries become 0, never a valid key)
  while (need > 0) {
    if (cnt_eq == need) {
      for (int i = tid; i < ntie; i += kSelectThreads) {
        const uint64_t C = S.tie[i];
        if (C) {
          const int pos = atomicAdd(&S.selcnt, 1);
          if (pos < kSelCap) S.sel[pos] = (int32_t)(0xFFFFFFFFu - (uint32_t)C);
        }
      }
      lds_barrier();
      break;
    }
    const int d = min(kHistBits, 64 - nbits);
    if (d <= 0) break;
    const int sh = 64 - nbits - d;
    for (int i = tid; i < (1 << d); i += kSelectThreads) S.h[i] = 0;
    lds_barrier();
    for (int i = tid; i < ntie; i += kSelectThreads) {
      const uint64_t C = S.tie[i];
      if (C) atomicAdd(&S.h[(uint32_t)(C >> sh) & ((1u << d) - 1)], 1u);
    }
    lds_barrier();
    find_digit(S.h, 1 << d, need, S.res);
    dstar = (int)S.res[0];
    for (int i = tid; i < ntie; i += kSelectThreads) {
      const uint64_t C = S.tie[i];
      if (!C) continue;
      const int dig = (int)((uint32_t)(C >> sh) & ((1u << d) - 1));
      if (dig > dstar) {
        const int pos = atomicAdd(&S.selcnt, 1);
        if (pos < kSelCap) S.sel[pos] = (int32_t)(0xFFFFFFFFu - (uint32_t)C);
        S.tie[i] = 0;
      } else if (dig < dstar) {
        S.tie[i] = 0;
      }
    }
    need -= S.res[1];
    nbits += d;
    P = (P << d) | (uint64_t)dstar;
    cnt_eq = S.h[dstar];
    lds_barrier();
  }

  // ascending order
  const int nsel = min(k, S.selcnt);
  const int nwords = (V + 31) >> 5;
  if (nwords <= kTieCap * 2) {
    // bitmap over the context in the (now free) parking buffer, then an
    // ordered compaction: thread t owns words [t*W, t*W + W)
    uint32_t* bm = reinterpret_cast<uint32_t*>(S.tie);
    for (int i = tid; i < nwords; i += kSelectThreads) bm[i] = 0;
    lds_barrier();
    for (int i = tid; i < nsel; i += kSelectThreads) {
      const int t = S.sel[i];
      atomicOr(&bm[t >> 5], 1u << (t & 31));
    }
    lds_barrier();
    const int W = (nwords + kSelectThreads - 1) / kSelectThreads;
    const int w0 = min(tid * W, nwords), w1 = min(w0 + W, nwords);
    uint32_t mine = 0;
    for (int i = w0; i < w1; ++i) mine += __builtin_popcount(bm[i]);
    const uint32_t x = wave_incl_sum(mine);
    if (lane == 63) S.scratch[wave] = x;
    lds_barrier();
    uint32_t pos = x - mine;
    for (int i = 0; i < wave; ++i) pos += S.scratch[i];
    for (int i = w0; i < w1; ++i) {
      uint32_t bits = bm[i];
      while (bits) {
        const int b = __builtin_ctz(bits);
        bits &= bits - 1;
        oi[pos++] = (i << 5) + b;
      }
    }
  } else {
    // bitonic sort of the k indices padded to a power of two
    int n2 = 1;
    while (n2 < k) n2 <<= 1;
    for (int i = tid; i < n2; i += kSelectThreads)
      if (i >= nsel) S.sel[i] = 0x7FFFFFFF;
    lds_barrier();
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < n2 / 2; i += kSelectThreads) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const int32_t a = S.sel[lo], b = S.sel[hi];
          if ((a > b) == up) { S.sel[lo] = b; S.sel[hi] = a; }
        }
        lds_barrier();
      }
    }
    for (int i = tid; i < k; i += kSelectThreads) oi[i] = S.sel[i];
  }
  if (tid == 0) { out_cnt[q] = k; ws.cand_cnt[q] = 0; }
}

hipError_t launch_topk_select(const IndexWs& ws, const int32_t* q_vis, int nq, int k, int max_vis,
                              int32_t* out_idx, int32_t* out_cnt, hipStream_t s, const KEvents& ev) {
  if (nq <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  const int nslices = max(1, (max_vis + kCollectSlice - 1) / kCollectSlice);
  launch(topk_collect_kernel, dim3((unsigned)((int64_t)nq * nslices)), dim3(kCollectThreads), s, ev.first(), ws,
         q_vis, k, nslices);
  launch(topk_final_kernel, dim3(nq), dim3(kSelectThreads), s, ev.last(), ws, q_vis, k, out_idx, out_cnt);
  return hipGetLastError();
}

hipError_t launch_topk_final(const IndexWs& ws, const int32_t* q_vis, int nq, int k, int32_t* out_idx,
                             int32_t* out_cnt, hipStream_t s, const KEvents& ev) {
  if (nq <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  launch(topk_final_kernel, dim3(nq), dim3(kSelectThreads), s, ev, ws, q_vis, k, out_idx, out_cnt);
  return hipGetLastError();
}

}  // namespace csa2
