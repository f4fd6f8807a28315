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
// descending" and no two entries tie.  The indexer has left a candidate list
// per query (indices and 32-bit score keys) that holds every entry at or
// above a key floor; the histogram of the candidates' top 11 key bits is
// counted here from the list:
//   - per-query scan: each 2,048-entry chunk kept its entries at or above its
//     own floor; a chunk whose floor lies above the bin of the k-th candidate
//     key may have left out entries of the Top-k, so this kernel scores that
//     chunk again (the scan's arithmetic, identical bits) and adds its
//     entries at or above that bin before selecting;
//   - dense prefill indexer: every entry at or above a sampled threshold, and
//     every entry of queries the threshold left short.
// One workgroup per query: a block scan over the histogram fixes the 11-bit
// prefix P holding the k-th key; candidates above P are selected, those equal
// to P are parked in LDS and refined digit by digit (heavily tied inputs
// first refine over the candidate list in global memory), the chosen indices
// are marked in an LDS bitmap over the context and written in index order by
// a block-wide prefix count (a bitonic sort when the context is too long for
// the bitmap).  It leaves the query's counters and threshold zeroed for the
// next call.
#include "csa2_device.h"
#include "csa2_internal.h"
#include "csa2_select.h"

namespace csa2 {

namespace {

constexpr int kSelCap = 2048;
constexpr int kRepairWaves = 8;             // waves of the final workgroup that rescore a chunk

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
// final
// ---------------------------------------------------------------------------
namespace {

struct SelShared {
  alignas(16) uint32_t h[kHistBins];
  int32_t sel[kSelCap];
  uint64_t tie[kTieCap];                        // parked keys; reused as the output bitmap
  uint32_t scratch[kSelectThreads / 64];
  uint32_t res[2];
  uint32_t res2[2];
  int32_t selcnt;
  int32_t tiecnt;
  int32_t repair;
};
static_assert(sizeof(uint64_t) * kTieCap >= (size_t)kRepairWaves * kFp8SlotBytes,
              "the parking buffer holds the repairing waves' operand slots");

}  // namespace

__global__ void __launch_bounds__(kSelectThreads)
topk_final_kernel(IndexWs ws, ScanArgs sa, const int32_t* __restrict__ q_vis, int k,
                  int32_t* __restrict__ out_idx, int32_t* __restrict__ out_cnt) {
  __shared__ SelShared S;
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = clamp_vis(q_vis[q], ws);
  const int32_t* cand = ws.cand + (int64_t)q * ws.vstride;
  const uint32_t* ckey = ws.ckey + (int64_t)q * ws.vstride;
  int32_t* oi = out_idx + (int64_t)q * k;

  if (V <= k) {                                       // everything visible is selected
    for (int i = tid; i < k; i += kSelectThreads) oi[i] = i < V ? i : -1;
    if (tid == 0) { out_cnt[q] = V; ws.cand_cnt[q] = 0; ws.tau[q] = 0.0f; ws.cnt2[q] = 0; }
    return;
  }
  // the candidate count: the dense indexer's full rescore appended after its
  // first pass's candidates
  const int nc = (int)ws.cand_cnt[q] + (ws.floor != nullptr ? 0 : (int)ws.cnt2[q]);
  // the histogram of the candidates' keys
  for (int i = tid; i < kHistBins; i += kSelectThreads) S.h[i] = 0;
  lds_barrier();
  for (int i = tid; i < nc; i += kSelectThreads) atomicAdd(&S.h[ckey[i] >> (32 - kHistBits)], 1u);
  if (tid == 0) { S.selcnt = 0; S.tiecnt = 0; S.repair = 0; }
  lds_barrier();

  uint32_t need = (uint32_t)k;
  int nbits = kHistBits;
  find_digit(S.h, kHistBins, need, S.res);
  int dstar = (int)S.res[0];

  if (ws.floor != nullptr) {
    // The k-th candidate key to 22 bits: a second digit over the candidates
    // in its 11-bit bin (counted into the parking buffer, free until later).
    const int ncand0 = ws.cand_cnt[q];
    const uint32_t* ckey_r = ws.ckey + (int64_t)q * ws.vstride;
    uint32_t* const h2 = reinterpret_cast<uint32_t*>(S.tie);
    for (int i = tid; i < kHistBins; i += kSelectThreads) h2[i] = 0;
    lds_barrier();
    for (int i = tid; i < ncand0; i += kSelectThreads) {
      const uint32_t key = ckey_r[i];
      if ((int)(key >> (32 - kHistBits)) == dstar) atomicAdd(&h2[(key >> (32 - 2 * kHistBits)) & (kHistBins - 1)], 1u);
    }
    lds_barrier();
    find_digit(h2, kHistBins, need - S.res[1], S.res2);
    // Every entry a chunk left out has a key below the chunk's floor.  A chunk
    // whose floor lies above the k-th candidate key's 22-bit prefix pfloor may
    // have left out entries at or above the k-th key: rescore it (same
    // arithmetic as the scan) and add its entries in [pfloor, floor); the k-th
    // key can only rise, so afterwards every entry at or above it is a
    // candidate (rare: it takes more of the Top-k in one chunk than it keeps).
    const uint32_t pfloor = ((uint32_t)dstar << (32 - kHistBits)) | (S.res2[0] << (32 - 2 * kHistBits));
    const int nch = (V + kScanChunk - 1) / kScanChunk;
    const uint32_t* fl = ws.floor + (int64_t)q * ws.fstride;
    for (int cc = tid; cc < nch; cc += kSelectThreads)
      if (fl[cc] > pfloor) atomicOr(&S.repair, 1);
    lds_barrier();
    if (S.repair) {
      const int lane_r = tid & 63, wave_r = tid >> 6;
      const int g = lane_r >> 4, r = lane_r & 15;
      intx8 a = {0, 0, 0, 0, 0, 0, 0, 0};
      float wv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (wave_r < kRepairWaves) {
        if (r < sa.h_idx) a = load_fp8_operand(sa.q_idx + ((int64_t)q * sa.h_idx + r) * kIndexDim, g);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          wv[i] = (4 * g + i < sa.h_idx) ? sa.w[(int64_t)q * sa.h_idx + 4 * g + i] : 0.0f;
      }
      // the parking buffer is free until the candidates are read: it holds
      // the repairing waves' operand slots
      uint8_t* const slot = reinterpret_cast<uint8_t*>(S.tie) + wave_r * kFp8SlotBytes;
      const int32_t* pt_row = sa.c.page_table + (int64_t)sa.q_seq[q] * sa.c.max_pages;
      int32_t* cand_w = ws.cand + (int64_t)q * ws.vstride;
      uint32_t* ckey_w = ws.ckey + (int64_t)q * ws.vstride;
      for (int cc = 0; cc < nch; ++cc) {
        const uint32_t fc = fl[cc];                   // uniform
        if (fc <= pfloor || wave_r >= kRepairWaves) continue;
        const int c0 = cc * kScanChunk, c1 = min(V, c0 + kScanChunk);
        const int ntl = (c1 - c0 + 15) >> 4;
        for (int j = wave_r; j < ntl; j += kRepairWaves) {
          const int ts = c0 + 16 * j;                 // tiles never straddle pages
          const int page = clamp_page(pt_row[ts >> sa.c.lg_page], sa.c);
          const intx8 lin = load_fp8_tile_linear(
              sa.c.idx_k + (((int64_t)page << sa.c.lg_page) + (ts & ((1 << sa.c.lg_page) - 1))) * kIndexDim, lane_r);
          const float sv = tile_score(a, wv, slot, lin, lane_r);
          const uint32_t key = score_key(sv);
          const int t = ts + r;
          // entries below the chunk's floor that reach the k-th candidate's bin
          const bool add = g == 0 && t < c1 && key >= pfloor && key < fc;
          const uint64_t m = __builtin_amdgcn_ballot_w64(add);
          if (m) {
            const int leader = __builtin_ctzll(m);
            int b0 = 0;
            if (lane_r == leader) b0 = (int)atomicAdd(&ws.cand_cnt[q], (uint32_t)__builtin_popcountll(m));
            b0 = __builtin_amdgcn_readlane(b0, leader);
            const int pos = b0 + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            if (add) {
              cand_w[pos] = t;
              ckey_w[pos] = key;
              atomicAdd(&S.h[key >> (32 - kHistBits)], 1u);
            }
          }
        }
      }
      __syncthreads();                                // new candidates (global) and histogram counts complete
      find_digit(S.h, kHistBins, need, S.res);
      dstar = (int)S.res[0];
    }
  }
  // the count as the repair left it (an atomic load: other waves added to it)
  const int ncand = ws.floor != nullptr
                        ? (int)__hip_atomic_load(&ws.cand_cnt[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        : nc;
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
  if (tid == 0) { out_cnt[q] = k; ws.cand_cnt[q] = 0; ws.tau[q] = 0.0f; ws.cnt2[q] = 0; }
}

hipError_t launch_topk_final(const IndexWs& ws, const ScanArgs& sa, const int32_t* q_vis, int nq, int k,
                             int32_t* out_idx, int32_t* out_cnt, hipStream_t s, const KEvents& ev) {
  if (nq <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  launch(topk_final_kernel, dim3(nq), dim3(kSelectThreads), s, ev, ws, sa, q_vis, k, out_idx, out_cnt);
  return hipGetLastError();
}

}  // namespace csa2
