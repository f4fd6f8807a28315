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
constexpr int kRegList = 4;                 // candidates per thread held in registers
constexpr int kListCap = kRegList * kSelectThreads;
constexpr int kRepairWaves = kSelectThreads / 64;                  // every wave rescores
constexpr int kRepairBatch = 8;                                     // tiles per wave with their loads in flight together
constexpr int kBlocksPerChunk = kScanChunk / kPruneBlockRows;       // 32
constexpr int kTilesPerBlock = kPruneBlockRows / 16;                // 4
constexpr int kPairCap = kTieCap * 2;                               // (chunk, block) pairs listed per pass

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
  int32_t ncand;                                // candidates, with those the repair appends
  int32_t npairs;                               // (chunk, block) pairs listed for the repair
};

}  // namespace

// kFloors: the per-query scan's candidates (ws.floor set; chunks may need
// rescoring), else the dense indexer's.  The dense form carries none of the
// rescoring code, so it keeps twice the occupancy for its many queries.
template <bool kFloors>
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
  const int nc = (int)ws.cand_cnt[q] + (kFloors ? 0 : (int)ws.cnt2[q]);
  // per-query scan: this thread's chunk floor, read now (used by the repair test)
  const int nch = (V + kScanChunk - 1) / kScanChunk;
  const uint32_t* fl = kFloors ? ws.floor + (int64_t)q * ws.fstride : nullptr;
  const uint32_t fl_mine = (kFloors && tid < nch) ? fl[tid] : 0u;
  // the histogram of the candidates' keys; a per-query scan's list of at
  // most kListCap candidates stays in registers (thread tid: entries tid +
  // 1,024 u), where the second digit and the partition read it, the indices'
  // loads completing while the digits are searched
  const bool in_regs = kFloors && nc <= kListCap;
  uint32_t rkey[kRegList];
  int32_t rcand[kRegList];
  for (int i = tid; i < kHistBins; i += kSelectThreads) S.h[i] = 0;
  lds_barrier();
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kRegList; ++u) rkey[u] = tid + u * kSelectThreads < nc ? ckey[tid + u * kSelectThreads] : 0u;
#pragma unroll
    for (int u = 0; u < kRegList; ++u)
      if (tid + u * kSelectThreads < nc) atomicAdd(&S.h[rkey[u] >> (32 - kHistBits)], 1u);
    // the indices are requested only now, so the histogram never waits for them
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kRegList; ++u) rcand[u] = tid + u * kSelectThreads < nc ? cand[tid + u * kSelectThreads] : 0;
  } else {
    for (int i = tid; i < nc; i += kSelectThreads) atomicAdd(&S.h[ckey[i] >> (32 - kHistBits)], 1u);
  }
  if (tid == 0) { S.selcnt = 0; S.tiecnt = 0; S.repair = 0; S.ncand = nc; }
  lds_barrier();

  uint32_t need = (uint32_t)k;
  int nbits = kHistBits;
  // Block-level pruning can leave a query with fewer than k candidates
  // (chunks keep only their top L, and pruned chunks none): then there is no
  // k-th candidate key yet, and the repair below, from the threshold alone,
  // brings in every entry that scores T or more, at least k of them.
  const bool short_list = kFloors && nc < k;
  int dstar = 0;
  // with no repair, the candidates' k-th key is known to 22 bits (its class
  // eq22 candidates wide, above22 above it) and the parking starts there
  bool digits22 = false;
  uint32_t eq22 = 0;
  if (!short_list) {
    find_digit(S.h, kHistBins, need, S.res);
    dstar = (int)S.res[0];
  }

  if constexpr (kFloors) {
    // The k-th candidate key to 22 bits: a second digit over the candidates
    // in its 11-bit bin (counted into the parking buffer, free until later).
    const int ncand0 = ws.cand_cnt[q];
    const uint32_t* ckey_r = ws.ckey + (int64_t)q * ws.vstride;
    uint32_t* const h2 = reinterpret_cast<uint32_t*>(S.tie);
    if (!short_list) {
      for (int i = tid; i < kHistBins; i += kSelectThreads) h2[i] = 0;
      lds_barrier();
      auto count2 = [&](uint32_t key) {
        if ((int)(key >> (32 - kHistBits)) == dstar) atomicAdd(&h2[(key >> (32 - 2 * kHistBits)) & (kHistBins - 1)], 1u);
      };
      if (in_regs) {
#pragma unroll
        for (int u = 0; u < kRegList; ++u)
          if (tid + u * kSelectThreads < ncand0) count2(rkey[u]);
      } else {
        for (int i = tid; i < ncand0; i += kSelectThreads) count2(ckey_r[i]);
      }
      lds_barrier();
      find_digit(h2, kHistBins, need - S.res[1], S.res2);
      eq22 = h2[S.res2[0]];
    }
    // Every entry a chunk left out has a key below the chunk's floor.  A chunk
    // whose floor lies above the k-th candidate key's 22-bit prefix pfloor may
    // have left out entries at or above the k-th key: rescore it (same
    // arithmetic as the scan) and add its entries in [pfloor, floor); the k-th
    // key can only rise, so afterwards every entry at or above it is a
    // candidate (rare: it takes more of the Top-k in one chunk than it keeps).
    // With block-level pruning, tau holds the query's threshold T, and at
    // least k entries score T or more: the k-th key is at least T's, so
    // chunks that left out only entries below T (every fully pruned chunk)
    // need no rescoring.
    uint32_t pfloor = short_list ? 0u : ((uint32_t)dstar << (32 - kHistBits)) | (S.res2[0] << (32 - 2 * kHistBits));
    if (ws.prune != nullptr) pfloor = max(pfloor, score_key(ws.tau[q]) & ~((1u << (32 - 2 * kHistBits)) - 1u));
    // the chunks to rescore, listed in the selection buffer (free until the
    // candidates are partitioned)
    for (int cc = tid; cc < nch; cc += kSelectThreads)
      if (((cc == tid ? fl_mine : fl[cc]) & ~kFloorBlockMax) > pfloor) {
        const int i = atomicAdd(&S.repair, 1);
        if (i < kSelCap) S.sel[i] = cc;
      }
    lds_barrier();
    const int nflag = S.repair;
    digits22 = !short_list && nflag == 0;
    if (nflag) {
      // Only blocks of flagged chunks whose largest key reaches pfloor can
      // hold what the chunks left out (a chunk without stored block maxima
      // offers all its blocks).  They are listed as (chunk, block)
      // pairs in the parking buffer (free until the candidates are
      // partitioned), kPairCap at a time, and their 16-entry tiles rescored
      // by all waves, kRepairBatch per wave at a time with all their row
      // loads in flight before the first score (lane (g, r) loads entry r's
      // operand bytes directly).  A wave scores a batch, then reserves the
      // place of all its additions at once.
      const int g = lane >> 4, r = lane & 15;
      const int wave_s = __builtin_amdgcn_readfirstlane(wave);
      intx8 a = {0, 0, 0, 0, 0, 0, 0, 0};
      float wv[4];
      if (r < sa.h_idx) a = load_fp8_operand(sa.q_idx + ((int64_t)q * sa.h_idx + r) * kIndexDim, g);
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[i] = (4 * g + i < sa.h_idx) ? sa.w[(int64_t)q * sa.h_idx + 4 * g + i] : 0.0f;
      const int32_t* pt_row = sa.c.page_table + (int64_t)sa.q_seq[q] * sa.c.max_pages;
      int32_t* cand_w = ws.cand + (int64_t)q * ws.vstride;
      uint32_t* ckey_w = ws.ckey + (int64_t)q * ws.vstride;
      const uint32_t* bm = ws.bmax + (int64_t)q * ws.fstride * kBlocksPerChunk;
      uint32_t* const pairs = reinterpret_cast<uint32_t*>(S.tie);
      // chunk slots: the flagged list, or every chunk were it to overflow.
      // (Fewer than ceil(k / L) chunks are ever flagged, L >= 16 the scan's
      // local rank: ceil(k / L) flagged chunks would hold k candidates above
      // the k-th key.  So at most 127 for k <= 2,048, one pass of pairs.)
      const bool listed = nflag <= kSelCap;
      const int nslots = listed ? nflag : nch;
      for (int s0 = 0; s0 < nslots; s0 += kPairCap / kBlocksPerChunk) {
        const int s1 = min(nslots, s0 + kPairCap / kBlocksPerChunk);
        if (tid == 0) S.npairs = 0;
        lds_barrier();
        for (int x = tid; x < (s1 - s0) * kBlocksPerChunk; x += kSelectThreads) {
          const int slot = s0 + x / kBlocksPerChunk, bl = x % kBlocksPerChunk;
          const int cc = listed ? S.sel[slot] : slot;
          const uint32_t f = fl[cc];
          // every block of a chunk that stored no block maxima
          if ((f & ~kFloorBlockMax) > pfloor && bl * kPruneBlockRows < V - cc * kScanChunk &&
              (!(f & kFloorBlockMax) || bm[(int64_t)cc * kBlocksPerChunk + bl] >= pfloor)) {
            const int i = atomicAdd(&S.npairs, 1);
            pairs[i] = (uint32_t)(cc * kBlocksPerChunk + bl);
          }
        }
        lds_barrier();
        const int ntl = S.npairs * kTilesPerBlock;
        for (int f0 = wave_s; f0 < ntl; f0 += kRepairBatch * kRepairWaves) {   // uniform
          intx8 b[kRepairBatch];
          int tstart[kRepairBatch];
#pragma unroll
          for (int u = 0; u < kRepairBatch; ++u) {
            const int f = min(f0 + u * kRepairWaves, ntl - 1);
            const uint32_t pr = pairs[f / kTilesPerBlock];
            tstart[u] = (int)pr * kPruneBlockRows + 16 * (f % kTilesPerBlock);
            const int c1 = min(V, (int)(pr / kBlocksPerChunk) * kScanChunk + kScanChunk);
            const int t = min(tstart[u] + r, c1 - 1);
            b[u] = load_fp8_operand(sa.c.idx_k + entry_row_clamped(pt_row, t, sa.c) * kIndexDim, g);
          }
          // entries below the chunk's floor that reach the k-th candidate's bin
          uint32_t key[kRepairBatch];
          uint64_t mk[kRepairBatch];
          int tot = 0;
#pragma unroll
          for (int u = 0; u < kRepairBatch; ++u) {
            key[u] = score_key(operand_score(a, wv, b[u]));
            const int cc = tstart[u] / kScanChunk;
            const int t = tstart[u] + r;
            const bool add = g == 0 && f0 + u * kRepairWaves < ntl && t < min(V, cc * kScanChunk + kScanChunk) &&
                             key[u] >= pfloor && key[u] < (fl[cc] & ~kFloorBlockMax);
            mk[u] = __builtin_amdgcn_ballot_w64(add);
            tot += __builtin_popcountll(mk[u]);
          }
          if (tot) {                                  // uniform
            int b0 = 0;
            // this workgroup alone appends to the query's list now: an LDS count
            if (lane == 0) b0 = atomicAdd(&S.ncand, tot);
            b0 = __builtin_amdgcn_readlane(b0, 0);
#pragma unroll
            for (int u = 0; u < kRepairBatch; ++u) {
              if ((mk[u] >> lane) & 1u) {
                const int pos = b0 + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk[u] >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)mk[u], 0));
                cand_w[pos] = tstart[u] + r;
                ckey_w[pos] = key[u];
                atomicAdd(&S.h[key[u] >> (32 - kHistBits)], 1u);
              }
              b0 += __builtin_popcountll(mk[u]);
            }
          }
        }
        lds_barrier();                                // the pair list is rebuilt by the next pass
      }
    }
    if (nflag || short_list) {
      __syncthreads();                                // new candidates (global) and histogram counts complete
      find_digit(S.h, kHistBins, need, S.res);
      dstar = (int)S.res[0];
    }
  }
  // the count as the repair left it
  const int ncand = S.ncand;
  uint64_t P = (uint64_t)dstar;
  need -= S.res[1];
  uint32_t cnt_eq = S.h[dstar];
  if (digits22) {
    P = (P << kHistBits) | (uint64_t)S.res2[0];
    need -= S.res2[1];
    cnt_eq = eq22;
    nbits = 2 * kHistBits;
  }
  lds_barrier();

  // heavily tied inputs: refine the prefix over the candidate list until its class fits in LDS
  while (cnt_eq > (uint32_t)kTieCap && nbits < 64) {
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
  if (in_regs && ncand == nc) {                      // the list in registers, nothing appended
#pragma unroll
    for (int u = 0; u < kRegList; ++u) {
      const bool valid = tid + u * kSelectThreads < nc;
      const uint64_t C = ((uint64_t)rkey[u] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)rcand[u]);
      const uint64_t pre = C >> (64 - nbits);
      wave_append<int32_t>(valid && pre > P, rcand[u], &S.selcnt, S.sel, kSelCap);
      wave_append<uint64_t>(valid && pre == P, C, &S.tiecnt, S.tie, kTieCap);
    }
  } else
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
  if (ws.floor != nullptr)
    launch(topk_final_kernel<true>, dim3(nq), dim3(kSelectThreads), s, ev, ws, sa, q_vis, k, out_idx, out_cnt);
  else
    launch(topk_final_kernel<false>, dim3(nq), dim3(kSelectThreads), s, ev, ws, sa, q_vis, k, out_idx, out_cnt);
  return hipGetLastError();
}

}  // namespace csa2
