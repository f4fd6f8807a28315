// Indexer scan: s_t = sum_h w_h * max(0, q_h . k_t) over every visible entry
// of a query's sequence, and the first half of the exact Top-k: each
// 2,048-entry chunk keeps its own top entries as candidates.
//
// The scan over the cached indexer-K is the step the Full and Reindex modes
// spend their indexing compute on ("Unlocking Extreme Context Scaling with
// DeepSeek-V4.1-Flash", section "Compressed Sparse Attention 2 (CSA2)"); the
// pages give no formula, the one above is the reading stated in csa2.h.
//
// Dot products run on the gfx950 FP8 matrix core: one
// V_MFMA_F32_16X16X128_F8F6F4 multiplies the (zero-padded to 16) indexer
// heads by a tile of 16 entries over the full 128-wide dimension.  Each
// 2 KB tile is read with fully coalesced loads and reaches the operand
// layout through the wave's LDS slot.  The result puts entry (l % 16) and
// heads 4*(l/16)+i in lane l, so the ReLU * w reduction is 4 FMAs and two
// lane-swap adds.
//
// Scores stay in LDS (no score is written to memory).  When the chunk is
// done, a two-level radix search over its 2,048-bin histogram of score-key
// prefixes finds the key of its L-th largest entry to 22 bits (L from
// scan_local_rank), and every entry whose key reaches that floor is appended
// to the query's candidate list (index and key, one reservation per
// workgroup); the floor is stored per chunk.  (Counting the candidates into a
// per-query histogram here, one global atomic per candidate, cost more than
// the whole scan: the candidates of all chunks fall into the same few top
// bins.  The final select counts them from the list instead.)  The final select takes the k-th key among the
// candidates; every chunk whose floor lies at or below that key's bin kept
// all entries that can belong to the Top-k, and any other chunk is rescored
// there (rare: it needs more than L of the Top-k in one chunk).
#include "csa2_device.h"
#include "csa2_internal.h"
#include "csa2_select.h"

namespace csa2 {

// Eight waves per 2,048-entry chunk: two workgroups per CU, so a 1,024-chunk
// launch runs in two rounds and the hardware hands the second round's chunks
// to whichever CUs finish first (64K decode group: 52.5 -> 48.5 us against
// four waves and one round; 16 waves: 59 us).
constexpr int kScanWaves = 8;
// Ring of 4 tiles per wave: three loads ahead of the one in use, so a launch
// keeps about 24 MB of loads in flight, enough to cover HBM latency; deeper
// rings only lengthen the memory queues, and every other load of the launch
// (a new workgroup's page ids, its query, the reservation atomics) waits
// behind them (64K decode group: 48.9 -> 47.3 us against 6 tiles; 3 tiles
// 49.4 us).
constexpr int kScanDepth = 4;

// DPP controls: rotate right within each row of 16 lanes
constexpr int kDppRowRor1 = 0x121, kDppRowRor2 = 0x122, kDppRowRor4 = 0x124, kDppRowRor8 = 0x128;

// The largest of the wave's 64 values, in every lane: rotations within each
// row of 16 lanes, then the rows' maxima across the two halves and pairs.
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowRor8, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowRor4, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowRor2, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowRor1, 0xF, 0xF, false));
  const auto h = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  x = max(h[0], h[1]);
  const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return max(p[0], p[1]);
}

// Row stride of the per-query score and candidate arrays: at least two slots
// past the longest visible range, which the indexer kernels use as write
// sinks that are never read.
int64_t index_vstride(int32_t max_vis) { return ((int64_t)max_vis + 2 + 63) / 64 * 64; }

size_t zero_state_bytes(int32_t nq) {
  return ((size_t)nq * 3 * 4 + 255) / 256 * 256;      // candidate counters, thresholds, rescore counters
}

size_t index_score_bytes(int32_t nq, int32_t max_vis) {
  const size_t v = (size_t)index_vstride(max_vis);
  const size_t fstride = ((size_t)max_vis + kScanChunk - 1) / kScanChunk;
  // candidates, candidate keys, chunk floors, prune masks, block maximum keys
  return (size_t)nq * 8 * v + (size_t)nq * fstride * 8 + (size_t)nq * fstride * 32 * 4;
}

// kAppend: the launch also appends ap.n <= kMaxFusedAppend rows: its first
// ceil(n / 4) workgroups write them (one wave per row), and a chunk that
// holds an appended row takes that row's E4M3 codes from its bf16 source
// instead of the cache, so no tile depends on those stores.
template <bool kAppend>
__global__ void __launch_bounds__(kScanWaves * 64)
index_scan_kernel(CacheArgs c, const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                  const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_vis,
                  int nq, int h_idx, int k, IndexWs ws, AppendArgs ap) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ float sc[kScanChunk + 1];                // the chunk's scores (+ a sink slot)
  __shared__ __attribute__((aligned(16))) uint8_t stage[kScanWaves][kFp8SlotBytes];   // then the candidate list
  __shared__ uint32_t res[2];
  __shared__ int nlist, base;                          // listed candidates, their place in the query's list
  __shared__ int concentrated;                         // candidates crowd into one block
  constexpr int kPatch = kAppend ? kMaxFusedAppend : 1;
  __shared__ int npatch_s;                             // appended rows inside this chunk
  __shared__ int patch_pos[kPatch], patch_src[kPatch];   // their position in the chunk, their source row
  __shared__ uint32_t patch_code[kPatch][kIndexDim / 4];  // their E4M3 codes
  int bid = blockIdx.x;
  if constexpr (kAppend) {
    const int na = (ap.n + 3) >> 2;
    if (bid < na) {                                    // an appending workgroup
      const int row = bid * 4 + (threadIdx.x >> 6);
      if (row < ap.n) append_row(ap.kv, ap.idx_k, ap.slots, ap.kv_rows, ap.idxk_rows, row, threadIdx.x & 63);
      return;
    }
    bid -= na;
  }
  // query-major: the chunks of one query are consecutive blocks.  On ragged
  // batches the grid is sized by the longest query and most blocks of the
  // short ones exit at once; in this order the working blocks of every query
  // are dispatched together (chunk-major order left the long queries' chunks
  // to a thin tail: 0.43 -> 0.62 of HBM on the ragged decode workload)
  const int nch = ws.fstride;                          // chunks per query
  const int q = bid / nch;
  const int chunk = bid - q * nch;
  const int seq = q_seq[q], vis_in = q_vis[q];
  asm volatile("" ::"s"(seq), "s"(vis_in));           // one trip for both (q_seq would wait for the exit test)
  const int vis = clamp_vis(vis_in, ws);
  const int t0 = chunk * kScanChunk;
  if (t0 >= vis || vis <= k) return;                  // uniform; with V <= k the select takes everything
  const int t1 = min(vis, t0 + kScanChunk);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Page ids of this chunk (at most kScanChunk / CSA2_MIN_PAGE_SIZE = 32),
  // one per lane; a tile's page is then a lane read with a uniform index, so
  // no load waits on a page-table load.  Loaded before the query's operand
  // and weights, so the first tile loads wait for this load alone (0.7 to
  // 1.2 us less per launch on the 64K decode workload).
  const int32_t* pt_row = c.page_table + (int64_t)seq * c.max_pages;
  const int pg0 = t0 >> c.lg_page;
  const int npg = ((t1 - 1) >> c.lg_page) - pg0 + 1;
  const int pt_entry = pt_row[pg0 + min(lane, npg - 1)];   // (unconditional: nothing waits for it here)
  // the appended rows' slots (lane i: row i), in the same trip
  const int ap_slot = kAppend ? ap.slots[min(lane, max(ap.n, 1) - 1)] : 0;
  // block-level pruning: blocks of this chunk that cannot hold a Top-k entry
  const uint32_t pmask = ws.prune ? ws.prune[(int64_t)q * ws.fstride + chunk] : 0u;
  const int nblk = (t1 - t0 + kPruneBlockRows - 1) / kPruneBlockRows;
  const uint32_t inrange = nblk >= 32 ? 0xFFFFFFFFu : ((1u << nblk) - 1u);
  if (pmask != 0 && (pmask & inrange) == inrange) {
    // nothing here reaches the threshold: no candidates; the floor is the
    // threshold's 22-bit prefix, so the final select never rescores the chunk
    // unless its k-th key falls below the threshold
    if (tid == 0)
      ws.floor[(int64_t)q * ws.fstride + chunk] = score_key(ws.tau[q]) & ~((1u << (32 - 2 * kHistBits)) - 1u);
    return;
  }
  auto pruned_tile = [&](int j) { return ((pmask >> (j >> 2)) & 1u) != 0u; };   // 4 tiles per block
  for (int i = tid; i < kHistBins; i += kScanWaves * 64) hist[i] = 0;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  // (loaded without branches, from clamped rows, and zeroed past the heads
  // afterwards: the first tile loads then wait for the page-table load alone)
  intx8 a = load_fp8_operand(q_idx + ((int64_t)q * h_idx + min(r, h_idx - 1)) * kIndexDim, g);
  if (r >= h_idx) a = intx8{0, 0, 0, 0, 0, 0, 0, 0};
  float wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wv[i] = w[(int64_t)q * h_idx + min(4 * g + i, h_idx - 1)];
    if (4 * g + i >= h_idx) wv[i] = 0.0f;
  }

  const int page_of_lane = lane < npg ? clamp_page(pt_entry, c) : 0;
  const int ntiles = (t1 - t0 + 15) >> 4;

  // Tiles j = wave, wave + kScanWaves, ... of this wave, kScanDepth - 1 in flight ahead
  // of the one in use (a ring of buffers addressed by name after unrolling).  A tile's 16 rows are 2 KB of
  // contiguous memory: loaded coalesced, turned into the MFMA operand through
  // the wave's LDS slot.  Loads past the end re-read the last tile.  The
  // ring's first loads go out before the appended rows are located (their
  // bytes are replaced when a tile is scored), so they wait for the page ids
  // alone.
  auto load = [&](int j, intx8& lin) {
    j = min(j, ntiles - 1);
    const int ts = t0 + 16 * j;                       // tiles never straddle pages
    const int page = __builtin_amdgcn_readlane(page_of_lane, (ts >> c.lg_page) - pg0);
    lin = load_fp8_tile_linear(c.idx_k + (((int64_t)page << c.lg_page) + (ts & ((1 << c.lg_page) - 1))) * kIndexDim,
                               lane);
  };
  intx8 buf[kScanDepth];
#pragma unroll
  for (int d = 0; d + 1 < kScanDepth; ++d) load(wave + d * kScanWaves, buf[d]);
  if constexpr (kAppend) {
    // the appended rows inside this chunk: lane i checks row i's slot
    // against the chunk's pages
    if (wave == 0) {
      int pos = -1;
      if (lane < ap.n) {
        const int sl = ap_slot;
        const int pg = sl >> c.lg_page;
        for (int p = 0; p < npg; ++p)
          if (__builtin_amdgcn_readlane(page_of_lane, p) == pg) {
            const int t = ((pg0 + p) << c.lg_page) + (sl & ((1 << c.lg_page) - 1));
            if (t >= t0 && t < t1) pos = t - t0;
          }
      }
      const uint64_t m = __builtin_amdgcn_ballot_w64(pos >= 0);
      if (pos >= 0) {
        const int at = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        patch_pos[at] = pos;
        patch_src[at] = lane;
      }
      if (lane == 0) npatch_s = __builtin_popcountll(m);
    }
  }
  lds_barrier();
  const int npatch = kAppend ? npatch_s : 0;          // uniform
  if constexpr (kAppend) {
    if (npatch > 0) {
      // their codes, encoded as the appending workgroups encode them
      for (int x = tid; x < npatch * (kIndexDim / 4); x += kScanWaves * 64) {
        const int p = x / (kIndexDim / 4), d = x % (kIndexDim / 4);
        const uint2 bf = *reinterpret_cast<const uint2*>(ap.idxk_rows + (int64_t)patch_src[p] * kIndexDim + 4 * d);
        patch_code[p][d] = e4m3_code(__uint_as_float(bf.x << 16)) | (e4m3_code(__uint_as_float(bf.x & 0xFFFF0000u)) << 8) |
                           (e4m3_code(__uint_as_float(bf.y << 16)) << 16) |
                           (e4m3_code(__uint_as_float(bf.y & 0xFFFF0000u)) << 24);
      }
      lds_barrier();
    }
  }
  // a loaded tile j with its appended rows' bytes replaced (lane l holds
  // bytes [32 (l % 4), +32) of the tile's row l / 4)
  auto patch = [&](int j, intx8& lin) {
    for (int p = 0; p < npatch; ++p) {                // uniform
      const int pos = patch_pos[p];
      if ((pos >> 4) == j && (lane >> 2) == (pos & 15)) {
        const uint32_t* src = &patch_code[p][8 * (lane & 3)];
        lin = intx8{(int)src[0], (int)src[1], (int)src[2], (int)src[3], (int)src[4], (int)src[5], (int)src[6],
                    (int)src[7]};
      }
    }
  };

  uint8_t* const slot = stage[wave];
  auto process = [&](int j, const intx8& lin) {
    const float sv = tile_score(a, wv, slot, lin, lane);   // every lane: entry r's score
    const int i = 16 * j + r;                         // position in the chunk
    if (g == 0) {
      sc[t0 + i < t1 ? i : kScanChunk] = sv;
      if (t0 + i < t1) atomicAdd(&hist[score_key(sv) >> (32 - kHistBits)], 1u);
    }
  };
  if (ntiles == kScanChunk / 16 && pmask == 0 && npatch == 0) {
    // full chunk: a fixed schedule, unrolled, so every wait on the ring is exact
    constexpr int kSteps = kScanChunk / 16 / kScanWaves;
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      if (u + kScanDepth - 1 < kSteps)
        load(wave + (u + kScanDepth - 1) * kScanWaves, buf[(u + kScanDepth - 1) % kScanDepth]);
      process(wave + u * kScanWaves, buf[u % kScanDepth]);
    }
  } else {
    // (tiles of pruned blocks are neither loaded nor scored)
    for (int j = wave; j < ntiles; j += kScanDepth * kScanWaves) {
#pragma unroll
      for (int u = 0; u < kScanDepth; ++u) {
        const int jl = j + (u + kScanDepth - 1) * kScanWaves;
        if (!pruned_tile(min(jl, ntiles - 1))) load(jl, buf[(u + kScanDepth - 1) % kScanDepth]);
        if (j + u * kScanWaves >= ntiles) break;
        if (!pruned_tile(j + u * kScanWaves)) {
          if (kAppend && npatch > 0) patch(j + u * kScanWaves, buf[u]);
          process(j + u * kScanWaves, buf[u]);
        }
      }
    }
  }
  lds_barrier();

  // the chunk's local threshold: key floor of its L-th largest entry, to 22 bits
  const int nloc = t1 - t0;
  // entries of unpruned blocks
  int nreal = nloc;
  if (pmask != 0)
    for (int bl = 0; bl < nblk; ++bl)
      if ((pmask >> bl) & 1u) nreal -= min(kPruneBlockRows, nloc - bl * kPruneBlockRows);
  auto live = [&](int i) { return ((pmask >> (i / kPruneBlockRows)) & 1u) == 0u; };
  const int L = scan_local_rank(k, vis);
  uint32_t floor_key = 0;                             // a chunk of at most L entries keeps them all
  int n = nreal;                                      // entries at or above the floor
  if (nreal > L) {
    find_digit(hist, kHistBins, (uint32_t)L, res);    // ends with a barrier
    const uint32_t d1 = res[0], above1 = res[1];
    for (int i = tid; i < kHistBins; i += kScanWaves * 64) hist[i] = 0;
    lds_barrier();
    for (int i = tid; i < nloc; i += kScanWaves * 64) {
      const uint32_t key = score_key(sc[i]);
      if (live(i) && (key >> (32 - kHistBits)) == d1)
        atomicAdd(&hist[(key >> (32 - 2 * kHistBits)) & (kHistBins - 1)], 1u);
    }
    lds_barrier();
    find_digit(hist, kHistBins, (uint32_t)L - above1, res);
    floor_key = (d1 << (32 - kHistBits)) | (res[0] << (32 - 2 * kHistBits));
    n = (int)(above1 + res[1] + hist[res[0]]);
  }
  // The count is known from the histograms: reserve the candidates' place in
  // the query's list now, so the atomic's round trip overlaps the listing.
  int my_base = 0;                                    // (thread 0) waited on only after the listing
  if (tid == 0) my_base = (int)atomicAdd(&ws.cand_cnt[q], (uint32_t)n);
  // candidates: every entry whose key reaches the floor, listed in LDS (one
  // scan and one reservation per wave)
  int32_t* const list = reinterpret_cast<int32_t*>(&stage[0][0]);
  if (tid == 0) { nlist = 0; concentrated = 0; }
  lds_barrier();
  constexpr int kPer = kScanChunk / (kScanWaves * 64);
  static_assert(kPer * kScanWaves == kScanChunk / kPruneBlockRows, "a wave's 64 entries of a round are one block");
  // A chunk whose candidates crowd into one block (more than a quarter of L
  // there) is one the final select may have to rescore; for it the largest
  // key of every block is stored too, so that only blocks that can hold
  // missing entries are rescored.
  const int crowd = max(16, L / 4);
  uint32_t mine = 0;
  bool crowded = false;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = u * kScanWaves * 64 + tid;         // block 4u + wave, entry lane
    const bool c = i < nloc && live(i) && score_key(sc[i]) >= floor_key;
    mine += c ? 1u : 0u;
    crowded |= __builtin_popcountll(__builtin_amdgcn_ballot_w64(c)) > crowd;   // (uniform)
  }
  if (crowded && floor_key != 0 && lane == 0) concentrated = 1;   // (a chunk that kept everything is never rescored)
  const uint32_t x = wave_incl_sum(mine);
  int wbase = 0;
  if (lane == 63 && x) wbase = atomicAdd(&nlist, (int)x);
  int pos = __shfl(wbase, 63) + (int)(x - mine);
  if (mine) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = u * kScanWaves * 64 + tid;
      if (i < nloc && live(i) && score_key(sc[i]) >= floor_key) list[pos++] = i;
    }
  }
  if (tid == 0) base = my_base;
  lds_barrier();                                     // the list, the reservation and the crowding flag
  const bool with_bmax = concentrated != 0;          // uniform
  if (tid == 0) ws.floor[(int64_t)q * ws.fstride + chunk] = floor_key | (with_bmax ? kFloorBlockMax : 0u);
  if (with_bmax) {
    uint32_t blk_max = 0;                            // lane u: the largest key of block 4u + wave
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = u * kScanWaves * 64 + tid;
      // (0 past the end and in a pruned block, none of whose entries can
      // reach the Top-k)
      const uint32_t m = wave_max((i < nloc && live(i)) ? score_key(sc[i]) : 0u);
      if (lane == u) blk_max = m;
    }
    if (lane < kPer)
      ws.bmax[((int64_t)q * ws.fstride + chunk) * (kScanChunk / kPruneBlockRows) + lane * kScanWaves + wave] = blk_max;
  }
  int32_t* cand = ws.cand + (int64_t)q * ws.vstride + base;
  uint32_t* ckey = ws.ckey + (int64_t)q * ws.vstride + base;
  for (int j = tid; j < n; j += kScanWaves * 64) {
    const int i = list[j];
    cand[j] = t0 + i;
    ckey[j] = score_key(sc[i]);
  }
}

hipError_t launch_index_scan(const CacheArgs& c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                             const int32_t* q_vis, int nq, int h_idx, int k, int max_vis, const IndexWs& ws,
                             hipStream_t s, const KEvents& ev, const AppendArgs* ap) {
  const int nchunks = (max_vis + kScanChunk - 1) / kScanChunk;
  const int64_t blocks = (int64_t)nq * nchunks;
  if (ap != nullptr && ap->n > 0) {
    // the rows are written whatever the scan covers
    launch(index_scan_kernel<true>, dim3((unsigned)(blocks + (ap->n + 3) / 4)), dim3(kScanWaves * 64), s, ev, c,
           q_idx, w, q_seq, q_vis, nq, h_idx, k, ws, *ap);
    return hipGetLastError();
  }
  if (blocks <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  launch(index_scan_kernel<false>, dim3((unsigned)blocks), dim3(kScanWaves * 64), s, ev, c, q_idx, w, q_seq, q_vis,
         nq, h_idx, k, ws, AppendArgs{});
  return hipGetLastError();
}

}  // namespace csa2
