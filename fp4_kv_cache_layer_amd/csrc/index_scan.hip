// Indexer scan: s_t = sum_h w_h * max(0, q_h . k_t) over every visible entry
// of a query's sequence, with the scores written to the workspace and a
// histogram of their top 11 key bits accumulated for the Top-K select.
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
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kScanWaves = 4;
constexpr int kScanDepth = 6;           // tiles per wave in the load ring

// Row stride of the per-query score and candidate arrays: at least two slots
// past the longest visible range, which the indexer kernels use as write
// sinks that are never read.
int64_t index_vstride(int32_t max_vis) { return ((int64_t)max_vis + 2 + 63) / 64 * 64; }

size_t zero_state_bytes(int32_t nq) {
  return ((size_t)nq * (kHistBins + 1) * 4 + 255) / 256 * 256;
}

size_t index_score_bytes(int32_t nq, int32_t max_vis) {
  const size_t v = (size_t)index_vstride(max_vis);
  const size_t nq16 = ((size_t)nq + 15) / 16 * 16;      // candidate masks cover whole 16-query blocks
  return (size_t)nq * 12 * v + nq16 * v / 8;           // scores, candidates, candidate keys, masks
}

__global__ void __launch_bounds__(kScanWaves * 64)
index_scan_kernel(CacheArgs c, const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                  const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_vis,
                  int nq, int h_idx, IndexWs ws) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ __attribute__((aligned(16))) uint8_t stage[kScanWaves][kFp8SlotBytes];
  // chunk-major: the short last chunks of equal-length queries come last, so
  // a grid larger than one round leaves only short work for the second round
  const int chunk = blockIdx.x / nq;
  const int q = blockIdx.x - chunk * nq;
  const int vis = clamp_vis(q_vis[q], ws);
  const int t0 = chunk * kScanChunk;
  if (t0 >= vis) return;                              // uniform for the block
  const int t1 = min(vis, t0 + kScanChunk);
  const int tid = threadIdx.x;
  for (int i = tid; i < kHistBins; i += kScanWaves * 64) hist[i] = 0;

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  intx8 a = {0, 0, 0, 0, 0, 0, 0, 0};
  if (r < h_idx) {
    a = load_fp8_operand(q_idx + ((int64_t)q * h_idx + r) * kIndexDim, g);
  }
  float wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wv[i] = (4 * g + i < h_idx) ? w[(int64_t)q * h_idx + 4 * g + i] : 0.0f;

  // Page ids of this chunk (at most kScanChunk / CSA2_MIN_PAGE_SIZE = 32),
  // one per lane; a tile's page is then a lane read with a uniform index, so
  // no load waits on a page-table load.
  const int32_t* pt_row = c.page_table + (int64_t)q_seq[q] * c.max_pages;
  const int pg0 = t0 >> c.lg_page;
  const int npg = ((t1 - 1) >> c.lg_page) - pg0 + 1;
  const int page_of_lane = lane < npg ? clamp_page(pt_row[pg0 + lane], c) : 0;
  float* srow = ws.scores + (int64_t)q * ws.vstride;
  const int ntiles = (t1 - t0 + 15) >> 4;
  lds_barrier();

  // Tiles j = wave, wave + 4, ... of this wave, kScanDepth - 1 in flight ahead
  // of the one in use (a ring of buffers addressed by name after unrolling).  A tile's 16 rows are 2 KB of
  // contiguous memory: loaded coalesced, turned into the MFMA operand through
  // the wave's LDS slot.  Loads past the end re-read the last tile; stores are
  // unconditional (lanes with nothing to write use the sink slot past every
  // visible entry), so the compiler can count loads in flight past them.
  uint8_t* const slot = stage[wave];
  auto load = [&](int j, intx8& lin) {
    j = min(j, ntiles - 1);
    const int ts = t0 + 16 * j;                       // tiles never straddle pages
    const int page = __builtin_amdgcn_readlane(page_of_lane, (ts >> c.lg_page) - pg0);
    lin = load_fp8_tile_linear(c.idx_k + (((int64_t)page << c.lg_page) + (ts & ((1 << c.lg_page) - 1))) * kIndexDim,
                               lane);
  };
  const int sink = (int)ws.vstride - 1;
  auto process = [&](int j, const intx8& lin) {
    const intx8 b = fp8_tile_operand(slot, lin, lane);
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
    const float part = halves_sum(rows_pair_sum(relu_weighted(acc, wv)));   // every lane: entry r's score
    const int t = t0 + 16 * j + r;
    uint32_t u32 = __float_as_uint(part);
    if ((u32 << 1) == 0) u32 = 0;                     // -0 -> +0
    srow[t < t1 ? t : sink] = __uint_as_float(u32);
    if (g == 0 && t < t1) atomicAdd(&hist[score_key(__uint_as_float(u32)) >> (32 - kHistBits)], 1u);
  };
  intx8 buf[kScanDepth];
#pragma unroll
  for (int d = 0; d + 1 < kScanDepth; ++d) load(wave + d * kScanWaves, buf[d]);
  if (ntiles == kScanChunk / 16) {
    // full chunk: a fixed schedule, unrolled, so every wait on the ring is exact
    constexpr int kSteps = kScanChunk / 16 / kScanWaves;
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      if (u + kScanDepth - 1 < kSteps)
        load(wave + (u + kScanDepth - 1) * kScanWaves, buf[(u + kScanDepth - 1) % kScanDepth]);
      process(wave + u * kScanWaves, buf[u % kScanDepth]);
    }
  } else {
    for (int j = wave; j < ntiles; j += kScanDepth * kScanWaves) {
#pragma unroll
      for (int u = 0; u < kScanDepth; ++u) {
        load(j + (u + kScanDepth - 1) * kScanWaves, buf[(u + kScanDepth - 1) % kScanDepth]);
        if (j + u * kScanWaves >= ntiles) break;
        process(j + u * kScanWaves, buf[u]);
      }
    }
  }
  lds_barrier();
  uint32_t* gh = ws.hist + (int64_t)q * kHistBins;
  for (int i = tid; i < kHistBins; i += kScanWaves * 64) {
    const uint32_t v = hist[i];
    if (v) atomicAdd(&gh[i], v);
  }
}

hipError_t launch_index_scan(const CacheArgs& c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                             const int32_t* q_vis, int nq, int h_idx, int max_vis, const IndexWs& ws,
                             hipStream_t s, const KEvents& ev) {
  const int nchunks = (max_vis + kScanChunk - 1) / kScanChunk;
  const int64_t blocks = (int64_t)nq * nchunks;
  if (blocks <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  launch(index_scan_kernel, dim3((unsigned)blocks), dim3(kScanWaves * 64), s, ev, c, q_idx, w, q_seq, q_vis, nq,
         h_idx, ws);
  return hipGetLastError();
}

}  // namespace csa2
