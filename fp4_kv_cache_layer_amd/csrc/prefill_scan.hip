// Dense indexer for a prefill chunk: s[i, t] = sum_h w[i, h] * max(0, q[i, h] . k_t)
// for many query rows of ONE sequence at once, as an FP8 matrix product with a
// causal mask (query i sees entries t < q_vis[i]).
//
// Prefill is the computationally expensive phase ("DeepSeek-V4.1-Flash"
// research-podcast summary, abstract); the indexer scoring it runs is the one
// of the Full and Reindex modes ("Unlocking Extreme Context Scaling with
// DeepSeek-V4.1-Flash", section "Compressed Sparse Attention 2 (CSA2)").
//
// Shape: A = the queries' indexer heads ([nq * h_idx] x 128 E4M3), B = the
// sequence's indexer-K rows (128 x V E4M3); every output element needs a
// ReLU and a weight before the per-query sum over heads, so the epilogue is
// about as long as the matrix product itself and the two must overlap.
//
// Workgroup = 8 waves; it owns 8 A tiles of 16 rows (QPT queries x 16/QPT
// heads each, held in registers by every wave) and one chunk of entries,
// which its waves stream as 16-entry B tiles straight from memory into MFMA
// operands (V_MFMA_F32_16X16X128_F8F6F4: lane l supplies row / entry l % 16,
// bytes [32*(l/16), +32)).  Each B tile feeds 8 MFMAs.  Workgroups that
// share a chunk run on the same XCD, so the chunk's indexer-K stays in that
// XCD's L2 while every query block streams it.
//
// Output: the same workspace as the per-query scan (fp32 scores per query
// row and a 2,048-bin histogram of the score key's top 11 bits), so the
// Top-K select is shared.  With QPT = 2 every score is the same fma chain and
// cross-row add as in the per-query scan, so both produce identical bits.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kPfWaves = 8;
constexpr int kPfTiles = 8;             // A tiles per workgroup
constexpr int kPfMaxChunk = 16384;      // entries per workgroup at most
constexpr int kPfUnroll = 2;            // B tiles in flight per wave

// Entries per chunk and chunks per XCD for a given visible range; chunks never
// span more than 64 pages (one page id per lane).
static void prefill_chunking(int max_vis, int lg_page, int* chunk, int* per_xcd) {
  const int cap = min(kPfMaxChunk, 63 << lg_page);
  int m = 1;
  while ((max_vis + 8 * m - 1) / (8 * m) > cap) ++m;
  const int c = ((max_vis + 8 * m - 1) / (8 * m) + 15) / 16 * 16;
  *chunk = max(c, 16);
  *per_xcd = m;
}

template <int QPT>
__global__ void __launch_bounds__(kPfWaves * 64)
prefill_scan_kernel(CacheArgs c, const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_vis,
                    int nq, int h_idx, int chunk, int per_xcd, IndexWs ws) {
  constexpr int kQ = kPfTiles * QPT;                 // queries per workgroup
  __shared__ uint32_t hist[kQ * kHistBins];
  const int b = blockIdx.x;
  const int chunk_id = (b & 7) + 8 * ((b >> 3) % per_xcd);
  const int q0 = ((b >> 3) / per_xcd) * kQ;
  const int e0 = chunk_id * chunk;

  // visible range of the block's queries (uniform loads)
  int vmax = 0;
#pragma unroll
  for (int j = 0; j < kQ; ++j) vmax = max(vmax, (q0 + j < nq) ? q_vis[q0 + j] : 0);
  if (e0 >= vmax) return;                            // uniform for the block
  const int e1 = min(e0 + chunk, vmax);

  const int tid = threadIdx.x;
  {
    uint4* h4 = reinterpret_cast<uint4*>(hist);
    for (int i = tid; i < kQ * kHistBins / 4; i += kPfWaves * 64) h4[i] = make_uint4(0, 0, 0, 0);
  }
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;

  // A tiles and head weights: tile t row m is query q0 + QPT*t + m/(16/QPT),
  // head m % (16/QPT); lane (r, g) holds row r's bytes [32g, +32) and the
  // weights of output rows 4g .. 4g+3.
  constexpr int kHeadsPerTile = 16 / QPT;
  intx8 a[kPfTiles];
  float wv[kPfTiles][4];
#pragma unroll
  for (int t = 0; t < kPfTiles; ++t) {
    const int qa = q0 + QPT * t + r / kHeadsPerTile, ha = r % kHeadsPerTile;
    a[t] = intx8{0, 0, 0, 0, 0, 0, 0, 0};
    if (qa < nq && ha < h_idx) {
      const intx4* src = reinterpret_cast<const intx4*>(q_idx + ((int64_t)qa * h_idx + ha) * kIndexDim + 32 * g);
      const intx4 lo = src[0], hi = src[1];
      a[t] = intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      const int qw = q0 + QPT * t + m / kHeadsPerTile, hw = m % kHeadsPerTile;
      wv[t][i] = (qw < nq && hw < h_idx) ? w[(int64_t)qw * h_idx + hw] : 0.0f;
    }
  }

  // After the head sums, output set p puts query ql(p, g) in lane row g:
  //   QPT = 2: tiles 2p and 2p+1 -> ql = 4p + 2*(g & 1) + (g >> 1)
  //   QPT = 1: tiles 4p .. 4p+3   -> ql = 4p + g
  constexpr int kSets = kPfTiles * QPT / 4;
  int vis_of[kSets];
  float* srow[kSets];
#pragma unroll
  for (int p = 0; p < kSets; ++p) {
    const int ql = (QPT == 2) ? 4 * p + 2 * (g & 1) + (g >> 1) : 4 * p + g;
    const int qg = q0 + ql;
    vis_of[p] = qg < nq ? q_vis[qg] : 0;
    srow[p] = ws.scores + (int64_t)min(qg, nq - 1) * ws.vstride;
  }

  // page ids of the chunk, one per lane
  const int32_t* pt_row = c.page_table + (int64_t)q_seq[q0] * c.max_pages;
  const int pg0 = e0 >> c.lg_page;
  const int npg = ((e1 - 1) >> c.lg_page) - pg0 + 1;
  const int page_of_lane = lane < npg ? pt_row[pg0 + lane] : 0;
  const int ntiles = (e1 - e0 + 15) >> 4;
  lds_barrier();

  auto load = [&](int j, intx8& bt) {
    j = min(j, ntiles - 1);
    const int ts = e0 + 16 * j;
    const int page = __builtin_amdgcn_readlane(page_of_lane, (ts >> c.lg_page) - pg0);
    const int64_t row = ((int64_t)page << c.lg_page) + (ts & ((1 << c.lg_page) - 1)) + r;
    const intx4* src = reinterpret_cast<const intx4*>(c.idx_k + row * kIndexDim + 32 * g);
    const intx4 lo = src[0], hi = src[1];
    bt = intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  intx8 cur[kPfUnroll], nxt[kPfUnroll];
#pragma unroll
  for (int u = 0; u < kPfUnroll; ++u) load(wave + kPfWaves * u, cur[u]);
  constexpr int kStride = kPfWaves * kPfUnroll;
  for (int base = wave; base < ntiles; base += kStride) {
#pragma unroll
    for (int u = 0; u < kPfUnroll; ++u) load(base + kStride + kPfWaves * u, nxt[u]);
#pragma unroll
    for (int u = 0; u < kPfUnroll; ++u) {
      const int j = base + kPfWaves * u;
      if (j >= ntiles) break;
      const int te = e0 + 16 * j;
      float part[kPfTiles];
#pragma unroll
      for (int t = 0; t < kPfTiles; ++t) {
        floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[t], cur[u], acc, 0, 0, 0, 0, 0, 0);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) s += wv[t][i] * fmaxf(acc[i], 0.0f);
        s = rows_pair_sum(s);
        if (QPT == 1) s = halves_sum(s);
        part[t] = s;
      }
      const int e = te + r;
#pragma unroll
      for (int p = 0; p < kSets; ++p) {
        float s;
        if (QPT == 2) {
          s = (g & 1) ? part[2 * p + 1] : part[2 * p];
        } else {
          s = g == 0 ? part[4 * p] : g == 1 ? part[4 * p + 1] : g == 2 ? part[4 * p + 2] : part[4 * p + 3];
        }
        const int ql = (QPT == 2) ? 4 * p + 2 * (g & 1) + (g >> 1) : 4 * p + g;
        if (e < vis_of[p]) {                         // causal mask; 0 for padding queries
          uint32_t u32 = __float_as_uint(s);
          if ((u32 << 1) == 0) u32 = 0;              // -0 -> +0
          srow[p][e] = __uint_as_float(u32);
          atomicAdd(&hist[ql * kHistBins + (score_key(__uint_as_float(u32)) >> (32 - kHistBits))], 1u);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kPfUnroll; ++u) cur[u] = nxt[u];
  }
  lds_barrier();
  for (int i = tid; i < kQ * kHistBins; i += kPfWaves * 64) {
    const int ql = i / kHistBins;
    const uint32_t v = hist[i];
    if (v && q0 + ql < nq) atomicAdd(&ws.hist[(int64_t)(q0 + ql) * kHistBins + (i - ql * kHistBins)], v);
  }
}

hipError_t launch_prefill_scan(const CacheArgs& c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                               const int32_t* q_vis, int nq, int h_idx, int max_vis, const IndexWs& ws,
                               hipStream_t s, const KEvents& ev) {
  if (nq <= 0 || max_vis <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  int chunk, per_xcd;
  prefill_chunking(max_vis, c.lg_page, &chunk, &per_xcd);
  const int qpt = h_idx <= 8 ? 2 : 1;
  const int64_t nqb = (nq + kPfTiles * qpt - 1) / (kPfTiles * qpt);
  const dim3 grid((unsigned)(8 * per_xcd * nqb));
  if (qpt == 2)
    launch(prefill_scan_kernel<2>, grid, dim3(kPfWaves * 64), s, ev, c, q_idx, w, q_seq, q_vis, nq, h_idx, chunk,
           per_xcd, ws);
  else
    launch(prefill_scan_kernel<1>, grid, dim3(kPfWaves * 64), s, ev, c, q_idx, w, q_seq, q_vis, nq, h_idx, chunk,
           per_xcd, ws);
  return hipGetLastError();
}

}  // namespace csa2
