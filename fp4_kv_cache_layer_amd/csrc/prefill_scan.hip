// Dense indexer for a prefill chunk: s[i, t] = sum_h w[i, h] * max(0, q[i, h] . k_t)
// for many query rows of ONE sequence at once, as an FP8 matrix product with a
// causal mask (query i sees entries t < q_vis[i]), followed by an exact
// Top-K over the candidates it keeps.
//
// Prefill is the computationally expensive phase ("DeepSeek-V4.1-Flash"
// research-podcast summary, abstract); the indexer scoring it runs is the one
// of the Full and Reindex modes ("Unlocking Extreme Context Scaling with
// DeepSeek-V4.1-Flash", section "Compressed Sparse Attention 2 (CSA2)").
//
// Writing every score (4 B per query and entry) would cost more HBM time than
// the matrix product, so only candidates are kept:
//
//  1. threshold (prefill_tau_kernel): each query scores a stratified sample
//     of 512 visible entries and takes the r-th largest sample score as its
//     threshold, r chosen so that about factor * k entries are expected to
//     pass.  Queries with V <= k need no threshold; short contexts keep all.
//  2. candidates (prefill_scan_kernel, first pass): the product itself; an
//     entry whose score reaches the threshold joins its query's candidate
//     list (index and score key).  Each wave gathers its candidates per query
//     in LDS and flushes a query's batch with one reservation on the query's
//     counter, so the lists are written contiguously and nothing else (no
//     score rows, no masks) leaves the kernel.  Every entry at or above the
//     k-th key is then a candidate whenever at least k entries reached the
//     threshold, so the final select sees the same k-th key and the same
//     entries above it as over all entries.
//  3. exactness (the scan kernel again): a query left with fewer than k
//     candidates (the sample was unlucky) is rescored in full, and its
//     entries below the threshold are appended after the first pass's, so
//     its list then holds every visible entry once; workgroups without such
//     a query exit at once.
//
// Matrix product: A = the queries' indexer heads ([nq * h_idx] x 128 E4M3),
// B = the sequence's indexer-K rows (128 x V E4M3).  A workgroup of 4 waves
// owns 8 A tiles of 16 query-head rows (16 queries in all; load_set_tile
// gives the row order), held in registers by every wave, and one chunk of
// entries, which its waves stream as 16-entry B tiles (loaded coalesced, put
// into the V_MFMA_F32_16X16X128_F8F6F4 operand layout of load_fp8_operand
// through a per-wave LDS slot); each B tile feeds 8 MFMAs.  Workgroups
// sharing a chunk run on the same XCD, so the chunk's indexer-K stays in
// that XCD's L2.  Every score is the same two four-head fma chains and the
// same add of the two as in the per-query scan, so both produce identical
// bits.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {

constexpr int kPfWaves = 4;
constexpr int kPfTiles = 8;             // A tiles per workgroup
constexpr int kPfMaxChunk = 16384;      // entries per workgroup at most
constexpr int kTauWaves = 4;
constexpr int kSampleTiles = 32;        // 512 sampled entries per query
constexpr int kMaxRank = 64;

constexpr int kPfCap = 1024;            // LDS candidate slots per wave
constexpr int kPfMaxQ = 2 * kPfTiles;   // queries per workgroup at most

// LDS of the candidate pass: per wave its staged B tile, the candidates not
// yet flushed to the lists (word 0: entry offset in the chunk in bits 0-13,
// query of the workgroup in bits 14-17, its rank among the flush's
// candidates of that query in bits 18-27; word 1: the score's bits) and
// per-query counters of a flush.
struct PfShared {
  uint8_t tile[kPfWaves][kFp8SlotBytes];
  float4 w[kPfTiles][4];             // head weights of A tile t's output rows 4g .. 4g+3 (row group g)
  uint2 pend[kPfWaves][kPfCap + 64];   // + one sink slot per lane
  uint32_t qcnt[kPfWaves][kPfMaxQ];
};
static_assert(kPfMaxChunk <= (1 << 14) && kPfMaxQ <= 16 && kPfCap <= (1 << 10), "candidate word fields");

// Entries per chunk and chunks per XCD for a given visible range; chunks never
// span more than 64 pages (one page id per lane).
void prefill_chunking(int max_vis, int lg_page, int* chunk, int* per_xcd) {
  const int cap = min(kPfMaxChunk, 63 << lg_page);
  int m = 1;
  while ((max_vis + 8 * m - 1) / (8 * m) > cap) ++m;
  const int c = ((max_vis + 8 * m - 1) / (8 * m) + 15) / 16 * 16;
  *chunk = max(c, 16);
  *per_xcd = m;
}

// A tile t and the weights of output rows 4g .. 4g+3 for queries q0 + QPT*t ...
template <int QPT>
__device__ __forceinline__ void load_a_tile(const uint8_t* q_idx, const float* w, int nq, int h_idx, int qt,
                                            int r, int g, intx8& a, float (&wv)[4]) {
  constexpr int kHeadsPerTile = 16 / QPT;
  const int qa = qt + r / kHeadsPerTile, ha = r % kHeadsPerTile;
  a = intx8{0, 0, 0, 0, 0, 0, 0, 0};
  if (qa < nq && ha < h_idx) a = load_fp8_operand(q_idx + ((int64_t)qa * h_idx + ha) * kIndexDim, g);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * g + i;
    const int qw = qt + m / kHeadsPerTile, hw = m % kHeadsPerTile;
    wv[i] = (qw < nq && hw < h_idx) ? w[(int64_t)qw * h_idx + hw] : 0.0f;
  }
}

// A tile t of the candidate pass and the weights of its output rows 4g .. 4g+3.
// QPT = 2 (at most 8 heads): output set p = t / 2 covers the four queries
// qs .. qs+3 (qs = q0 + 4p); tile 2p carries heads 0..3 and tile 2p+1 heads
// 4..7 of each (A row m: query qs + m / 4, head 4 * (t & 1) + m % 4), so
// output rows 4g .. 4g+3 of the two tiles are all heads of query qs + g and
// a lane's score is the sum of its two four-head partials, with no lane
// exchange.  QPT = 1: tile t is query q0 + t, rows = heads.
template <int QPT>
__device__ __forceinline__ void load_set_tile(const uint8_t* q_idx, const float* w, int nq, int h_idx, int q0, int t,
                                              int r, int g, intx8& a, float (&wv)[4]) {
  if constexpr (QPT == 2) {
    const int qs = q0 + 4 * (t >> 1), hb = 4 * (t & 1);
    const int qa = qs + (r >> 2), ha = hb + (r & 3);
    a = intx8{0, 0, 0, 0, 0, 0, 0, 0};
    if (qa < nq && ha < h_idx) a = load_fp8_operand(q_idx + ((int64_t)qa * h_idx + ha) * kIndexDim, g);
    const int qw = qs + g;
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[i] = (qw < nq && hb + i < h_idx) ? w[(int64_t)qw * h_idx + hb + i] : 0.0f;
  } else {
    load_a_tile<1>(q_idx, w, nq, h_idx, q0 + t, r, g, a, wv);
  }
}

__device__ __forceinline__ float row16_max(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int row16_sum(int x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. threshold per query from a stratified sample
// ---------------------------------------------------------------------------
template <int QPT>
__global__ void __launch_bounds__(kTauWaves * 64)
prefill_tau_kernel(CacheArgs c, const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                   const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_vis, int nq, int h_idx, int k,
                   int factor, IndexWs ws) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int qt = (blockIdx.x * kTauWaves + wave) * QPT;       // first query of this wave's A tile
  if (qt >= nq) return;                                       // wave-uniform; no barriers below

  // the output row of this lane holds query qrow (QPT = 2: rows 0,1 -> qt, rows 2,3 -> qt+1)
  const int qrow = qt + (QPT == 2 ? (g >> 1) : 0);
  const bool valid = qrow < nq;
  const int V = valid ? clamp_vis(q_vis[qrow], ws) : 0;
  int vmin = clamp_vis(q_vis[qt], ws);
  if (QPT == 2 && qt + 1 < nq) vmin = min(vmin, clamp_vis(q_vis[qt + 1], ws));
  const int ntv = vmin >> 4;                                  // 16-entry tiles visible to the whole tile

  // rank r in the sample; 0 = no sampled threshold for this row
  float tau;
  int rank = 0;
  if (!valid || V <= k || factor == 0) {
    tau = INFINITY;                                           // nothing to keep (V <= k selects everything)
  } else {
    const int64_t rr = ((int64_t)factor * k * (16 * kSampleTiles) + V - 1) / V;
    if (rr > kMaxRank || ntv < kSampleTiles) tau = -INFINITY; // keep every visible entry
    else { tau = -INFINITY; rank = (int)rr; }
  }
  if (__builtin_amdgcn_ballot_w64(rank > 0)) {
    intx8 a;
    float wv[4];
    load_a_tile<QPT>(q_idx, w, nq, h_idx, qt, r, g, a, wv);
    const int32_t* pt_row = c.page_table + (int64_t)q_seq[qt] * c.max_pages;
    float vals[kSampleTiles];
#pragma unroll
    for (int j = 0; j < kSampleTiles; ++j) {
      const int ts = (j * ntv / kSampleTiles) * 16;
      const int page = clamp_page(pt_row[ts >> c.lg_page], c);
      const int64_t row = ((int64_t)page << c.lg_page) + (ts & ((1 << c.lg_page) - 1)) + r;
      const intx8 b = load_fp8_operand(c.idx_k + row * kIndexDim, g);
      floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
      float s = rows_pair_sum(relu_weighted(acc, wv));
      if (QPT == 1) s = halves_sum(s);
      vals[j] = s;
    }
    // r-th largest of the row's 16 x 32 values: take out the current maximum
    // (all copies) until r values have been taken out
    int left = rank;
    for (int it = 0; it < kMaxRank && __builtin_amdgcn_ballot_w64(left > 0); ++it) {
      float m = vals[0];
#pragma unroll
      for (int j = 1; j < kSampleTiles; ++j) m = fmaxf(m, vals[j]);
      m = row16_max(m);
      int ceq = 0;
#pragma unroll
      for (int j = 0; j < kSampleTiles; ++j) ceq += vals[j] == m ? 1 : 0;
      ceq = row16_sum(ceq);
      if (left > 0) {
        if (ceq >= left) { tau = m; left = 0; }
        else left -= ceq;
      }
#pragma unroll
      for (int j = 0; j < kSampleTiles; ++j) vals[j] = vals[j] == m ? -INFINITY : vals[j];
    }
  }
  const bool writer = r == 0 && (QPT == 1 ? g == 0 : (g & 1) == 0);
  if (writer && valid) ws.tau[qrow] = tau;
}

// ---------------------------------------------------------------------------
// 2./3. candidate pass (RESCORE = false) and full rescore of short queries
// ---------------------------------------------------------------------------
// Three workgroups per CU; the one-query-per-tile form (more than 8 indexer
// heads) holds four partial sums per set and runs two, so it needs no spills.
template <int QPT, bool RESCORE>
__global__ void __launch_bounds__(kPfWaves * 64, QPT == 2 ? 3 : 2)
prefill_scan_kernel(CacheArgs c, const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_vis,
                    int nq, int h_idx, int k, int chunk, int per_xcd, IndexWs ws) {
  constexpr int kQ = kPfTiles * QPT;                 // queries per workgroup
  static_assert(kQ <= kPfMaxQ && kQ <= 64, "one lane per query in the flushes");
  __shared__ PfShared S;
  const int b = blockIdx.x;
  const int chunk_id = (b & 7) + 8 * ((b >> 3) % per_xcd);
  const int q0 = ((b >> 3) / per_xcd) * kQ;
  const int e0 = chunk_id * chunk;

  // visible range of the block's queries; the rescore pass only serves
  // queries left with fewer than k candidates (uniform loads; the rescore
  // never changes the first pass's counters, so every block reads the same)
  int vmax = 0;
  bool any_fail = false;
#pragma unroll
  for (int j = 0; j < kQ; ++j) {
    const int v = (q0 + j < nq) ? clamp_vis(q_vis[q0 + j], ws) : 0;
    vmax = max(vmax, v);
    if (RESCORE && v > k && (int)ws.cand_cnt[q0 + j] < k) any_fail = true;
  }
  if (RESCORE && !any_fail) return;                  // uniform for the block
  if (e0 >= vmax) return;
  const int e1 = min(e0 + chunk, vmax);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: tile indices stay scalar
  const int g = lane >> 4, r = lane & 15;
  // A tiles in registers; their head weights, the same for all 16 lanes of a
  // row group, staged through LDS once and then held in registers (three
  // waves per SIMD leave room for them, so no epilogue waits on LDS)
  intx8 a[kPfTiles];
#pragma unroll
  for (int t = 0; t < kPfTiles; ++t) {
    float wv[4];
    load_set_tile<QPT>(q_idx, w, nq, h_idx, q0, t, r, g, a[t], wv);
    if (wave == 0 && r == 0) S.w[t][g] = make_float4(wv[0], wv[1], wv[2], wv[3]);
  }
  lds_barrier();

  // After the head sums, output set p puts query ql = 4p + g in lane row g
  // (QPT = 2: tiles 2p and 2p+1; QPT = 1: tiles 4p .. 4p+3).
  constexpr int kSets = kPfTiles * QPT / 4;
  int vis_of[kSets];
  float tau_of[kSets];
  int npend = 0;                                     // this wave's unflushed candidates (uniform)
  if (lane < kPfMaxQ) S.qcnt[wave][lane] = 0;
#pragma unroll
  for (int p = 0; p < kSets; ++p) {
    const int qg = q0 + 4 * p + g;
    const bool valid = qg < nq;
    const int v = valid ? clamp_vis(q_vis[qg], ws) : 0;
    const bool own = RESCORE ? (valid && v > k && (int)ws.cand_cnt[qg] < k) : valid;
    vis_of[p] = own ? v : 0;
    tau_of[p] = valid ? ws.tau[qg] : INFINITY;
  }
  // the rescore appends after the first pass's candidates (lane ql: query q0 + ql)
  const int list_base = (RESCORE && lane < kQ && q0 + lane < nq) ? (int)ws.cand_cnt[q0 + lane] : 0;

  // page ids of the chunk, one per lane
  const int32_t* pt_row = c.page_table + (int64_t)q_seq[q0] * c.max_pages;
  const int pg0 = e0 >> c.lg_page;
  const int npg = ((e1 - 1) >> c.lg_page) - pg0 + 1;
  const int page_of_lane = lane < npg ? clamp_page(pt_row[pg0 + lane], c) : 0;
  const int ntiles = (e1 - e0 + 15) >> 4;

  // Every query block streams the same chunk; starting each block at its own
  // offset keeps the XCD's workgroups from requesting the same tile at the
  // same moment, so all but the first reader of a tile hit in L2.
  const int rot = (int)(((int64_t)((b >> 3) / per_xcd) * 37) % ntiles);
  auto tile_at = [&](int j) {                        // j-th tile of this block's rotated order
    j = min(j, ntiles - 1) + rot;
    return j >= ntiles ? j - ntiles : j;
  };
  // A tile's 16 rows are 2 KB of contiguous memory, loaded coalesced and
  // turned into the MFMA operand through the wave's LDS slot.
  // The scheduling barrier after each tile's loads keeps them in program
  // order, so the wait before a tile's use counts exactly the loads issued
  // after it and the two tiles ahead stay in flight.
  auto load = [&](int j, intx8& lin) {
    const int ts = e0 + 16 * tile_at(j);
    const int page = __builtin_amdgcn_readlane(page_of_lane, (ts >> c.lg_page) - pg0);
    lin = load_fp8_tile_linear(
        c.idx_k + (((int64_t)page << c.lg_page) + (ts & ((1 << c.lg_page) - 1))) * kIndexDim, lane);
    __builtin_amdgcn_sched_barrier(0);
  };
  uint8_t* const slot = S.tile[wave];
  auto to_operand = [&](const intx8& lin) { return fp8_tile_operand(slot, lin, lane); };

  // Scores of one tile for output set p (see ql above): the set's matrix
  // products are issued one set ahead of their epilogue, so the epilogue never
  // waits on a product that was just issued.
  constexpr int kPerSet = 4 / QPT;                   // MFMAs per output set
  auto products = [&](const intx8& bop, int p, floatx4 (&acc)[kPerSet]) {
#pragma unroll
    for (int i = 0; i < kPerSet; ++i) {
      acc[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[kPerSet * p + i], bop, acc[i], 0, 0, 0, 0, 0, 0);
    }
  };
  float4 wreg[kPfTiles];
#pragma unroll
  for (int t = 0; t < kPfTiles; ++t) wreg[t] = S.w[t][g];
  auto finish = [&](int p, const floatx4 (&acc)[kPerSet]) {
    if (QPT == 2) {
      // heads 0..3 + heads 4..7: the per-query scan adds the same two
      // partials (across a lane pair), so the bits agree
      return relu_weighted4(acc[0], wreg[2 * p]) + relu_weighted4(acc[1], wreg[2 * p + 1]);
    } else {
      float sq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sq[i] = halves_sum(rows_pair_sum(relu_weighted4(acc[i], wreg[4 * p + i])));
      return g == 0 ? sq[0] : g == 1 ? sq[1] : g == 2 ? sq[2] : sq[3];
    }
  };

  // Flush: the wave's pending candidates go to their queries' lists.  Each
  // takes its rank among the flush's candidates of its query (LDS counters);
  // lane ql then reserves query ql's place with one atomic (all queries in one
  // round trip), and every candidate is stored at its query's base + rank.
  auto flush = [&]() {
    uint2* const pl = S.pend[wave];
    uint32_t* const qc = S.qcnt[wave];
    for (int i = lane; i < npend; i += 64) {
      const uint32_t w0 = pl[i].x;
      const uint32_t rank = atomicAdd(&qc[(w0 >> 14) & 15u], 1u);
      pl[i].x = w0 | (rank << 18);
    }
    __builtin_amdgcn_wave_barrier();
    // the bases go through LDS (a lane permute would read 0 from lanes the
    // copy loop's last, partial round leaves inactive)
    if (lane < kQ) {
      const uint32_t n = qc[lane];
      uint32_t* const ctr = RESCORE ? ws.cnt2 : ws.cand_cnt;
      qc[lane] = n ? (uint32_t)list_base + atomicAdd(&ctr[q0 + lane], n) : 0u;
    }
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < npend; i += 64) {
      const uint2 v = pl[i];
      const int ql = (int)((v.x >> 14) & 15u), rank = (int)(v.x >> 18);
      const int64_t at = (int64_t)(q0 + ql) * ws.vstride + (int)qc[ql] + rank;
      ws.cand[at] = e0 + (int)(v.x & 0x3FFFu);
      ws.ckey[at] = score_key(__uint_as_float(v.y));
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < kQ) qc[lane] = 0;
    npend = 0;
    // the list stores complete here (vmcnt 0, other counters untouched), so
    // after a flush no store is in flight: the compiler's count of the loads
    // in flight stays exact across the loop's back edge and its waits keep
    // the two tiles ahead in flight
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_wave_barrier();                 // the copies' LDS reads stay above later appends
  };

  // candidate word of this lane's entry in output set 0, less the tile offset
  // (set p adds p << 16: its query is 4p + g)
  const uint32_t word0 = (uint32_t)r | ((uint32_t)g << 14);
  auto process = [&](int j, const intx8& lin) {
    const int te = e0 + 16 * tile_at(j);
    const int e = te + r;
    const intx8 bop = to_operand(lin);
    floatx4 cur[kPerSet], nxt[kPerSet];
    products(bop, 0, cur);
#pragma unroll
    for (int p = 0; p < kSets; ++p) {
      if (p + 1 < kSets) products(bop, p + 1, nxt);
      const float sc = finish(p, cur);
      // the rescore takes exactly the entries the first pass did not
      const bool reach = sc >= tau_of[p];
      const bool keep = e < vis_of[p] && (RESCORE ? !reach : reach);
      // every lane stores (no branch): a kept entry at its place in the
      // wave's list, the others into their lane's sink slot past the list
      const uint64_t m = __builtin_amdgcn_ballot_w64(keep);
      const int pos = keep ? npend + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0))
                           : kPfCap + lane;
      S.pend[wave][pos] = make_uint2(word0 + ((uint32_t)(te - e0) + ((uint32_t)p << 16)), __float_as_uint(sc));
      npend += __builtin_popcountll(m);
#pragma unroll
      for (int i = 0; i < kPerSet; ++i) cur[i] = nxt[i];
    }
    if (npend > kPfCap - 64 * kSets) flush();        // a tile adds at most 64 per set
  };
  // B tiles j = wave, wave + 4, ...; two tiles in flight ahead of the one in
  // use, in three buffers that rotate by name (unrolled by three)
  intx8 l0, l1, l2;
  load(wave, l0);
  load(wave + kPfWaves, l1);
  for (int j = wave; j < ntiles; j += 3 * kPfWaves) {
    load(j + 2 * kPfWaves, l2);
    process(j, l0);
    if (j + kPfWaves >= ntiles) break;
    load(j + 3 * kPfWaves, l0);
    process(j + kPfWaves, l1);
    if (j + 2 * kPfWaves >= ntiles) break;
    load(j + 4 * kPfWaves, l1);
    process(j + 2 * kPfWaves, l2);
  }
  if (npend > 0) flush();
}

hipError_t launch_prefill_scan(const CacheArgs& c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                               const int32_t* q_vis, int nq, int h_idx, int k, int max_vis, const IndexWs& ws,
                               int cand_factor, hipStream_t s, const KEvents& ev, const KEvents& ev_product) {
  if (nq <= 0 || max_vis <= 0) {
    record_empty(ev, s);
    record_empty(ev_product, s);
    return hipSuccess;
  }
  int chunk, per_xcd;
  prefill_chunking(max_vis, c.lg_page, &chunk, &per_xcd);
  const int qpt = h_idx <= 8 ? 2 : 1;
  const int64_t nqb = (nq + kPfTiles * qpt - 1) / (kPfTiles * qpt);
  const dim3 grid((unsigned)(8 * per_xcd * nqb)), block(kPfWaves * 64);
  const dim3 tgrid((unsigned)((nq + kTauWaves * qpt - 1) / (kTauWaves * qpt))), tblock(kTauWaves * 64);
  const int factor = cand_factor;
  // threshold, candidates (which count each query's candidates), full
  // rescore of the queries left short
  if (qpt == 2) {
    launch(prefill_tau_kernel<2>, tgrid, tblock, s, ev.first(), c, q_idx, w, q_seq, q_vis, nq, h_idx, k, factor, ws);
    launch(prefill_scan_kernel<2, false>, grid, block, s, ev_product, c, q_idx, w, q_seq, q_vis, nq, h_idx, k, chunk,
           per_xcd, ws);
    launch(prefill_scan_kernel<2, true>, grid, block, s, ev.last(), c, q_idx, w, q_seq, q_vis, nq, h_idx, k, chunk,
           per_xcd, ws);
  } else {
    launch(prefill_tau_kernel<1>, tgrid, tblock, s, ev.first(), c, q_idx, w, q_seq, q_vis, nq, h_idx, k, factor, ws);
    launch(prefill_scan_kernel<1, false>, grid, block, s, ev_product, c, q_idx, w, q_seq, q_vis, nq, h_idx, k, chunk,
           per_xcd, ws);
    launch(prefill_scan_kernel<1, true>, grid, block, s, ev.last(), c, q_idx, w, q_seq, q_vis, nq, h_idx, k, chunk,
           per_xcd, ws);
  }
  return hipGetLastError();
}

}  // namespace csa2
