// Block-level pruning for the indexer: the other half of the hierarchical
// indexer.  The indexer it is informed by scores token-level entries and
// prunes them by block-level representations ("DeepSeek-V4.1-Flash: Pushing
// the Limits of KV Cache Compression", Related Work); the pages give no block
// summary or rule, and the reading here keeps the Top-K exact:
//
//   - a block is 64 consecutive cache rows (pages are whole blocks), its
//     representation the per-dimension maximum and minimum E4M3 code of its
//     indexer-K rows (256 bytes; idxk_bounds_kernel builds or refreshes it);
//   - every score of the block lies below
//       UB = sum_h w_h * max(0, w_h >= 0 ? hi_h : lo_h),
//       hi_h = q_h+ . M + q_h- . m,  lo_h = q_h+ . m + q_h- . M
//     (q+ / q- the positive / negative parts of the query, M / m the block's
//     maxima / minima), since q_h . k lies in [lo_h, hi_h] for every k in the
//     block's box and max(0, .) never decreases;
//   - a query's threshold T is the k-th largest score of k distinct visible
//     entries it names (its seed, such as its previous Top-K), scored with
//     the scan's arithmetic: at least k entries reach T, so T never exceeds
//     the query's k-th largest score, and a block whose bound lies below T
//     holds no entry of the Top-K; prune_mask_kernel marks such blocks and
//     the scan never reads them.
//
// The products are the FP8 matrix-core products of the scan (q+, q- and the
// bounds are E4M3 codes, so every product is exact); the bound is widened by
// 2^-14 of the magnitudes it sums, more than the fp32 rounding of the scan's
// score and of the bound itself can reach, so a pruned block never holds a
// score at or above T.
#include "csa2.h"
#include "csa2_device.h"
#include "csa2_internal.h"
#include "csa2_select.h"

namespace csa2 {

namespace {

constexpr int kPruneThreads = 1024;
constexpr int kPruneWaves = kPruneThreads / 64;
constexpr float kBoundSlack = 1.0f / 16384.0f;     // 2^-14 of the summed magnitudes
constexpr int kSeedBatch = 4;                      // seed tiles per wave with their loads in flight together
constexpr int kMaxSplit = 16;                      // workgroups per query of the mask kernel

// Order key of an E4M3 code by value: negative codes below positive ones,
// larger magnitudes further from the middle (+-0 differ only in the key).
__device__ __forceinline__ uint32_t e4m3_order(uint32_t c) {
  return (c & 0x80u) ? 0x7Fu - (c & 0x7Fu) : 0x80u + c;
}

// Per byte of four packed E4M3 codes: the code of the larger magnitude of a
// and b (sign bits cleared).  SWAR: with 7-bit lanes, bit 7 of
// (a | 0x80) - b is set exactly where a >= b, and no lane borrows.
__device__ __forceinline__ uint32_t max_magnitude4(uint32_t a, uint32_t b) {
  a &= 0x7F7F7F7Fu;
  b &= 0x7F7F7F7Fu;
  const uint32_t ge = (((a | 0x80808080u) - b) & 0x80808080u) >> 7;
  const uint32_t m = (ge << 8) - ge;                 // 0xFF where a >= b
  return (a & m) | (b & ~m);
}

// Sign masks of four packed E4M3 codes: 0xFF where the code is negative.
__device__ __forceinline__ uint32_t negative4(uint32_t x) {
  const uint32_t s = (x & 0x80808080u) >> 7;
  return (s << 8) - s;
}

}  // namespace

// One workgroup of 128 threads per block: the block's 64 rows go through LDS,
// thread d keeps dimension d's largest and smallest code.  blocks: explicit
// block ids (slots / 64) or, when null, first_block + blockIdx.x.
__global__ void __launch_bounds__(128)
idxk_bounds_kernel(const uint8_t* __restrict__ idx_k, uint8_t* __restrict__ bounds, const int32_t* __restrict__ slots,
                   int first_block, int64_t n_rows) {
  __shared__ __attribute__((aligned(16))) uint8_t rows[kPruneBlockRows * kIndexDim];
  const int64_t blk = slots ? (int64_t)slots[blockIdx.x] / kPruneBlockRows : (int64_t)first_block + blockIdx.x;
  const int64_t r0 = blk * kPruneBlockRows;
  if (r0 < 0 || r0 + kPruneBlockRows > n_rows) return;   // uniform; a slot outside the cache names no block
  const int tid = threadIdx.x;
  const uint4* src = reinterpret_cast<const uint4*>(idx_k + r0 * kIndexDim);
  uint4* dst = reinterpret_cast<uint4*>(rows);
#pragma unroll
  for (int i = 0; i < kPruneBlockRows * kIndexDim / 16 / 128; ++i) dst[tid + 128 * i] = src[tid + 128 * i];
  __syncthreads();
  uint32_t hi = rows[tid], lo = hi;
  uint32_t khi = e4m3_order(hi), klo = khi;
  for (int r = 1; r < kPruneBlockRows; ++r) {
    const uint32_t c = rows[r * kIndexDim + tid];
    const uint32_t kc = e4m3_order(c);
    if (kc > khi) { khi = kc; hi = c; }
    if (kc < klo) { klo = kc; lo = c; }
  }
  bounds[blk * kPruneBoundBytes + tid] = (uint8_t)hi;
  bounds[blk * kPruneBoundBytes + kIndexDim + tid] = (uint8_t)lo;
}

// The pruned-block masks, spread over nsplit workgroups per query (the
// seed's threshold is recomputed by each, so no workgroup waits on another):
// 16-wave workgroup (q, split) takes chunks split * 16 + wave, then every
// 16 * nsplit further.  Each computes T from the seed, writes the mask word
// of each of its chunks (bit i of word c: block 32c + i) to ws.prune; split
// 0 writes T
// to ws.tau (the scan's floor of a fully pruned chunk, the final select's
// lower bound of the k-th key).  Fewer than k distinct visible seed entries:
// no threshold (-inf), nothing pruned.
__global__ void __launch_bounds__(kPruneThreads)
prune_mask_kernel(CacheArgs c, const uint8_t* __restrict__ bounds, const uint8_t* __restrict__ q_idx,
                  const float* __restrict__ w, const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_vis,
                  const int32_t* __restrict__ seed, const int32_t* __restrict__ seed_cnt, int h_idx, int k,
                  int nsplit, IndexWs ws) {
  __shared__ int32_t sd[CSA2_MAX_K];
  __shared__ __attribute__((aligned(16))) uint8_t stage[kPruneWaves][kFp8SlotBytes];
  __shared__ float tmin[kPruneWaves];
  __shared__ int nvalid_s, unsorted;
  const int q = blockIdx.x / nsplit, split = blockIdx.x - q * nsplit;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int V = clamp_vis(q_vis[q], ws);
  const int nchunks = (V + kScanChunk - 1) / kScanChunk;
  if (split > 0 && split * kPruneWaves >= nchunks) return;          // uniform: no chunk here, T written by split 0
  const int ns = min(max(seed_cnt[q], 0), k);
  const int32_t* pt_row = c.page_table + (int64_t)q_seq[q] * c.max_pages;

  // the query's operands: heads as rows (h_idx <= 16)
  intx8 a = {0, 0, 0, 0, 0, 0, 0, 0};
  if (r < h_idx) a = load_fp8_operand(q_idx + ((int64_t)q * h_idx + r) * kIndexDim, g);
  float wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wv[i] = (4 * g + i < h_idx) ? w[(int64_t)q * h_idx + 4 * g + i] : 0.0f;

  // the bounds of this wave's first chunk, in flight while the seed is read
  // (lane (g, r): block r of each half, the 32-byte operand pieces of group g)
  const int nblocks = (V + kPruneBlockRows - 1) / kPruneBlockRows;
  auto bound_ptr = [&](int ch, int half) {
    const int bc = min(ch * (kScanChunk / kPruneBlockRows) + 16 * half + r, nblocks - 1);
    const int64_t pblk = entry_row_clamped(pt_row, bc * kPruneBlockRows, c) / kPruneBlockRows;
    return bounds + pblk * kPruneBoundBytes;
  };
  const int ch0 = split * kPruneWaves + wave;
  intx8 M0[2], m0[2];
  if (ch0 < nchunks) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint8_t* bp = bound_ptr(ch0, half);
      M0[half] = load_fp8_operand(bp, g);
      m0[half] = load_fp8_operand(bp + kIndexDim, g);
    }
  }

  // the seed, sorted (a Top-K row is already ascending; others are sorted
  // here) so duplicates are neighbours
  int n2 = 1;
  while (n2 < ns) n2 <<= 1;
  if (tid == 0) { unsorted = 0; nvalid_s = 0; }
  for (int i = tid; i < n2; i += kPruneThreads) sd[i] = i < ns ? seed[(int64_t)q * k + i] : 0x7FFFFFFF;
  __syncthreads();
  for (int i = tid; i + 1 < ns; i += kPruneThreads)
    if (sd[i] >= sd[i + 1]) unsorted = 1;
  __syncthreads();
  if (unsorted) {                                    // uniform
    for (int size = 2; size <= n2; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < n2 / 2; i += kPruneThreads) {
          const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
          const bool up = (lo & size) == 0;
          const int32_t x = sd[lo], y = sd[hi];
          if ((x > y) == up) { sd[lo] = y; sd[hi] = x; }
        }
        __syncthreads();
      }
  }
  // distinct visible entries (duplicates after sorting are neighbours)
  int mine = 0;
  for (int i = tid; i < ns; i += kPruneThreads) {
    const int32_t t = sd[i];
    mine += (t >= 0 && t < V && (i == 0 || sd[i - 1] != t)) ? 1 : 0;
  }
  if (mine) atomicAdd(&nvalid_s, mine);
  __syncthreads();
  const bool prune = nvalid_s >= k;                  // uniform; then all ns == k entries are distinct and visible

  // threshold: the smallest score of the seed's k entries, each scored as the
  // scan scores it (tile_score: the scan's operand path, MFMA and
  // reduction).  A wave takes 16-entry tiles wave, wave + 16, ..., kSeedBatch
  // at a time with every row load issued before the first score (lane l:
  // bytes [32 (l % 4), +32) of entry l / 4's row, as a linear 2 KB tile load
  // would hold them).
  float T = -INFINITY;
  if (prune) {
    float m = INFINITY;
    const int ntiles = (ns + 15) >> 4;
    for (int b0 = wave; b0 < ntiles; b0 += kSeedBatch * kPruneWaves) {
      intx8 lin[kSeedBatch];
#pragma unroll
      for (int u = 0; u < kSeedBatch; ++u) {
        const int i = min(16 * min(b0 + u * kPruneWaves, ntiles - 1) + (lane >> 2), ns - 1);
        const uint8_t* src = c.idx_k + entry_row_clamped(pt_row, sd[i], c) * kIndexDim + 32 * (lane & 3);
        const intx4 lo = *reinterpret_cast<const intx4*>(src);
        const intx4 hi = *reinterpret_cast<const intx4*>(src + 16);
        lin[u] = intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int u = 0; u < kSeedBatch; ++u) {
        const float sv = tile_score(a, wv, stage[wave], lin[u], lane);   // every lane: entry r's score
        if (16 * (b0 + u * kPruneWaves) + r < ns) m = (sv == sv) ? fminf(m, sv) : -INFINITY;   // NaN: no threshold
      }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = fminf(m, __shfl_xor(m, o));
    if (lane == 0) tmin[wave] = m;
    __syncthreads();
    T = tmin[0];
#pragma unroll
    for (int i = 1; i < kPruneWaves; ++i) T = fminf(T, tmin[i]);
  }
  if (split == 0 && tid == 0) ws.tau[q] = T;

  // q+, q- and |q| codes of the query
  const uint32_t neg[8] = {negative4(a[0]), negative4(a[1]), negative4(a[2]), negative4(a[3]),
                           negative4(a[4]), negative4(a[5]), negative4(a[6]), negative4(a[7])};
  intx8 qpos, qneg, qabs;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    qpos[i] = (int)((uint32_t)a[i] & ~neg[i]);
    qneg[i] = (int)((uint32_t)a[i] & neg[i]);
    qabs[i] = (int)((uint32_t)a[i] & 0x7F7F7F7Fu);
  }
  // block bounds, 16 blocks per MFMA tile, two tiles per chunk word
  for (int ch = ch0; ch < nchunks; ch += kPruneWaves * nsplit) {
    uint32_t word = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      intx8 M, mn;
      if (ch == ch0) {
        M = M0[half];
        mn = m0[half];
      } else {
        const uint8_t* bp = bound_ptr(ch, half);
        M = load_fp8_operand(bp, g);
        mn = load_fp8_operand(bp + kIndexDim, g);
      }
      intx8 X;
#pragma unroll
      for (int i = 0; i < 8; ++i) X[i] = (int)max_magnitude4((uint32_t)M[i], (uint32_t)mn[i]);
      const floatx4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      floatx4 hi = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qpos, M, z, 0, 0, 0, 0, 0, 0);
      hi = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qneg, mn, hi, 0, 0, 0, 0, 0, 0);
      floatx4 lo = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qpos, mn, z, 0, 0, 0, 0, 0, 0);
      lo = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qneg, M, lo, 0, 0, 0, 0, 0, 0);
      const floatx4 mag = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qabs, X, z, 0, 0, 0, 0, 0, 0);
      // this lane's four heads 4g .. 4g+3 of block r
      float sacc = 0.0f, sabs = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = kBoundSlack * mag[i];
        // max(0, .) that keeps a NaN (a NaN code in a never-written row of
        // the block): the bound turns NaN and the block is kept
        const float hu = hi[i] + d, ld = lo[i] - d;
        const float up = hu < 0.0f ? 0.0f : hu, dn = ld < 0.0f ? 0.0f : ld;
        sacc += wv[i] * (wv[i] >= 0.0f ? up : dn);
        sabs += fabsf(wv[i]) * up;
      }
      sacc = halves_sum(rows_pair_sum(sacc));
      sabs = halves_sum(rows_pair_sum(sabs));
      const float ub = sacc + kBoundSlack * sabs + 1e-30f;
      const int b = ch * (kScanChunk / kPruneBlockRows) + 16 * half + r;
      const bool pruned = prune && b < nblocks && ub < T;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(pruned && g == 0);
      word |= (uint32_t)(bal & 0xFFFFu) << (16 * half);
    }
    if (lane == 0) ws.prune[(int64_t)q * ws.fstride + ch] = word;
  }
}

hipError_t launch_idxk_bounds(const uint8_t* idx_k, uint8_t* bounds, const int32_t* slots, int first_block,
                              int n, int64_t n_rows, hipStream_t s, const KEvents& ev) {
  if (n <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  launch(idxk_bounds_kernel, dim3((unsigned)n), dim3(128), s, ev, idx_k, bounds, slots, first_block, n_rows);
  return hipGetLastError();
}

hipError_t launch_prune_mask(const CacheArgs& c, const uint8_t* bounds, const uint8_t* q_idx, const float* w,
                             const int32_t* q_seq, const int32_t* q_vis, const int32_t* seed, const int32_t* seed_cnt,
                             int nq, int h_idx, int k, const IndexWs& ws, hipStream_t s, const KEvents& ev) {
  if (nq <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  // workgroups per query: 16 chunks each, at most kMaxSplit (longer
  // contexts give each wave several chunks)
  const int per = (ws.fstride + kPruneWaves - 1) / kPruneWaves;
  const int nsplit = per < 1 ? 1 : per > kMaxSplit ? kMaxSplit : per;
  launch(prune_mask_kernel, dim3((unsigned)(nq * nsplit)), dim3(kPruneThreads), s, ev, c, bounds, q_idx, w, q_seq,
         q_vis, seed, seed_cnt, h_idx, k, nsplit, ws);
  return hipGetLastError();
}

}  // namespace csa2
