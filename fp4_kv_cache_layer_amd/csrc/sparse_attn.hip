// Sparse attention over the selected FP4 rows: for each query and head,
// O = softmax(sm_scale * q . X_j) . X_j over the selected rows j, with X the
// dequantised 512-wide latent (K = V = X), plus the natural-log LSE.
//
// Every CSA2 mode ends in attention over the selected global-KV entries; the
// Reuse mode reuses an earlier layer's KV and indices ("Unlocking Extreme
// Context Scaling with DeepSeek-V4.1-Flash", section "Compressed Sparse
// Attention 2 (CSA2)").  Attention cost is fixed by the Top-512 selection, not
// by the context length ("DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
// Compression", Introduction: near-constant decode FLOPs from 4K to 1M).
//
// Work split.  A workgroup serves one (query, group of 16 heads) unit, or a
// share of its selected rows (large batches of 64-head queries instead give
// each query one workgroup for all its heads: sparse_attn_hg_kernel below).
// Its waves form RG row groups of four: the four
// waves of a row group own the four 128-wide slices of the latent, and row
// group g takes tiles g, g + RG, ...; at the end row groups merge their
// (output, running max, running sum) through LDS.  Small decode batches use
// RG = 2; a share split across workgroups (small batches) writes its
// unnormalised output with its running max and sum and a combine kernel
// merges the shares.  The workgroup first resolves the physical
// row of every selected entry of its share into LDS, then streams 32-row
// tiles with the row gathers of the next kPrefetch tiles in flight.  For every
// tile a wave
//   - gathers whole 64-byte row segments of its slice (four lanes per row)
//     with their scale bytes, dequantises them with
//     V_CVT_SCALEF32_PK_BF16_FP4 into its bf16 slice rows in LDS (row stride
//     288 B: the 16-byte accesses and the transposing 8-byte reads both spread
//     evenly over the banks), and reads back the A operand of S^T = X Q^T
//     (bf16 MFMA 16x16x32, K = its 128 dims, permuted alike in the Q operand),
//   - publishes its partial S^T (32 rows x 16 heads) in LDS,
//   - sums the four partial S^T (same order in every wave), runs the online
//     softmax (the output is rescaled only when the running max grows by more
//     than 8 nats, so probabilities stay below e^8) and accumulates
//     O[16 heads][its 128 dims] += P X with P split into bf16 hi + lo terms;
//     the B operand (rows as K) comes from LDS through the transposing read
//     DS_READ_B64_TR_B16.
#include <cfloat>

#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kTileRows = 32;
constexpr int kSliceStride = 288;                       // bytes per bf16 slice row (128 * 2 + 32 pad)
constexpr int kSliceBytes = kTileRows * kSliceStride;   // 9,216
constexpr int kPrefetch = 4;                            // tiles of row gathers in flight per wave
constexpr float kRescaleSlack = 8.0f;                   // nats the running max may lag the true max
constexpr int kMaxShareRows = 2048;

typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

__device__ __forceinline__ shortx4 lds_read_tr16(const uint8_t* base_generic, int byte_off) {
  const __attribute__((address_space(3))) uint8_t* p =
      (const __attribute__((address_space(3))) uint8_t*)(base_generic) + byte_off;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)p);
}

template <int SEL>
__device__ __forceinline__ bf16x2 cvt_fp4x2(uint32_t word, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, SEL);
}

__device__ __forceinline__ bf16x8 dequant8(uint32_t wd, float scale) {
  const bf16x2 p0 = cvt_fp4x2<0>(wd, scale), p1 = cvt_fp4x2<1>(wd, scale);
  const bf16x2 p2 = cvt_fp4x2<2>(wd, scale), p3 = cvt_fp4x2<3>(wd, scale);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <int RG>
struct AttnShared {
  uint8_t xs[4 * RG][kSliceBytes];   // [wave] bf16 slice rows of its current tile (9,216 B each)
  floatx4 sp[RG == 2 ? 2 : 1][RG][4][2][4][16];   // [buffer][row group][wave]: partial S^T, [m-tile][row quad][head]
  uint32_t row[kMaxShareRows];       // physical row of every selected entry of the share (8,192 B)
};

template <int RG>
__global__ void __launch_bounds__(256 * RG, RG == 1 ? 2 : 1)
sparse_attn_kernel(CacheArgs c, const uint16_t* __restrict__ q, const int32_t* __restrict__ q_seq,
                   const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int h, int k,
                   float sm_scale, float* __restrict__ out, float* __restrict__ lse, int nsplit, int npairs,
                   float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int kThreads = 256 * RG;
  __shared__ AttnShared<RG> S;
  // Block order: the head groups of one (query, share) are 8 blocks apart,
  // so they run on the same XCD (blocks go to XCDs round-robin) and gather
  // the same rows through one L2.
  const int ngroups = (h + 15) >> 4;
  const int b = blockIdx.x;
  const int hg = (b >> 3) % ngroups;
  const int pair = (b / (8 * ngroups)) * 8 + (b & 7);    // (query, share)
  if (pair >= npairs) return;                            // uniform: padding of the last group of 8
  const int qi = pair / nsplit;
  const int split = pair - qi * nsplit;
  const int unit = qi * ngroups + hg;                    // (query, head group)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ds = wv & 3, rg = wv >> 2;                  // latent slice, row group
  const int g = lane >> 4, r = lane & 15;
  const int head = hg * 16 + r;
  const int n_all = max(0, min(cnt[qi], k));            // counts outside [0, k] are clamped
  const int ntiles_all = (n_all + kTileRows - 1) / kTileRows;
  const int per_split = (ntiles_all + nsplit - 1) / nsplit;
  const int j0 = split * per_split * kTileRows;         // first selected row of this share
  const int n = max(0, min(n_all, j0 + per_split * kTileRows) - j0);

  // Q^T operand: head r, K-step s holds dims 128*ds + 32*g + 8*s .. +7.
  bf16x8 qop[4];
  {
    const bool ok = head < h;
    const uint4* src = reinterpret_cast<const uint4*>(q + ((int64_t)qi * h + (ok ? head : 0)) * kLatent + 128 * ds + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) qop[s] = __builtin_bit_cast(bf16x8, ok ? src[s] : make_uint4(0, 0, 0, 0));
  }
  // physical rows of the share, resolved once (index loads clamped to the
  // row of k entries so they need not wait for the count)
  {
    const int32_t* pt_row = c.page_table + (int64_t)q_seq[qi] * c.max_pages;
    const int32_t* irow = idx + (int64_t)qi * k;
    for (int j = tid; j < per_split * kTileRows; j += kThreads) {
      const int t = irow[min(j0 + j, k - 1)];
      if (j < n) S.row[j] = (uint32_t)entry_row_clamped(pt_row, t, c);
    }
  }
  lds_barrier();

  floatx4 oacc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) oacc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  // Running max of the unscaled logits q.X (finite: the first tile with a
  // visible row replaces it) and running sum of 2^((v - m_run) * c2) =
  // e^(sm_scale (v - m_run)).
  float m_run = -FLT_MAX, l_run = 0.0f;
  const float c2 = sm_scale * 1.44269504088896341f;       // sm_scale * log2(e)
  const float slack = kRescaleSlack / sm_scale;            // the rescale slack in unscaled units
  const int ntiles = (n + kTileRows - 1) / kTileRows;
  const int ntiles_rg = (ntiles + RG - 1) / RG;          // tiles rg, rg + RG, ... of this row group
  uint8_t* xs = &S.xs[wv][0];

  // Ring of row gathers.  Lanes 4i .. 4i+3 read row i's 64 code bytes of
  // this slice (one 32-value scale block each) and its 4 scale bytes, so a
  // load covers whole row segments; slot u holds tile t0+u (two groups of 16
  // rows).  Loads are unconditional (a row past the share reads physical row
  // 0, which always exists) so the compiler counts gathers in flight instead
  // of draining them.
  const int grow = lane >> 2, gblk = lane & 3;          // gather layout: row, scale block
  uint4 cd[kPrefetch][2];
  uint32_t sb[kPrefetch][2];
  auto gather = [&](int tt, uint4 (&c2)[2], uint32_t (&s2)[2]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int j = (rg + RG * tt) * kTileRows + mt * 16 + grow;
      const uint8_t* src = c.kv + (size_t)(j < n ? S.row[j] : 0u) * kKvRowBytes;
      c2[mt] = *reinterpret_cast<const uint4*>(src + 64 * ds + 16 * gblk);
      s2[mt] = src[kCodeBytes + 4 * ds + gblk];
    }
  };
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) gather(u, cd[u], sb[u]);

  // The trip count is padded to whole rings (tiles past the share are masked)
  // so the ring slots are consumed in a fixed order; it is the same for every
  // row group, so all waves meet the same barriers.
  const int ntiles_pad = (ntiles_rg + kPrefetch - 1) / kPrefetch * kPrefetch;
  for (int t0 = 0; t0 < ntiles_pad; t0 += kPrefetch) {
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) {
    const int tt = t0 + u;
    const int lim = n - (rg + RG * tt) * kTileRows;     // rows of this tile inside the share
    // ---- dequantise (gather layout) into this wave's bf16 slice rows ----
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      // a row past the share keeps its (finite) codes but gets scale 1: its
      // logit is masked below, so it only ever meets a zero probability
      const float scale = e8m0_to_float(mt * 16 + grow < lim ? sb[u][mt] : 127u);
      const uint32_t wds[4] = {cd[u][mt].x, cd[u][mt].y, cd[u][mt].z, cd[u][mt].w};
      uint8_t* rowp = xs + (mt * 16 + grow) * kSliceStride + 64 * gblk;
#pragma unroll
      for (int s = 0; s < 4; ++s) *reinterpret_cast<bf16x8*>(rowp + 16 * s) = dequant8(wds[s], scale);
    }
    gather(tt + kPrefetch, cd[u], sb[u]);               // refill the slot kPrefetch tiles ahead
    // ---- partial S^T over this slice: the A operand (row r, dims 32g + 8s)
    //      read back from the slice rows ----
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const uint8_t* rowp = xs + (mt * 16 + r) * kSliceStride + 64 * g;
      floatx4 st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(rowp + 16 * s), qop[s], st,
                                                     0, 0, 0);
      S.sp[RG == 2 ? (tt & 1) : 0][rg][ds][mt][g][r] = st;   // lanes write consecutive 16 B: no bank conflicts
    }
    lds_barrier();
    // ---- full scores of head r, rows mt*16 + 4g + i (fixed summation order) ----
    float v[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int sb = RG == 2 ? (tt & 1) : 0;
      floatx4 acc = S.sp[sb][rg][0][mt][g][r];
#pragma unroll
      for (int d2 = 1; d2 < 4; ++d2) acc += S.sp[sb][rg][d2][mt][g][r];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[mt][i] = acc[i];
    }
    if (lim < kTileRows) {                              // uniform: only a tile holding the end of the share
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (mt * 16 + 4 * g + i >= lim) v[mt][i] = -INFINITY;
    }
    float tmax = fmaxf(fmaxf(fmaxf(v[0][0], v[0][1]), fmaxf(v[0][2], v[0][3])),
                       fmaxf(fmaxf(v[1][0], v[1][1]), fmaxf(v[1][2], v[1][3])));
    tmax = halves_max(rows_pair_max(tmax));
    // rescale only when the max moved by more than the slack
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + slack)) {
      const float m_new = tmax > m_run + slack ? tmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);   // first visible tile: 0
      l_run *= alpha;
      m_run = m_new;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);   // O rows are heads 4g+i
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[nt][i] *= al[i];
    }
    const float mc = -m_run * c2;
    float p[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[mt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[mt][i], c2, mc));   // masked (-inf) -> 0
        psum += p[mt][i];
      }
    psum = halves_sum(rows_pair_sum(psum));
    l_run += psum;
    // p = hi + lo, both bf16 (V_CVT_PK_BF16_F32, round to nearest even)
    uint32_t whi[4], wlo[4];
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const float a = p[pr >> 1][2 * (pr & 1)], b = p[pr >> 1][2 * (pr & 1) + 1];
      const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2{a, b}), bf16x2));
      const float ra = a - __uint_as_float(hi << 16), rb = b - __uint_as_float(hi & 0xFFFF0000u);
      whi[pr] = hi;
      wlo[pr] = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2{ra, rb}), bf16x2));
    }
    const bf16x8 pa_hi = __builtin_bit_cast(bf16x8, make_uint4(whi[0], whi[1], whi[2], whi[3]));
    const bf16x8 pa_lo = __builtin_bit_cast(bf16x8, make_uint4(wlo[0], wlo[1], wlo[2], wlo[3]));
    // ---- O[16 heads][slice] += P X_slice: rows 4g+j and 16+4g+j through transposing reads ----
    const int off_a = (4 * g + (r >> 2)) * kSliceStride + 8 * (r & 3);
    const int off_b = off_a + 16 * kSliceStride;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const shortx4 lo = lds_read_tr16(xs, off_a + 32 * nt);
      const shortx4 hi = lds_read_tr16(xs, off_b + 32 * nt);
      typedef short shortx8 __attribute__((ext_vector_type(8)));
      const shortx8 b8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8 xb = __builtin_bit_cast(bf16x8, b8);
      oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, xb, oacc[nt], 0, 0, 0);
      oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, xb, oacc[nt], 0, 0, 0);
    }
    // With two partial-S buffers, a wave may write tile t+1's partial while
    // others still read tile t's: every read of the buffer it overwrites
    // (tile t-1) came before this tile's barrier.  Slice rows are per wave.
    if (RG != 2) lds_barrier();
  }
  }

  if (RG > 1) {
    // Row groups 1 .. RG-1 hand their (O, running max, running sum) to row
    // group 0 through the freed slice-row buffers; row group 0 merges them.
    constexpr int kMergeFloats = 64 * 34;                 // per wave: 32 outputs + max + sum per lane
    float* mbuf = reinterpret_cast<float*>(&S.xs[0][0]);
    lds_barrier();                                        // every wave is done with its slice rows
    if (rg > 0) {
      float* mine = mbuf + ((rg - 1) * 4 + ds) * kMergeFloats + lane * 34;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[4 * nt + i] = oacc[nt][i];
      mine[32] = m_run;
      mine[33] = l_run;
    }
    lds_barrier();
    if (rg > 0) return;                                   // no barrier follows
#pragma unroll
    for (int o = 1; o < RG; ++o) {
      const float* other = mbuf + ((o - 1) * 4 + ds) * kMergeFloats + lane * 34;
      const float m_o = other[32], l_o = other[33];
      const float m_new = fmaxf(m_run, m_o);
      const float a_me = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      const float a_o = __builtin_amdgcn_exp2f((m_o - m_new) * c2);
      l_run = a_me * l_run + a_o * l_o;
      m_run = m_new;
      float am[4], ao[4];                                 // O rows are heads 4g+i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        am[i] = __shfl(a_me, 4 * g + i);
        ao[i] = __shfl(a_o, 4 * g + i);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[nt][i] = am[i] * oacc[nt][i] + ao[i] * other[4 * nt + i];
    }
  }

  if (nsplit == 1) {
    float linv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float Li = __shfl(l_run, 4 * g + i);
      linv[i] = Li > 0.0f ? 1.0f / Li : 0.0f;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hd = hg * 16 + 4 * g + i;
        if (hd < h) out[((int64_t)qi * h + hd) * kLatent + 128 * ds + 16 * nt + r] = oacc[nt][i] * linv[i];
      }
    if (lse != nullptr && ds == 0 && g == 0 && head < h)
      lse[(int64_t)qi * h + head] = l_run > 0.0f ? m_run * sm_scale + __logf(l_run) : -INFINITY;
    return;
  }
  // share of a split unit: unnormalised output, running max and sum
  const int64_t pbase = (int64_t)unit * nsplit + split;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      part_o[(pbase * 16 + 4 * g + i) * kLatent + 128 * ds + 16 * nt + r] = oacc[nt][i];
  if (ds == 0 && g == 0) {
    part_ml[pbase * 32 + r] = l_run > 0.0f ? m_run * sm_scale : -INFINITY;   // the combine works in scaled units
    part_ml[pbase * 32 + 16 + r] = l_run;
  }
}

// Large batches (prefill): one workgroup of 16 waves serves the 64 heads of
// a query (4 head groups of 16).  Wave (head group hg, slice ds) gathers and
// dequantises 8 of the tile's 32 rows of slice ds into slice rows that the
// four head groups share, so each selected row is fetched and converted once
// per query instead of once per head group.  Per head group the arithmetic is
// that of sparse_attn_kernel<1> (the same partial sums in the same order, the
// same softmax and P split), so both forms give identical bits.  Slice rows
// and partial-S tiles are double buffered: two barriers per tile.
constexpr int kHg = 4;                                  // head groups per workgroup

struct AttnHgShared {
  uint8_t xs[2][4][kSliceBytes];     // [buffer][slice] bf16 slice rows of the tile (73,728 B)
  floatx4 sp[2][kHg][4][2][4][16];   // [buffer][head group][slice]: partial S^T (65,536 B)
  uint32_t row[kMaxShareRows];       // physical row of every selected entry (8,192 B)
};

__global__ void __launch_bounds__(256 * kHg, 1)
sparse_attn_hg_kernel(CacheArgs c, const uint16_t* __restrict__ q, const int32_t* __restrict__ q_seq,
                      const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int h, int k,
                      float sm_scale, float* __restrict__ out, float* __restrict__ lse, int nunits, int per_xcd) {
  __shared__ AttnHgShared S;
  // Block order: XCD x (blocks go to XCDs round-robin) serves the units
  // x * per_xcd .. x * per_xcd + per_xcd - 1, so neighbouring queries, which
  // select many of the same rows, share that XCD's L2.
  const int b = blockIdx.x;
  const int unit = (b & 7) * per_xcd + (b >> 3);         // (query, quad of head groups)
  if (unit >= nunits) return;                            // uniform
  const int nquads = h / (16 * kHg);
  const int qi = unit / nquads, hq = unit - qi * nquads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ds = wv & 3, hgl = wv >> 2;                 // latent slice, head group within the quad
  const int g = lane >> 4, r = lane & 15;
  const int hg = hq * kHg + hgl;
  const int head = hg * 16 + r;                          // < h: h is a multiple of 64
  const int n = max(0, min(cnt[qi], k));                // counts outside [0, k] are clamped

  // Q^T operand: head r, K-step s holds dims 128*ds + 32*g + 8*s .. +7.
  bf16x8 qop[4];
  {
    const uint4* src = reinterpret_cast<const uint4*>(q + ((int64_t)qi * h + head) * kLatent + 128 * ds + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) qop[s] = __builtin_bit_cast(bf16x8, src[s]);
  }
  const int ntiles = (n + kTileRows - 1) / kTileRows;
  {
    const int32_t* pt_row = c.page_table + (int64_t)q_seq[qi] * c.max_pages;
    const int32_t* irow = idx + (int64_t)qi * k;
    for (int j = tid; j < ntiles * kTileRows; j += 256 * kHg) {
      const int t = irow[min(j, k - 1)];
      if (j < n) S.row[j] = (uint32_t)entry_row_clamped(pt_row, t, c);
    }
  }
  lds_barrier();

  floatx4 oacc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) oacc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -FLT_MAX, l_run = 0.0f;
  const float c2 = sm_scale * 1.44269504088896341f;
  const float slack = kRescaleSlack / sm_scale;

  // Ring of row gathers: lanes 8i .. 8i+7 read 8 code bytes each of row
  // 8 * hgl + i's 64-byte segment of this slice, and the scale byte of their
  // 32-value block.  Loads are unconditional (rows past the selection read
  // physical row 0, which always exists).
  const int grow = 8 * hgl + (lane >> 3), gpart = lane & 7;
  uint2 cd[kPrefetch];
  uint32_t sb[kPrefetch];
  auto gather = [&](int tt, uint2& cw, uint32_t& sw) {
    const int j = tt * kTileRows + grow;
    const uint8_t* src = c.kv + (size_t)(j < n ? S.row[j] : 0u) * kKvRowBytes;
    cw = *reinterpret_cast<const uint2*>(src + 64 * ds + 8 * gpart);
    sw = src[kCodeBytes + 4 * ds + (gpart >> 1)];
  };
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) gather(u, cd[u], sb[u]);

  const int ntiles_pad = (ntiles + kPrefetch - 1) / kPrefetch * kPrefetch;
  for (int t0 = 0; t0 < ntiles_pad; t0 += kPrefetch) {
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) {
    const int tt = t0 + u;
    const int buf = tt & 1;
    const int lim = n - tt * kTileRows;                 // rows of this tile inside the selection
    uint8_t* xs = &S.xs[buf][ds][0];
    {
      // a row past the selection keeps its (finite) codes but gets scale 1:
      // its logit is masked below, so it only ever meets a zero probability
      const float scale = e8m0_to_float(grow < lim ? sb[u] : 127u);
      uint8_t* rowp = xs + grow * kSliceStride + 32 * gpart;
      *reinterpret_cast<bf16x8*>(rowp) = dequant8(cd[u].x, scale);
      *reinterpret_cast<bf16x8*>(rowp + 16) = dequant8(cd[u].y, scale);
    }
    gather(tt + kPrefetch, cd[u], sb[u]);
    // the tile's slice rows are complete; the buffers of tile tt-2 were
    // last read before every wave reached the previous tile's first barrier
    lds_barrier();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const uint8_t* rowp = xs + (mt * 16 + r) * kSliceStride + 64 * g;
      floatx4 st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(rowp + 16 * s), qop[s], st,
                                                     0, 0, 0);
      S.sp[buf][hgl][ds][mt][g][r] = st;
    }
    lds_barrier();
    float v[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      floatx4 acc = S.sp[buf][hgl][0][mt][g][r];
#pragma unroll
      for (int d2 = 1; d2 < 4; ++d2) acc += S.sp[buf][hgl][d2][mt][g][r];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[mt][i] = acc[i];
    }
    if (lim < kTileRows) {                              // uniform: only a tile holding the end of the selection
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (mt * 16 + 4 * g + i >= lim) v[mt][i] = -INFINITY;
    }
    float tmax = fmaxf(fmaxf(fmaxf(v[0][0], v[0][1]), fmaxf(v[0][2], v[0][3])),
                       fmaxf(fmaxf(v[1][0], v[1][1]), fmaxf(v[1][2], v[1][3])));
    tmax = halves_max(rows_pair_max(tmax));
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + slack)) {
      const float m_new = tmax > m_run + slack ? tmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      l_run *= alpha;
      m_run = m_new;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[nt][i] *= al[i];
    }
    const float mc = -m_run * c2;
    float p[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[mt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[mt][i], c2, mc));
        psum += p[mt][i];
      }
    psum = halves_sum(rows_pair_sum(psum));
    l_run += psum;
    uint32_t whi[4], wlo[4];
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const float a = p[pr >> 1][2 * (pr & 1)], b2 = p[pr >> 1][2 * (pr & 1) + 1];
      const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2{a, b2}), bf16x2));
      const float ra = a - __uint_as_float(hi << 16), rb = b2 - __uint_as_float(hi & 0xFFFF0000u);
      whi[pr] = hi;
      wlo[pr] = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2{ra, rb}), bf16x2));
    }
    const bf16x8 pa_hi = __builtin_bit_cast(bf16x8, make_uint4(whi[0], whi[1], whi[2], whi[3]));
    const bf16x8 pa_lo = __builtin_bit_cast(bf16x8, make_uint4(wlo[0], wlo[1], wlo[2], wlo[3]));
    const int off_a = (4 * g + (r >> 2)) * kSliceStride + 8 * (r & 3);
    const int off_b = off_a + 16 * kSliceStride;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const shortx4 lo = lds_read_tr16(xs, off_a + 32 * nt);
      const shortx4 hi = lds_read_tr16(xs, off_b + 32 * nt);
      typedef short shortx8 __attribute__((ext_vector_type(8)));
      const shortx8 b8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8 xb = __builtin_bit_cast(bf16x8, b8);
      oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, xb, oacc[nt], 0, 0, 0);
      oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, xb, oacc[nt], 0, 0, 0);
    }
  }
  }

  float linv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float Li = __shfl(l_run, 4 * g + i);
    linv[i] = Li > 0.0f ? 1.0f / Li : 0.0f;
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hd = hg * 16 + 4 * g + i;
      out[((int64_t)qi * h + hd) * kLatent + 128 * ds + 16 * nt + r] = oacc[nt][i] * linv[i];
    }
  if (lse != nullptr && ds == 0 && g == 0)
    lse[(int64_t)qi * h + head] = l_run > 0.0f ? m_run * sm_scale + __logf(l_run) : -INFINITY;
}

// Decode batches: one workgroup per (query, 16-head group, half of the
// latent's output dims), so a batch of 32 queries with 64 heads fills all 256
// CUs, with the 8 workgroups of a query on one XCD (blocks go to XCDs
// round-robin), where they share the gathered rows through its L2.  Each of
// its W waves owns whole 32-row tiles (tiles wv, wv + W, ...):
//   - Q.X^T over all 512 dims straight from registers: lane (row r, group g)
//     gathers bytes [64c + 16g, +16) of chunk c of its row (dims
//     [128c + 32g, +32), one scale block), dequantises 8 dims per K-step with
//     V_CVT_SCALEF32_PK_BF16_FP4 into the A operand of a bf16 16x16x32 MFMA
//     whose K order is permuted alike in the Q operand; no LDS, no exchange
//     of partial scores, no barrier;
//   - the online softmax of its rows in registers (as sparse_attn_kernel);
//   - O[16 heads][its 256 dims] += P X with the dequantised rows of its half
//     written to the wave's own LDS rows (the values the QK step converted)
//     and read back transposed (DS_READ_B64_TR_B16), P split into bf16 hi+lo.
// The waves merge their (O, running max, running sum) through LDS at the end,
// each wave producing 16 / W n-tiles of the output.
constexpr int kDsHalf = 256;                        // output dims per workgroup
constexpr int kPtRegPages = 256;                    // page-table rows held in registers up to this length
constexpr int kDsStride = 2 * kDsHalf + 32;         // bytes per staged bf16 row (512 + 32 pad)

template <int W>
struct AttnDsShared {
  uint8_t xs[W][kTileRows * kDsStride];    // [wave] staged rows of its current tile, this half (17,408 B each)
  uint32_t row[kMaxShareRows + 1];         // physical row of every selected entry (8,192 B), a sink slot
  float m[W][16];
  float l[W][16];
};

template <int W>
__global__ void __launch_bounds__(64 * W, 1)
sparse_attn_ds_kernel(CacheArgs c, const uint16_t* __restrict__ q, const int32_t* __restrict__ q_seq,
                      const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int nq, int h, int k,
                      float sm_scale, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ AttnDsShared<W> S;
  static_assert(sizeof(S.xs) >= (size_t)W * 16 * 64 * 16, "merge buffer aliases the staged rows");
  const int ngroups = (h + 15) >> 4;
  const int upq = 2 * ngroups;                           // units per query: head groups x halves
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int qx = slot / upq, u = slot - qx * upq;
  const int qi = qx * 8 + xcd;
  if (qi >= nq) return;                                  // uniform
  const int hg = u >> 1, half = u & 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int head = hg * 16 + r;
  const int n = max(0, min(cnt[qi], k));                // counts outside [0, k] are clamped
  const int ntiles = (n + kTileRows - 1) / kTileRows;

  // The four 128-dim chunks of the latent in slot order: slots 0 and 1 are
  // this workgroup's half (their dequantised rows are staged for P.V), slots
  // 2 and 3 the other half (Q.X^T only).  chunk(s) = (s + 2 half) mod 4.
  const int ch_of[4] = {2 * half, 2 * half + 1, 2 - 2 * half, 3 - 2 * half};
  // Physical rows of this wave's own tiles (wv, wv + W, ...; half a wave per
  // tile), resolved by the wave itself, so no workgroup barrier stands
  // between a wave's lookups and its first gathers.  The loads the lookups
  // need go out first and together: the page-table row when it has at most
  // kPtRegPages entries (into the wave's registers, lane l: entries l + 64 i,
  // looked up with cross-lane reads; a longer row is read per index) and the
  // indices of the wave's first eight tiles (clamped to the k-entry row and
  // loaded whatever the count, so they wait neither for it nor for each
  // other), with the Q operand's loads in the same trip.  (Index loads under
  // a branch each waited for the one before: four trips, then four more for
  // the page ids.)
  const int32_t* pt_row = c.page_table + (int64_t)q_seq[qi] * c.max_pages;
  const int32_t* irow = idx + (int64_t)qi * k;
  const int ktiles = (k + kTileRows - 1) / kTileRows;
  const bool pt_regs = c.max_pages <= kPtRegPages;        // uniform
  const int npr = (c.max_pages + 63) >> 6;
  int ptv[kPtRegPages / 64];
  // indices of tiles wv + W (i0 + 2u), u < 4, with i0 = i0b + (lane >= 32)
  auto index_loads = [&](int i0b, int (&tv)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int T = wv + W * (i0b + (lane >> 5) + 2 * u);
      tv[u] = irow[min(T * kTileRows + (lane & 31), k - 1)];
    }
  };
  const int tmax = (c.max_pages << c.lg_page) - 1;
  // (kRegs: the row is in ptv; neither form loads under a branch)
  auto lookups = [&](int i0b, const int (&tv)[4], auto regs) {
    constexpr bool kRegs = decltype(regs)::value;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int T = wv + W * (i0b + (lane >> 5) + 2 * u);
      const int j = T * kTileRows + (lane & 31);
      const int t = min(max(tv[u], 0), tmax);            // (as entry_row_clamped)
      const int pg = t >> c.lg_page;
      int page = 0;
      if constexpr (kRegs) {
#pragma unroll
        for (int i = 0; i < kPtRegPages / 64; ++i)
          if (i < npr) {                                 // (uniform)
            const int v = __builtin_amdgcn_ds_bpermute((pg & 63) << 2, ptv[i]);
            page = (pg >> 6) == i ? v : page;
          }
      } else {
        page = pt_row[pg];
      }
      // (stored by every lane, the ones outside the selection into a sink
      // slot, so no load above moves into a branch)
      S.row[T < ktiles && j < n ? j : kMaxShareRows] =
          ((uint32_t)clamp_page(page, c) << c.lg_page) + (uint32_t)(t & ((1 << c.lg_page) - 1));
    }
  };
  // Q^T operand: head r; slot s, K-step t holds dims 128 chunk(s) + 32 g + 8 t .. +7.
  // Lanes of heads past h load head 0 (their columns of S and rows of O are
  // computed but never stored).
  bf16x8 qop[4][4];
  const uint4* qsrc = reinterpret_cast<const uint4*>(q + ((int64_t)qi * h + (head < h ? head : 0)) * kLatent + 32 * g);
  // (one instance per form, each with its loads in the order above)
  auto prologue = [&](auto regs) {
    if constexpr (decltype(regs)::value) {
#pragma unroll
      for (int i = 0; i < kPtRegPages / 64; ++i) ptv[i] = pt_row[min(lane + 64 * i, c.max_pages - 1)];
    }
    int tv0[4];
    index_loads(0, tv0);
    // (the Q loads stay behind the index loads: loads complete in order, so
    // the lookups then wait for the indices alone)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
      for (int t = 0; t < 4; ++t) qop[sl][t] = __builtin_bit_cast(bf16x8, qsrc[16 * ch_of[sl] + t]);
    lookups(0, tv0, regs);
    for (int i0b = 8; wv + W * i0b < ktiles; i0b += 8) {    // (k > 32 W tiles only)
      int tv[4];
      index_loads(i0b, tv);
      lookups(i0b, tv, regs);
    }
  };
  if (pt_regs)
    prologue(std::true_type{});
  else
    prologue(std::false_type{});
  __builtin_amdgcn_wave_barrier();                       // the wave's row writes stay above its gathers

  floatx4 oacc[16];
#pragma unroll
  for (int nt = 0; nt < 16; ++nt) oacc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -FLT_MAX, l_run = 0.0f;
  const float c2 = sm_scale * 1.44269504088896341f;
  const float slack = kRescaleSlack / sm_scale;
  uint8_t* const xs = &S.xs[wv][0];
  const int my_tiles = ntiles > wv ? (ntiles - wv + W - 1) / W : 0;

  // Gathers of one tile (rows past the selection read physical row 0, which
  // always exists): per M-tile, the row's four 16-byte code pieces of this
  // lane's group, in slot order, and its 16 scale bytes.  Loads are
  // unconditional.
  struct Gath {
    uint4 cd[2][4];
    uint4 sc[2];
  };
  auto gather = [&](int tt, Gath& G) {
    const int T = wv + W * min(tt, my_tiles - 1);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int j = T * kTileRows + mt * 16 + r;
      const uint8_t* src = c.kv + (size_t)(j < n ? S.row[j] : 0u) * kKvRowBytes;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
        G.cd[mt][sl] = *reinterpret_cast<const uint4*>(src + 64 * ch_of[sl] + 16 * g);
      G.sc[mt] = *reinterpret_cast<const uint4*>(src + kCodeBytes);
    }
  };
  auto process = [&](int tt, const Gath& G) {
    const int T = wv + W * tt;
    const int lim = n - T * kTileRows;                   // rows of this tile inside the selection
    // S^T = X Q^T as four independent accumulator chains (M-tile, K-step
    // parity), so consecutive matrix-core ops never wait on each other;
    // straight-line code (no branch per K-step) lets the conversions of the
    // next step run under the current one
    floatx4 st[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) st[mt][0] = st[mt][1] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    float scale[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      // a row past the selection keeps its (finite) codes but gets scale 1:
      // its logit is masked below, so it only ever meets a zero probability
      const bool valid = mt * 16 + r < lim;
      const uint32_t scw[4] = {G.sc[mt].x, G.sc[mt].y, G.sc[mt].z, G.sc[mt].w};
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        // dword chunk(s) of the scale bytes, picked without dynamic indexing
        const uint32_t d = half ? scw[(sl + 2) & 3] : scw[sl];
        scale[mt][sl] = e8m0_to_float(valid ? (d >> (8 * g)) & 0xFFu : 127u);
      }
    }
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const uint32_t wd = t == 0 ? G.cd[mt][sl].x : t == 1 ? G.cd[mt][sl].y : t == 2 ? G.cd[mt][sl].z
                                                                                          : G.cd[mt][sl].w;
          const bf16x8 a = dequant8(wd, scale[mt][sl]);
          st[mt][t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[sl][t], st[mt][t & 1], 0, 0, 0);
          if (sl < 2)                                    // this half's dims go to the staged rows
            *reinterpret_cast<bf16x8*>(xs + (mt * 16 + r) * kDsStride + 64 * g + 256 * sl + 16 * t) = a;
        }
    float v[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[mt][i] = st[mt][0][i] + st[mt][1][i];
    if (lim < kTileRows) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (mt * 16 + 4 * g + i >= lim) v[mt][i] = -INFINITY;
    }
    float tmax = fmaxf(fmaxf(fmaxf(v[0][0], v[0][1]), fmaxf(v[0][2], v[0][3])),
                       fmaxf(fmaxf(v[1][0], v[1][1]), fmaxf(v[1][2], v[1][3])));
    tmax = halves_max(rows_pair_max(tmax));
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + slack)) {
      const float m_new = tmax > m_run + slack ? tmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      l_run *= alpha;
      m_run = m_new;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int nt = 0; nt < 16; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[nt][i] *= al[i];
    }
    const float mc = -m_run * c2;
    float p[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[mt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[mt][i], c2, mc));
        psum += p[mt][i];
      }
    psum = halves_sum(rows_pair_sum(psum));
    l_run += psum;
    uint32_t whi[4], wlo[4];
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const float a = p[pr >> 1][2 * (pr & 1)], b2 = p[pr >> 1][2 * (pr & 1) + 1];
      const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2{a, b2}), bf16x2));
      const float ra = a - __uint_as_float(hi << 16), rb = b2 - __uint_as_float(hi & 0xFFFF0000u);
      whi[pr] = hi;
      wlo[pr] = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2{ra, rb}), bf16x2));
    }
    const bf16x8 pa_hi = __builtin_bit_cast(bf16x8, make_uint4(whi[0], whi[1], whi[2], whi[3]));
    const bf16x8 pa_lo = __builtin_bit_cast(bf16x8, make_uint4(wlo[0], wlo[1], wlo[2], wlo[3]));
    // the staged rows were written by this wave: LDS keeps a wave's accesses
    // in order, and the wave barrier keeps the compiler from moving the reads
    // above the writes
    __builtin_amdgcn_wave_barrier();
    const int off_a = (4 * g + (r >> 2)) * kDsStride + 8 * (r & 3);
    const int off_b = off_a + 16 * kDsStride;
    // groups of four n-tiles: their hi terms, then their lo terms, so each
    // accumulator's two updates are four matrix-core ops apart
#pragma unroll
    for (int n0 = 0; n0 < 16; n0 += 4) {
      bf16x8 xb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const shortx4 lo = lds_read_tr16(xs, off_a + 32 * (n0 + u));
        const shortx4 hi = lds_read_tr16(xs, off_b + 32 * (n0 + u));
        typedef short shortx8 __attribute__((ext_vector_type(8)));
        const shortx8 b8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        xb[u] = __builtin_bit_cast(bf16x8, b8);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        oacc[n0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, xb[u], oacc[n0 + u], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        oacc[n0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, xb[u], oacc[n0 + u], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();                     // the next tile's row writes stay below these reads
  };
  if (my_tiles > 0) {
    Gath ga, gb;
    gather(0, ga);
    int tt = 0;
    for (; tt + 2 < my_tiles; tt += 2) {                 // two or more tiles after these
      gather(tt + 1, gb);
      process(tt, ga);
      gather(tt + 2, ga);
      process(tt + 1, gb);
    }
    // the last one or two: nothing is gathered past the wave's tiles, so the
    // merge below waits for no load
    if (tt + 1 < my_tiles) {
      gather(tt + 1, gb);
      process(tt, ga);
      process(tt + 1, gb);
    } else {
      process(tt, ga);
    }
  }

  // merge the waves: every wave publishes (O, m, l); wave wv then combines
  // n-tiles [wv * 16 / W, (wv + 1) * 16 / W) of all of them
  lds_barrier();                                         // every wave is done with its staged rows
  floatx4* const mb = reinterpret_cast<floatx4*>(&S.xs[0][0]);
#pragma unroll
  for (int nt = 0; nt < 16; ++nt) mb[(wv * 16 + nt) * 64 + lane] = oacc[nt];
  if (g == 0) {
    S.m[wv][r] = m_run;
    S.l[wv][r] = l_run;
  }
  lds_barrier();
  float Mx[4], linv[4], ap[W][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * g + i;                            // O rows of this lane are heads 4g + i
    float M = -FLT_MAX;
#pragma unroll
    for (int w2 = 0; w2 < W; ++w2) M = fmaxf(M, S.m[w2][hh]);
    float L = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < W; ++w2) {
      ap[w2][i] = __builtin_amdgcn_exp2f((S.m[w2][hh] - M) * c2);
      L += ap[w2][i] * S.l[w2][hh];
    }
    Mx[i] = M;
    linv[i] = L > 0.0f ? 1.0f / L : 0.0f;
    if (lse != nullptr && half == 0 && wv == 0 && r == 0 && hg * 16 + hh < h)
      lse[(int64_t)qi * h + hg * 16 + hh] = L > 0.0f ? M * sm_scale + __logf(L) : -INFINITY;
  }
  (void)Mx;
  constexpr int kNtPer = 16 / W;
#pragma unroll
  for (int u2 = 0; u2 < kNtPer; ++u2) {
    const int nt = wv * kNtPer + u2;
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w2 = 0; w2 < W; ++w2) {
      const floatx4 o = mb[(w2 * 16 + nt) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += ap[w2][i] * o[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hd = hg * 16 + 4 * g + i;
      if (hd < h) out[((int64_t)qi * h + hd) * kLatent + kDsHalf * half + 16 * nt + r] = acc[i] * linv[i];
    }
  }
}

// Shared-row workgroups (sparse_attn_hg_kernel) need a batch that gives every
// CU a few of them; below that the 16-head form spreads the work wider.
constexpr int64_t kHgMinUnits = 512;
// Batches of fewer (query, 16-head group) units than this (decode) take
// sparse_attn_ds_kernel, with kDsWaves waves per workgroup; larger ones the
// shared-row form or one workgroup per (query, 16-head group).
constexpr int64_t kDsMaxUnits = 512;
constexpr int kDsWaves = 4;

hipError_t launch_sparse_attn(const CacheArgs& c, const uint16_t* q, const int32_t* q_seq, const int32_t* idx,
                              const int32_t* cnt, int nq, int h, int k, float sm_scale, float* out, float* lse,
                              bool share_heads, hipStream_t s, const KEvents& ev) {
  if (nq <= 0 || h <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  const int ngroups = (h + 15) / 16;
  const int64_t units = (int64_t)nq * ngroups;
  if (units < kDsMaxUnits) {
    // decode batches: (query, head group, half of the dims) workgroups
    const int64_t blocks = (int64_t)((nq + 7) / 8) * 2 * ngroups * 8;
    launch(sparse_attn_ds_kernel<kDsWaves>, dim3((unsigned)blocks), dim3(64 * kDsWaves), s, ev, c, q, q_seq, idx,
           cnt, nq, h, k, sm_scale, out, lse);
    return hipGetLastError();
  }
  const int64_t hg_units = (h % (16 * kHg) == 0) ? (int64_t)nq * (h / (16 * kHg)) : 0;
  if (share_heads && hg_units >= kHgMinUnits) {
    const int per_xcd = (int)((hg_units + 7) / 8);
    launch(sparse_attn_hg_kernel, dim3((unsigned)(per_xcd * 8)), dim3(256 * kHg), s, ev, c, q, q_seq, idx, cnt, h, k,
           sm_scale, out, lse, (int)hg_units, per_xcd);
  } else {
    const int64_t blocks = (int64_t)(nq + 7) / 8 * 8 * ngroups;
    launch(sparse_attn_kernel<1>, dim3((unsigned)blocks), dim3(256), s, ev, c, q, q_seq, idx, cnt, h, k, sm_scale,
           out, lse, 1, nq, static_cast<float*>(nullptr), static_cast<float*>(nullptr));
  }
  return hipGetLastError();
}

}  // namespace csa2
