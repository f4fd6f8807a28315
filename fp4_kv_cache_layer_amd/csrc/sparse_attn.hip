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

// Merges the nsplit shares of one (query, head): O = sum_s e^(m_s - M) O_s / L,
// L = sum_s e^(m_s - M) l_s, LSE = M + ln L.  One workgroup per head, one
// float4 of the output per thread, so every share is read in one round trip.
__global__ void __launch_bounds__(128)
attn_combine_kernel(int h, int nsplit, const float* __restrict__ part_o, const float* __restrict__ part_ml,
                    float* __restrict__ out, float* __restrict__ lse) {
  const int ngroups = (h + 15) >> 4;
  const int unit = blockIdx.x >> 4, hh = blockIdx.x & 15;
  const int qi = unit / ngroups, hg = unit - qi * ngroups;
  const int hd = hg * 16 + hh;
  if (hd >= h) return;
  const int tid = threadIdx.x;
  const float* ml = part_ml + (int64_t)unit * nsplit * 32;
  float M = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, ml[sp * 32 + hh]);
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4* po = reinterpret_cast<const float4*>(part_o + ((int64_t)unit * nsplit * 16 + hh) * kLatent);
  for (int sp = 0; sp < nsplit; ++sp) {
    const float ms = ml[sp * 32 + hh];
    const float f = (M == -INFINITY || ms == -INFINITY) ? 0.0f : __expf(ms - M);
    L += f * ml[sp * 32 + 16 + hh];
    const float4 x = po[(int64_t)sp * 16 * kLatent / 4 + tid];
    acc.x += f * x.x; acc.y += f * x.y; acc.z += f * x.z; acc.w += f * x.w;
  }
  const float linv = L > 0.0f ? 1.0f / L : 0.0f;
  acc.x *= linv; acc.y *= linv; acc.z *= linv; acc.w *= linv;
  reinterpret_cast<float4*>(out + ((int64_t)qi * h + hd) * kLatent)[tid] = acc;
  if (lse != nullptr && tid == 0) lse[(int64_t)qi * h + hd] = (M == -INFINITY) ? -INFINITY : M + __logf(L);
}

// Shared-row workgroups (sparse_attn_hg_kernel) need a batch that gives every
// CU a few of them; below that the 16-head form spreads the work wider.
constexpr int64_t kHgMinUnits = 512;

// Row groups per workgroup: small batches (decode) split each query's rows
// among 2 row groups of 4 waves inside one workgroup, merged through LDS;
// large batches already cover the chip with one 4-wave workgroup per unit.
static int attn_rgroups(int nq, int h) {
  const int units = nq * ((h + 15) / 16);
  return units < 256 ? 2 : 1;
}

int attn_nsplit(int nq, int h, int k) {
  const int units = nq * ((h + 15) / 16);
  const int ntiles = (k + kTileRows - 1) / kTileRows;
  const int rg = attn_rgroups(nq, h);
  // Splitting pays only while few units run: a split halves the tile loop but
  // adds the share write-out and a combine launch, which at 128 units (32
  // decode queries x 64 heads) already cost more than they save.
  const int target = rg > 1 ? 128 : 512;
  int ns = 1;
  // split across workgroups only while every row group keeps two tiles per share
  while (ns < 16 && units * ns < target && ntiles >= 2 * rg * 2 * ns) ns *= 2;
  while ((ntiles + ns - 1) / ns * kTileRows > kMaxShareRows) ns *= 2;   // shares must fit the row table
  return ns;
}

size_t attn_part_bytes(int nq, int h, int k) {
  const int ns = attn_nsplit(nq, h, k);
  if (ns == 1 || nq <= 0) return 0;
  const size_t units = (size_t)nq * ((h + 15) / 16);
  return (units * ns * (16 * kLatent + 32) * 4 + 255) / 256 * 256;
}

hipError_t launch_sparse_attn(const CacheArgs& c, const uint16_t* q, const int32_t* q_seq, const int32_t* idx,
                              const int32_t* cnt, int nq, int h, int k, float sm_scale, float* out, float* lse,
                              void* part, bool share_heads, hipStream_t s, const KEvents& ev) {
  if (nq <= 0 || h <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  const int ngroups = (h + 15) / 16;
  const int ns = part ? attn_nsplit(nq, h, k) : 1;
  const int64_t units = (int64_t)nq * ngroups;
  float* part_o = reinterpret_cast<float*>(part);
  float* part_ml = part_o ? part_o + units * ns * 16 * kLatent : nullptr;
  const int64_t npairs = (int64_t)nq * ns;
  const int64_t blocks = (npairs + 7) / 8 * 8 * ngroups;
  const int64_t hg_units = (h % (16 * kHg) == 0) ? (int64_t)nq * (h / (16 * kHg)) : 0;
  if (share_heads && ns == 1 && hg_units >= kHgMinUnits) {
    const int per_xcd = (int)((hg_units + 7) / 8);
    launch(sparse_attn_hg_kernel, dim3((unsigned)(per_xcd * 8)), dim3(256 * kHg), s, ev, c, q, q_seq, idx, cnt, h, k,
           sm_scale, out, lse, (int)hg_units, per_xcd);
  } else if (attn_rgroups(nq, h) == 2)
    launch(sparse_attn_kernel<2>, dim3((unsigned)blocks), dim3(256 * 2), s, ns > 1 ? ev.first() : ev, c, q, q_seq,
           idx, cnt, h, k, sm_scale, out, lse, ns, (int)npairs, part_o, part_ml);
  else
    launch(sparse_attn_kernel<1>, dim3((unsigned)blocks), dim3(256), s, ns > 1 ? ev.first() : ev, c, q, q_seq, idx,
           cnt, h, k, sm_scale, out, lse, ns, (int)npairs, part_o, part_ml);
  if (ns > 1)
    launch(attn_combine_kernel, dim3((unsigned)(units * 16)), dim3(128), s, ev.last(), h, ns, part_o, part_ml, out,
           lse);
  return hipGetLastError();
}

}  // namespace csa2
