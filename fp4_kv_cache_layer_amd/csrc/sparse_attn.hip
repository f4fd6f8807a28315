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
// Work split.  A (query, group of 16 heads) unit is cut into nsplit
// contiguous shares of its selected rows so that a small decode batch still
// covers the chip; a workgroup serves one share and writes its unnormalised
// output with its running max and sum, and a combine kernel merges the shares
// (nsplit = 1 writes the final output directly).  The four waves of a
// workgroup own the four 128-wide slices of the latent.  The workgroup first
// resolves the physical row of every selected entry of its share into LDS,
// then streams 32-row tiles with the row gathers of the next kPrefetch tiles
// in flight.  For every tile a wave
//   - gathers, for two rows per lane, the 16 code bytes of one 32-element
//     scale block of its slice and dequantises them with
//     V_CVT_SCALEF32_PK_BF16_FP4 straight into the A operand of
//     S^T = X Q^T (bf16 MFMA 16x16x32, K = its 128 dims, permuted alike in
//     the Q operand),
//   - publishes its partial S^T (32 rows x 16 heads) and its bf16 slice of the
//     rows in LDS (row stride 272 B: the 16-byte writes and the transposing
//     8-byte reads both spread evenly over the 64 banks),
//   - sums the four partial S^T (same order in every wave), runs the online
//     softmax (the output is rescaled only when the running max grows by more
//     than 8 nats, so probabilities stay below e^8) and accumulates
//     O[16 heads][its 128 dims] += P X with P split into bf16 hi + lo terms;
//     the B operand (rows as K) comes from LDS through the transposing read
//     DS_READ_B64_TR_B16.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kAttnThreads = 256;
constexpr int kTileRows = 32;
constexpr int kSliceStride = 272;                       // bytes per bf16 slice row (128 * 2 + 16 pad)
constexpr int kSliceBytes = kTileRows * kSliceStride;   // 8,704
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

struct AttnShared {
  uint8_t xs[4][kSliceBytes];        // [slice] bf16 rows of the current tile (34,816 B)
  floatx4 sp[4][2][4][16];           // partial S^T per wave: [m-tile][row quad][head] of 4 rows (8,192 B)
  uint32_t row[kMaxShareRows];       // physical row of every selected entry of the share (8,192 B)
};

__global__ void __launch_bounds__(kAttnThreads, 2)
sparse_attn_kernel(CacheArgs c, const uint16_t* __restrict__ q, const int32_t* __restrict__ q_seq,
                   const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int h, int k,
                   float sm_scale, float* __restrict__ out, float* __restrict__ lse, int nsplit,
                   float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ AttnShared S;
  const int ngroups = (h + 15) >> 4;
  const int unit = blockIdx.x / nsplit;                 // (query, head group)
  const int split = blockIdx.x - unit * nsplit;
  const int qi = unit / ngroups;
  const int hg = unit - qi * ngroups;
  const int tid = threadIdx.x, lane = tid & 63, ds = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int head = hg * 16 + r;
  const int n_all = cnt[qi];
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
    for (int j = tid; j < per_split * kTileRows; j += kAttnThreads) {
      const int t = irow[min(j0 + j, k - 1)];
      if (j < n) S.row[j] = (uint32_t)entry_row(pt_row, t, c.lg_page);
    }
  }
  lds_barrier();

  floatx4 oacc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) oacc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;
  const int ntiles = (n + kTileRows - 1) / kTileRows;
  uint8_t* xs = &S.xs[ds][0];

  // Ring of row gathers: slot u holds tile t0+u's 16 code bytes (one scale
  // block of this slice) and scale byte for two rows per lane.  Loads are
  // unconditional (a row past the share reads physical row 0, which always
  // exists) so the compiler counts gathers in flight instead of draining them.
  uint4 cd[kPrefetch][2];
  uint32_t sb[kPrefetch][2];
  auto gather = [&](int tile, uint4 (&c2)[2], uint32_t (&s2)[2]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int j = tile * kTileRows + mt * 16 + r;
      const uint8_t* src = c.kv + (size_t)(j < n ? S.row[j] : 0u) * kKvRowBytes;
      c2[mt] = *reinterpret_cast<const uint4*>(src + 64 * ds + 16 * g);
      s2[mt] = src[kCodeBytes + 4 * ds + g];
    }
  };
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) gather(u, cd[u], sb[u]);

  // The trip count is padded to whole rings (tiles past the share are masked)
  // so the ring slots are consumed in a fixed order.
  const int ntiles_pad = (ntiles + kPrefetch - 1) / kPrefetch * kPrefetch;
  for (int t0 = 0; t0 < ntiles_pad; t0 += kPrefetch) {
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) {
    const int tile = t0 + u;
    const int lim = n - tile * kTileRows;               // rows of this tile inside the share
    // ---- dequantise into the S^T A operand; partial S^T over this slice ----
    bf16x8 xa[2][4];
    floatx4 st[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      // a row past the share keeps its (finite) codes but gets scale 1: its
      // logit is masked below, so it only ever meets a zero probability
      const float scale = e8m0_to_float(mt * 16 + r < lim ? sb[u][mt] : 127u);
      const uint32_t wds[4] = {cd[u][mt].x, cd[u][mt].y, cd[u][mt].z, cd[u][mt].w};
      st[mt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        xa[mt][s] = dequant8(wds[s], scale);
        st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mt][s], qop[s], st[mt], 0, 0, 0);
      }
    }
    gather(tile + kPrefetch, cd[u], sb[u]);             // refill the slot kPrefetch tiles ahead
    // ---- publish the bf16 slice rows and the partial scores ----
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      uint8_t* rowp = xs + (mt * 16 + r) * kSliceStride + 64 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s) *reinterpret_cast<bf16x8*>(rowp + 16 * s) = xa[mt][s];
      S.sp[ds][mt][g][r] = st[mt];                      // lanes write consecutive 16 B: no bank conflicts
    }
    lds_barrier();
    // ---- full scores of head r, rows mt*16 + 4g + i (fixed summation order) ----
    float v[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      floatx4 acc = S.sp[0][mt][g][r];
#pragma unroll
      for (int d2 = 1; d2 < 4; ++d2) acc += S.sp[d2][mt][g][r];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[mt][i] = acc[i] * sm_scale;
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
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + kRescaleSlack)) {
      const float m_new = tmax > m_run + kRescaleSlack ? tmax : m_run;
      const float alpha = (m_new == m_run) ? 1.0f : __expf(m_run - m_new);   // m_run = -inf -> 0
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
    float p[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[mt][i] = m_run == -INFINITY ? 0.0f : __expf(v[mt][i] - m_run);   // -inf -> 0
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
    lds_barrier();
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
      lse[(int64_t)qi * h + head] = (m_run == -INFINITY) ? -INFINITY : m_run + __logf(l_run);
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
    part_ml[pbase * 32 + r] = m_run;
    part_ml[pbase * 32 + 16 + r] = l_run;
  }
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

int attn_nsplit(int nq, int h, int k) {
  const int units = nq * ((h + 15) / 16);
  const int ntiles = (k + kTileRows - 1) / kTileRows;
  int ns = 1;
  // aim at >= 512 workgroups with at least two tiles per share; shares must fit the row table
  while (ns < 16 && units * ns < 512 && ntiles >= 4 * ns) ns *= 2;
  while ((ntiles + ns - 1) / ns * kTileRows > kMaxShareRows) ns *= 2;
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
                              void* part, hipStream_t s, const KEvents& ev) {
  if (nq <= 0 || h <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  const int ngroups = (h + 15) / 16;
  const int ns = part ? attn_nsplit(nq, h, k) : 1;
  const int64_t units = (int64_t)nq * ngroups;
  float* part_o = reinterpret_cast<float*>(part);
  float* part_ml = part_o ? part_o + units * ns * 16 * kLatent : nullptr;
  launch(sparse_attn_kernel, dim3((unsigned)(units * ns)), dim3(kAttnThreads), s, ns > 1 ? ev.first() : ev, c, q,
         q_seq, idx, cnt, h, k, sm_scale, out, lse, ns, part_o, part_ml);
  if (ns > 1)
    launch(attn_combine_kernel, dim3((unsigned)(units * 16)), dim3(128), s, ev.last(), h, ns, part_o, part_ml, out,
           lse);
  return hipGetLastError();
}

}  // namespace csa2
