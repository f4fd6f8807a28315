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
// Work split.  A workgroup serves one query and one group of 16 heads.  It
// first resolves the physical row of every selected entry into LDS (one round
// of index and page-table loads for the whole selection), then its eight
// waves, two row groups x four 128-wide slices of the latent, stream 32-row
// tiles with the row gathers of the next kPrefetch tiles in flight.  For every
// tile a wave
//   - gathers, for two rows per lane, the 16 code bytes of one 32-element
//     scale block of its slice and dequantises them with
//     V_CVT_SCALEF32_PK_BF16_FP4 straight into the A operand of
//     S^T = X Q^T (bf16 MFMA 16x16x32, K = its 128 dims, permuted alike in
//     the Q operand),
//   - publishes its partial S^T (32 rows x 16 heads) and its bf16 slice of the
//     rows in LDS (row stride 272 B: the 16-byte writes and the transposing
//     8-byte reads both spread evenly over the 64 banks),
//   - sums the four partial S^T of its row group (same order in every wave),
//     runs the online softmax and accumulates O[16 heads][its 128 dims] +=
//     P X with P split into bf16 hi + lo terms; the B operand (rows as K)
//     comes from LDS through the transposing read DS_READ_B64_TR_B16.
// So each latent element is dequantised once per head group, the O
// accumulator is 32 registers per lane, and the only cross-wave traffic per
// tile is 2 KB of partial scores per wave.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kAttnThreads = 512;
constexpr int kTileRows = 32;
constexpr int kSliceStride = 272;                       // bytes per bf16 slice row (128 * 2 + 16 pad)
constexpr int kSliceBytes = kTileRows * kSliceStride;   // 8,704

typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

__device__ __forceinline__ shortx4 lds_read_tr16(const uint8_t* base_generic, int byte_off) {
  const __attribute__((address_space(3))) uint8_t* p =
      (const __attribute__((address_space(3))) uint8_t*)(base_generic) + byte_off;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)p);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  a += 0x7FFFu + ((a >> 16) & 1u);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (a >> 16) | (b & 0xFFFF0000u);
}

__device__ __forceinline__ float bf16_round(float x) {
  uint32_t a = __float_as_uint(x);
  a += 0x7FFFu + ((a >> 16) & 1u);
  return __uint_as_float(a & 0xFFFF0000u);
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

constexpr int kPrefetch = 4;                            // tiles of row gathers in flight per wave

struct AttnShared {
  uint8_t xs[2][4][kSliceBytes];     // [row group][slice] bf16 rows of the current tile (69,632 B)
  floatx4 sp[2][4][2][4][16];        // partial S^T per wave: [m-tile][row quad][head] of 4 rows (16,384 B)
  int64_t rowoff[2048];              // byte offset of every selected row (16,384 B)
  float st_m[4][16];                 // row-group merge scratch
  float st_l[4][16];
};

__global__ void __launch_bounds__(kAttnThreads, 1)
sparse_attn_kernel(CacheArgs c, const uint16_t* __restrict__ q, const int32_t* __restrict__ q_seq,
                   const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int h, int k,
                   float sm_scale, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ AttnShared S;
  const int ngroups = (h + 15) >> 4;
  const int qi = blockIdx.x / ngroups;
  const int hg = blockIdx.x - qi * ngroups;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ds = wave & 3, rg = wave >> 2;
  const int g = lane >> 4, r = lane & 15;
  const int n = cnt[qi];
  const int head = hg * 16 + r;

  // Q^T operand: head r, K-step s holds dims 128*ds + 32*g + 8*s .. +7.
  bf16x8 qop[4];
  {
    const bool ok = head < h;
    const uint4* src = reinterpret_cast<const uint4*>(q + ((int64_t)qi * h + (ok ? head : 0)) * kLatent + 128 * ds + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) qop[s] = __builtin_bit_cast(bf16x8, ok ? src[s] : make_uint4(0, 0, 0, 0));
  }

  floatx4 oacc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) oacc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  // physical rows of the whole selection, resolved once
  {
    const int32_t* pt_row = c.page_table + (int64_t)q_seq[qi] * c.max_pages;
    const int32_t* irow = idx + (int64_t)qi * k;
    for (int j = tid; j < n; j += kAttnThreads) S.rowoff[j] = entry_row(pt_row, irow[j], c.lg_page) * kKvRowBytes;
  }
  lds_barrier();
  const int ntiles = (n + kTileRows - 1) / kTileRows;
  const int iters = (ntiles + 1) >> 1;

  uint8_t* xs = &S.xs[rg][ds][0];

  // ring of row gathers: slot u holds iteration it + u's 16 code bytes (one
  // scale block of this slice) and scale byte, for two rows per lane
  uint4 cd[kPrefetch][2];
  uint32_t sb[kPrefetch][2];
  // Loads are unconditional (a row past the selection reads row 0 of page 0,
  // which always exists) so the compiler can count gathers in flight; the
  // data of such rows is replaced by zeros at use.
  auto gather = [&](int iter, uint4 (&c2)[2], uint32_t (&s2)[2]) {
    const int tile = 2 * iter + rg;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int j = tile * kTileRows + mt * 16 + r;
      const uint8_t* src = c.kv + ((iter < iters && j < n) ? S.rowoff[j] : 0);
      c2[mt] = *reinterpret_cast<const uint4*>(src + 64 * ds + 16 * g);
      s2[mt] = src[kCodeBytes + 4 * ds + g];
    }
  };
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) gather(u, cd[u], sb[u]);

  // The trip count is padded to whole rings (tiles past the selection are
  // masked), so every ring slot is consumed in a fixed order and the compiler
  // can keep the younger gathers in flight.
  const int iters_pad = (iters + kPrefetch - 1) / kPrefetch * kPrefetch;
  for (int it0 = 0; it0 < iters_pad; it0 += kPrefetch) {
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) {
    const int it = it0 + u;
    const int tile = 2 * it + rg;
    // ---- dequantise into the S^T A operand; partial S^T over this slice ----
    bf16x8 xa[2][4];
    floatx4 st[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const bool ok = tile * kTileRows + mt * 16 + r < n;
      const float scale = e8m0_to_float(ok ? sb[u][mt] : 127u);
      const uint32_t wds[4] = {ok ? cd[u][mt].x : 0u, ok ? cd[u][mt].y : 0u, ok ? cd[u][mt].z : 0u, ok ? cd[u][mt].w : 0u};
      st[mt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        xa[mt][s] = dequant8(wds[s], scale);
        st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mt][s], qop[s], st[mt], 0, 0, 0);
      }
    }
    gather(it + kPrefetch, cd[u], sb[u]);               // refill the slot kPrefetch tiles ahead
    // ---- publish the bf16 slice rows and the partial scores ----
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      uint8_t* rowp = xs + (mt * 16 + r) * kSliceStride + 64 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s) *reinterpret_cast<bf16x8*>(rowp + 16 * s) = xa[mt][s];
      S.sp[rg][ds][mt][g][r] = st[mt];                  // lanes write consecutive 16 B: no bank conflicts
    }
    lds_barrier();
    // ---- full scores of head r, rows mt*16 + 4g + i (fixed summation order) ----
    float v[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      floatx4 acc = S.sp[rg][0][mt][g][r];
#pragma unroll
      for (int d2 = 1; d2 < 4; ++d2) acc += S.sp[rg][d2][mt][g][r];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = tile * kTileRows + mt * 16 + 4 * g + i;
        v[mt][i] = j < n ? acc[i] * sm_scale : -INFINITY;
        tmax = fmaxf(tmax, v[mt][i]);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    float alpha = 1.0f, psum = 0.0f;
    float phi[2][4], plo[2][4];                         // p = phi + plo, both bf16
    if (m_new == -INFINITY) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) phi[mt][i] = plo[mt][i] = 0.0f;
    } else {
      alpha = __expf(m_run - m_new);                    // m_run = -inf -> 0
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __expf(v[mt][i] - m_new);     // -inf -> 0
          psum += p;
          phi[mt][i] = bf16_round(p);
          plo[mt][i] = bf16_round(p - phi[mt][i]);
        }
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    {
      // O rows are heads 4g+i: their rescale factor lives in lane 4g+i
      float al[4];
      bool any = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        al[i] = __shfl(alpha, 4 * g + i);
        any |= al[i] != 1.0f;
      }
      if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[nt][i] *= al[i];
      }
    }
    const bf16x8 pa_hi = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(phi[0][0], phi[0][1]), pack_bf16x2(phi[0][2], phi[0][3]),
                                                               pack_bf16x2(phi[1][0], phi[1][1]), pack_bf16x2(phi[1][2], phi[1][3])));
    const bf16x8 pa_lo = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(plo[0][0], plo[0][1]), pack_bf16x2(plo[0][2], plo[0][3]),
                                                               pack_bf16x2(plo[1][0], plo[1][1]), pack_bf16x2(plo[1][2], plo[1][3])));
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

  // ---- merge the two row groups (row group 1 hands its state to row group 0) ----
  float* red = reinterpret_cast<float*>(&S.xs[0][0][0]);   // [slice][16 heads][128] fp32 = 32 KB
  if (rg == 1) {
    if (g == 0) { S.st_m[ds][r] = m_run; S.st_l[ds][r] = l_run; }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(ds * 16 + 4 * g + i) * 128 + 16 * nt + r] = oacc[nt][i];
  }
  lds_barrier();
  if (rg == 0) {
    const float m1 = S.st_m[ds][r], l1 = S.st_l[ds][r];
    const float M = fmaxf(m_run, m1);
    const float f0 = (M == -INFINITY || m_run == -INFINITY) ? 0.0f : __expf(m_run - M);
    const float f1 = (M == -INFINITY || m1 == -INFINITY) ? 0.0f : __expf(m1 - M);
    const float L = f0 * l_run + f1 * l1;
    float a0[4], a1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { a0[i] = __shfl(f0, 4 * g + i); a1[i] = __shfl(f1, 4 * g + i); }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        oacc[nt][i] = a0[i] * oacc[nt][i] + a1[i] * red[(ds * 16 + 4 * g + i) * 128 + 16 * nt + r];
    m_run = M;
    l_run = L;
  }
  if (rg == 0) {
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
  }
}

hipError_t launch_sparse_attn(const CacheArgs& c, const uint16_t* q, const int32_t* q_seq, const int32_t* idx,
                              const int32_t* cnt, int nq, int h, int k, float sm_scale, float* out, float* lse,
                              hipStream_t s) {
  const int ngroups = (h + 15) / 16;
  hipLaunchKernelGGL(sparse_attn_kernel, dim3((unsigned)((int64_t)nq * ngroups)), dim3(kAttnThreads), 0, s, c, q,
                     q_seq, idx, cnt, h, k, sm_scale, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
