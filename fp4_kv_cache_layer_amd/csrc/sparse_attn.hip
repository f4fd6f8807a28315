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
// Work split: one workgroup per (query, group of 16 heads), four waves taking
// 32-row tiles round-robin.  Per tile a lane gathers two rows (l%16 and
// 16 + l%16), 64 code bytes each (dims 128*(l/16) .. +127) and their scales,
// dequantises with V_CVT_SCALEF32_PK_BF16_FP4 straight into the A operand of
// S^T = X Q^T (bf16 MFMA 16x16x32; the K order is permuted identically in the
// Q operand), and also writes the bf16 rows to the wave's LDS tile.  S^T puts
// head l%16 in lane l, so the probabilities are already the A operand of
// O = P X; the B operand (rows as K) comes out of LDS with the transposing
// read DS_READ_B64_TR_B16.  Online softmax across tiles; the four waves are
// merged through LDS at the end.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kAttnWaves = 4;
constexpr int kTileRows = 32;
constexpr int kLdsStride = 1040;                       // bytes per bf16 row (512 * 2 + 16 pad)
constexpr int kWaveLds = kTileRows * kLdsStride;       // 33,280 B

typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

__device__ __forceinline__ shortx4 lds_read_tr16(const uint8_t* base_generic, int byte_off) {
  const __attribute__((address_space(3))) uint8_t* p =
      (const __attribute__((address_space(3))) uint8_t*)(base_generic) + byte_off;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)p);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // round-to-nearest-even fp32 -> bf16 (finite inputs)
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

__device__ __forceinline__ bf16x2 cvt_fp4x2(uint32_t word, float scale, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3);
  }
}

__global__ void __launch_bounds__(kAttnWaves * 64, 1)
sparse_attn_kernel(CacheArgs c, const uint16_t* __restrict__ q, const int32_t* __restrict__ q_seq,
                   const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int h, int k,
                   float sm_scale, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kAttnWaves * kWaveLds];
  __shared__ float stat_m[kAttnWaves][16], stat_l[kAttnWaves][16];

  const int ngroups = (h + 15) >> 4;
  const int qi = blockIdx.x / ngroups;
  const int hg = blockIdx.x - qi * ngroups;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int n = cnt[qi];
  const int head = hg * 16 + r;

  // Q^T operand: head r, K-step s covers dims 128g + 8s .. +7.
  bf16x8 qop[16];
  {
    const bool ok = head < h;
    const uint4* src = reinterpret_cast<const uint4*>(q + ((int64_t)qi * h + (ok ? head : 0)) * kLatent + 128 * g);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      uint4 v = ok ? src[s] : make_uint4(0, 0, 0, 0);
      qop[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  floatx4 oacc[32];
#pragma unroll
  for (int nt = 0; nt < 32; ++nt) oacc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  uint8_t* my = lds + wave * kWaveLds;
  const int32_t* pt_row = c.page_table + (int64_t)q_seq[qi] * c.max_pages;
  const int32_t* irow = idx + (int64_t)qi * k;
  const int ntiles = (n + kTileRows - 1) / kTileRows;
  const int iters = (ntiles + kAttnWaves - 1) / kAttnWaves;

  for (int it = 0; it < iters; ++it) {
    const int tile = it * kAttnWaves + wave;
    // ---- gather two rows per lane and dequantise ----
    uint4 codes[2][4];
    uint32_t sbytes[2];
    bool valid[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int j = tile * kTileRows + mt * 16 + r;
      valid[mt] = j < n;
      if (valid[mt]) {
        const int t = irow[j];
        const uint8_t* src = c.kv + entry_row(pt_row, t, c.lg_page) * kKvRowBytes;
        const uint4* cs = reinterpret_cast<const uint4*>(src + 64 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) codes[mt][i] = cs[i];
        sbytes[mt] = *reinterpret_cast<const uint32_t*>(src + kCodeBytes + 4 * g);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) codes[mt][i] = make_uint4(0, 0, 0, 0);
        sbytes[mt] = 0x7F7F7F7Fu;
      }
    }
    floatx4 st[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      st[mt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      uint8_t* rowp = my + (mt * 16 + r) * kLdsStride + 256 * g;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const uint32_t wd = (s & 3) == 0 ? codes[mt][s >> 2].x
                          : (s & 3) == 1 ? codes[mt][s >> 2].y
                          : (s & 3) == 2 ? codes[mt][s >> 2].z : codes[mt][s >> 2].w;
        const float scale = e8m0_to_float((sbytes[mt] >> (8 * (s >> 2))) & 0xFFu);
        const bf16x2 p0 = cvt_fp4x2(wd, scale, 0), p1 = cvt_fp4x2(wd, scale, 1);
        const bf16x2 p2 = cvt_fp4x2(wd, scale, 2), p3 = cvt_fp4x2(wd, scale, 3);
        const bf16x8 xa = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        *reinterpret_cast<bf16x8*>(rowp + 16 * s) = xa;
        st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, qop[s], st[mt], 0, 0, 0);
      }
    }
    // ---- online softmax for head r over rows mt*16 + 4g + i ----
    float v[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = tile * kTileRows + mt * 16 + 4 * g + i;
        v[mt][i] = j < n ? st[mt][i] * sm_scale : -INFINITY;
        tmax = fmaxf(tmax, v[mt][i]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    float alpha = 1.0f;
    float psum = 0.0f;
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
    // O rows are heads 4g+i: fetch their alpha from lane 4g+i
    {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
      bool any = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) any |= al[i] != 1.0f;
      if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
        for (int nt = 0; nt < 32; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[nt][i] *= al[i];
      }
    }
    // ---- O += P X, with P split into two bf16 terms (hi + lo) ----
    bf16x8 pa_hi, pa_lo;
    {
      pa_hi = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(phi[0][0], phi[0][1]), pack_bf16x2(phi[0][2], phi[0][3]),
                                                    pack_bf16x2(phi[1][0], phi[1][1]), pack_bf16x2(phi[1][2], phi[1][3])));
      pa_lo = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(plo[0][0], plo[0][1]), pack_bf16x2(plo[0][2], plo[0][3]),
                                                    pack_bf16x2(plo[1][0], plo[1][1]), pack_bf16x2(plo[1][2], plo[1][3])));
    }
    // make this wave's LDS writes visible to its own transposing reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int off_a = (4 * g + (r >> 2)) * kLdsStride + 8 * (r & 3);
    const int off_b = off_a + 16 * kLdsStride;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) {
      const shortx4 lo = lds_read_tr16(my, off_a + 32 * nt);
      const shortx4 hi = lds_read_tr16(my, off_b + 32 * nt);
      const shortx4 x8lo = lo, x8hi = hi;
      typedef short shortx8 __attribute__((ext_vector_type(8)));
      const shortx8 b8 = {x8lo[0], x8lo[1], x8lo[2], x8lo[3], x8hi[0], x8hi[1], x8hi[2], x8hi[3]};
      const bf16x8 xb = __builtin_bit_cast(bf16x8, b8);
      oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, xb, oacc[nt], 0, 0, 0);
      oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, xb, oacc[nt], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the four waves ----
  if (g == 0) { stat_m[wave][r] = m_run; stat_l[wave][r] = l_run; }
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);          // [wave][16 heads][512] fp32 = 32 KB per wave
  {
    float f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * g + i;
      float M = -INFINITY;
#pragma unroll
      for (int w2 = 0; w2 < kAttnWaves; ++w2) M = fmaxf(M, stat_m[w2][hh]);
      f[i] = (M == -INFINITY || stat_m[wave][hh] == -INFINITY) ? 0.0f : __expf(stat_m[wave][hh] - M);
    }
#pragma unroll
    for (int nt = 0; nt < 32; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(wave * 16 + 4 * g + i) * kLatent + 16 * nt + r] = oacc[nt][i] * f[i];
  }
  __syncthreads();
  for (int e = tid; e < 16 * kLatent; e += kAttnWaves * 64) {
    const int hh = e / kLatent, d = e - hh * kLatent;
    const int hd = hg * 16 + hh;
    if (hd >= h) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < kAttnWaves; ++w2) M = fmaxf(M, stat_m[w2][hh]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < kAttnWaves; ++w2) {
      const float f = (M == -INFINITY || stat_m[w2][hh] == -INFINITY) ? 0.0f : __expf(stat_m[w2][hh] - M);
      L += f * stat_l[w2][hh];
      acc += red[(w2 * 16 + hh) * kLatent + d];
    }
    out[((int64_t)qi * h + hd) * kLatent + d] = L > 0.0f ? acc / L : 0.0f;
  }
  if (lse != nullptr && tid < 16) {
    const int hd = hg * 16 + tid;
    if (hd < h) {
      float M = -INFINITY;
      for (int w2 = 0; w2 < kAttnWaves; ++w2) M = fmaxf(M, stat_m[w2][tid]);
      float Le = 0.0f;
      for (int w2 = 0; w2 < kAttnWaves; ++w2)
        if (M != -INFINITY && stat_m[w2][tid] != -INFINITY) Le += __expf(stat_m[w2][tid] - M) * stat_l[w2][tid];
      lse[(int64_t)qi * h + hd] = (M == -INFINITY) ? -INFINITY : M + __logf(Le);
    }
  }
}

hipError_t launch_sparse_attn(const CacheArgs& c, const uint16_t* q, const int32_t* q_seq, const int32_t* idx,
                              const int32_t* cnt, int nq, int h, int k, float sm_scale, float* out, float* lse,
                              hipStream_t s) {
  const int ngroups = (h + 15) / 16;
  hipLaunchKernelGGL(sparse_attn_kernel, dim3((unsigned)((int64_t)nq * ngroups)), dim3(kAttnWaves * 64), 0, s, c, q,
                     q_seq, idx, cnt, h, k, sm_scale, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
