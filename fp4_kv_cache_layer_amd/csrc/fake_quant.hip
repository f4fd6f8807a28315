// FP4 fake quantisation for quantization-aware training: every 32-element
// block of x is encoded exactly as quantize-on-append encodes a main-KV row
// (E8M0 scale 2^e, the smallest with amax <= 6 * 2^e; E2M1 codes of x / 2^e,
// round to nearest, ties to the even code, sign kept) and decoded back,
// y = E2M1(code) * 2^e, in the input's own dtype (the decoded values are
// exact in fp32 and bf16).  The straight-through gradient is the identity:
// the scale rule never clips.
//
// FP4 is used for the global KV during training, by quantization-aware
// training ("DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
// Compression"); the block rules are the main-KV ones stated in csa2.h.
//
// Streaming and HBM-bound: the lanes of one block read consecutive 16-byte
// pieces (8 lanes x 4 fp32, or 4 lanes x 8 bf16), take the block max with
// lane swaps, and write their pieces back; grid-stride over the array.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kFqThreads = 256;
constexpr int kFqMaxBlocks = 16384;

// E2M1 magnitude of a 3-bit code: 0, .5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_magnitude(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  return e == 0 ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * (float)(1u << (e - 1));
}

// Quantise-dequantise of one value given its block's scale and inverse scale.
__device__ __forceinline__ float fake_e2m1(float x, float scale, float inv) {
  const uint32_t code = e2m1_code(x * inv);                  // x / 2^e, exact
  const float mag = e2m1_magnitude(code) * scale;            // exact
  return __uint_as_float(__float_as_uint(mag) | ((code & 8u) << 28));
}

// Block scale 2^e and 2^-e from the lanes' local maxima (LANES lanes per block).
template <int LANES>
__device__ __forceinline__ void block_scale(float amax, float& scale, float& inv) {
#pragma unroll
  for (int o = 1; o < LANES; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const int e = block_exponent(amax);                       // [-127, 127]
  scale = e8m0_to_float((uint32_t)(e + 127));
  inv = e8m0_to_float((uint32_t)(127 - e));
}

__global__ void __launch_bounds__(kFqThreads)
fake_quant_f32_kernel(const float4* x, float4* y, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * kFqThreads;     // a multiple of 8: blocks stay in one wave
  for (int64_t g = (int64_t)blockIdx.x * kFqThreads + threadIdx.x; g < n4; g += stride) {
    const float4 v = x[g];
    float scale, inv;
    block_scale<8>(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))), scale, inv);
    y[g] = make_float4(fake_e2m1(v.x, scale, inv), fake_e2m1(v.y, scale, inv), fake_e2m1(v.z, scale, inv),
                       fake_e2m1(v.w, scale, inv));
  }
}

__global__ void __launch_bounds__(kFqThreads)
fake_quant_bf16_kernel(const uint4* x, uint4* y, int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * kFqThreads;     // a multiple of 4
  for (int64_t g = (int64_t)blockIdx.x * kFqThreads + threadIdx.x; g < n8; g += stride) {
    const uint4 v = x[g];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    float scale, inv;
    block_scale<4>(amax, scale, inv);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {                              // decoded values are exact in bf16
      const uint32_t lo = __float_as_uint(fake_e2m1(f[2 * i], scale, inv)) >> 16;
      const uint32_t hi = __float_as_uint(fake_e2m1(f[2 * i + 1], scale, inv)) & 0xFFFF0000u;
      o[i] = lo | hi;
    }
    y[g] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_fake_quant(const void* x, void* y, int64_t n, bool bf16, hipStream_t s, const KEvents& ev) {
  const int64_t groups = bf16 ? n / 8 : n / 4;
  if (groups <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  const int64_t blocks = std::min<int64_t>((groups + kFqThreads - 1) / kFqThreads, kFqMaxBlocks);
  if (bf16)
    launch(fake_quant_bf16_kernel, dim3((unsigned)blocks), dim3(kFqThreads), s, ev, reinterpret_cast<const uint4*>(x),
           reinterpret_cast<uint4*>(y), groups);
  else
    launch(fake_quant_f32_kernel, dim3((unsigned)blocks), dim3(kFqThreads), s, ev,
           reinterpret_cast<const float4*>(x), reinterpret_cast<float4*>(y), groups);
  return hipGetLastError();
}

}  // namespace csa2
