// Quantize-on-append: bf16 latent rows -> 272-byte E2M1/E8M0 rows, bf16
// indexer rows -> 128-byte E4M3FN rows, written at caller-given slots.
//
// The FP4 global KV and an inference system that serves the format come from
// "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression", Method;
// the E2M1 format from the aiany.app "DeepSeek-V4.1-Flash" page, "What Sets
// It Apart".  Block size, scale rule and byte layout are stated in csa2.h.
//
// One wavefront per row.  Lane l owns latent elements 8l..8l+7 (one 16-byte
// load), so a 32-element scale block is 4 adjacent lanes and its amax is two
// lane swaps away.  The same lane owns indexer elements 2l, 2l+1.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

__global__ void __launch_bounds__(256)
append_quant_kernel(uint8_t* __restrict__ kv, uint8_t* __restrict__ idx_k,
                    const int32_t* __restrict__ slots,
                    const uint16_t* __restrict__ kv_rows, const uint16_t* __restrict__ idxk_rows, int n) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  append_row(kv, idx_k, slots, kv_rows, idxk_rows, row, threadIdx.x & 63);
}

hipError_t launch_append_quant(uint8_t* kv, uint8_t* idx_k, const int32_t* slots, const uint16_t* kv_rows,
                               const uint16_t* idxk_rows, int n, hipStream_t s, const KEvents& ev) {
  const int blocks = (n + 3) / 4;
  if (blocks <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  launch(append_quant_kernel, dim3(blocks), dim3(256), s, ev, kv, idx_k, slots, kv_rows, idxk_rows, n);
  return hipGetLastError();
}

// Fill kernel used to clear workspaces without a memset node.
__global__ void fill_zero_kernel(uint4* __restrict__ p, size_t n16, uint8_t* __restrict__ tail, int ntail) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const int ntail = (int)(bytes - n16 * 16);
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<uint4*>(p), n16, reinterpret_cast<uint8_t*>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace csa2
