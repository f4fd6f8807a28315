// Merge of the global (CSA2) attention branch with the local sliding-window
// branch: one softmax over the union of the two branches' keys, from each
// branch's output O and natural-log LSE.  With M = max(lse_a, lse_b),
//   w_a = e^(lse_a - M), w_b = e^(lse_b - M),
//   O = (w_a O_a + w_b O_b) / (w_a + w_b),  LSE = M + ln(w_a + w_b);
// a branch with no keys (LSE = -inf) counts for nothing, and both empty give
// O = 0, LSE = -inf.
//
// The global branch sits beside local sliding-window attention ("DeepSeek-
// V4.1-Flash: Pushing the Limits of KV Cache Compression", the global
// attention branch over the full context together with local sliding-window
// attention; the research-podcast summary, global context decoupled from
// local sliding-window attention); the pages give no combination formula, the
// one above is the reading stated in csa2.h.
//
// Streaming and HBM-bound: each thread owns float4 pieces of the outputs,
// reads the two rows' LSEs (shared by the row's threads through the caches)
// and the two float4 inputs, and writes one float4; grid-stride over the
// whole [rows][dim] array, so every load is a coalesced 16-byte access.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kMergeThreads = 256;
constexpr int kMergeMaxBlocks = 16384;

__global__ void __launch_bounds__(kMergeThreads)
lse_merge_kernel(const float4* __restrict__ oa, const float* __restrict__ la, const float4* __restrict__ ob,
                 const float* __restrict__ lb, int64_t n4, int d4, float4* o, float* __restrict__ lse) {
  const int64_t stride = (int64_t)gridDim.x * kMergeThreads;
  for (int64_t e = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x; e < n4; e += stride) {
    const int64_t row = e / d4;
    const float a = la[row], b = lb[row];
    const float m = fmaxf(a, b);
    float wa = 0.0f, wb = 0.0f, inv = 0.0f;
    if (m != -INFINITY) {
      wa = a == -INFINITY ? 0.0f : __expf(a - m);
      wb = b == -INFINITY ? 0.0f : __expf(b - m);
      inv = 1.0f / (wa + wb);                       // wa + wb >= 1: the larger side weighs 1
    }
    const float4 x = oa[e], y = ob[e];
    o[e] = make_float4((wa * x.x + wb * y.x) * inv, (wa * x.y + wb * y.y) * inv, (wa * x.z + wb * y.z) * inv,
                       (wa * x.w + wb * y.w) * inv);
    if (lse != nullptr && e - row * d4 == 0) lse[row] = m == -INFINITY ? -INFINITY : m + __logf(wa + wb);
  }
}

hipError_t launch_lse_merge(const float* oa, const float* la, const float* ob, const float* lb, int rows, int dim,
                            float* o, float* lse, hipStream_t s, const KEvents& ev) {
  const int d4 = dim / 4;
  const int64_t n4 = (int64_t)rows * d4;
  if (n4 <= 0) {
    record_empty(ev, s);
    return hipSuccess;
  }
  const int64_t blocks = std::min<int64_t>((n4 + kMergeThreads - 1) / kMergeThreads, kMergeMaxBlocks);
  launch(lse_merge_kernel, dim3((unsigned)blocks), dim3(kMergeThreads), s, ev, reinterpret_cast<const float4*>(oa),
         la, reinterpret_cast<const float4*>(ob), lb, n4, d4, reinterpret_cast<float4*>(o), lse);
  return hipGetLastError();
}

}  // namespace csa2
