// Device-side helpers shared by the CSA2 kernels (gfx950 only).
//
// Number formats follow the choices stated in include/csa2.h: main-KV rows
// are E2M1 codes with one E8M0 scale per 32 values, indexer rows are OCP
// E4M3FN.  The E2M1 format for the main KV is named on the aiany.app
// "DeepSeek-V4.1-Flash" page, "What Sets It Apart".
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

constexpr int kLatent = 512;
constexpr int kIndexDim = 128;
constexpr int kKvRowBytes = 272;
constexpr int kCodeBytes = 256;

// ---------------------------------------------------------------------------
// E8M0 block exponent: the smallest integer e with amax <= 6 * 2^e, read off
// the fp32 bit pattern of amax.  For amax = 1.f * 2^E (normal), 6 * 2^e >=
// amax holds first at e = E - 2 when 1.f <= 1.5 and at e = E - 1 otherwise;
// amax below 2^-126 (or zero) needs e < -127 and is clamped there.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int block_exponent(float amax) {
  uint32_t u = __float_as_uint(amax);
  int ef = (int)((u >> 23) & 0xFF);
  if (ef == 0) return -127;
  int e = ef - 127 - 2 + ((u & 0x7FFFFF) > 0x400000 ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E2M1 code of r = x / 2^e (|r| <= 6 by construction): round to the nearest of
// {0, .5, 1, 1.5, 2, 3, 4, 6}; at a midpoint the code with a 0 low bit wins,
// so 0.25, 1.25, 2.5 and 5 round down and 0.75, 1.75 and 3.5 round up.  The
// magnitude code is the number of decision points at or below |r|.
__device__ __forceinline__ uint32_t e2m1_code(float r) {
  float a = fabsf(r);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
               (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return c | ((__float_as_uint(r) >> 28) & 0x8u);
}

// OCP E4M3FN byte of an fp32 value: round to nearest even, saturate to 448,
// sign bit copied (so -0 and small negatives give 0x80).
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fabsf(x);
  uint32_t c;
  if (a >= 448.0f) {
    c = 0x7E;
  } else if (a < 0.015625f) {                  // below 2^-6: multiples of 2^-9
    c = (uint32_t)__builtin_rintf(a * 512.0f); // exact product; rint is ties-to-even
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);           // round the 23-bit mantissa to 3 bits
    c = (u >> 20) - (120u << 3);                // rebias 127 -> 7, keep 3 mantissa bits
    if (c > 0x7E) c = 0x7E;
  }
  return c | sign;
}

// Quantize-on-append of one row by one wavefront (lane = 0..63): the bf16
// latent row kv_rows[row] -> 256 E2M1 code bytes and 16 E8M0 scale bytes,
// the bf16 indexer row idxk_rows[row] -> 128 E4M3FN bytes, both written at
// physical slot slots[row].  Lane l owns latent elements 8l..8l+7 (one
// 16-byte load), so a 32-element scale block is 4 adjacent lanes and its
// amax is two lane swaps away; the same lane owns indexer elements 2l, 2l+1.
__device__ __forceinline__ void append_row(uint8_t* __restrict__ kv, uint8_t* __restrict__ idx_k,
                                           const int32_t* __restrict__ slots,
                                           const uint16_t* __restrict__ kv_rows,
                                           const uint16_t* __restrict__ idxk_rows, int row, int lane) {
  const int64_t slot = slots[row];
  // ---- main-KV row ----
  const uint4 raw = *reinterpret_cast<const uint4*>(kv_rows + (int64_t)row * kLatent + 8 * lane);
  float x[8];
  const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(wds[i] << 16);
    x[2 * i + 1] = __uint_as_float(wds[i] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int e = block_exponent(amax);
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) packed |= e2m1_code(ldexpf(x[i], -e)) << (4 * i);
  uint8_t* dst = kv + slot * kKvRowBytes;
  *reinterpret_cast<uint32_t*>(dst + 4 * lane) = packed;
  if ((lane & 3) == 0) dst[kCodeBytes + (lane >> 2)] = (uint8_t)(e + 127);
  // ---- indexer-K row ----
  const uint32_t iw = *reinterpret_cast<const uint32_t*>(idxk_rows + (int64_t)row * kIndexDim + 2 * lane);
  const uint32_t c0 = e4m3_code(__uint_as_float(iw << 16));
  const uint32_t c1 = e4m3_code(__uint_as_float(iw & 0xFFFF0000u));
  *reinterpret_cast<uint16_t*>(idx_k + slot * kIndexDim + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
}

// fp32 score -> unsigned key whose order is the float order; -0 counts as +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One lane's 32-byte MFMA operand (V_MFMA_*_F8F6F4, K = 128) from a 128-byte
// FP8 row: lanes 16g .. 16g+15 take bytes [16g, +16) and [64 + 16g, +16).
// This is a fixed permutation of K applied to both operands alike, so the
// product is unchanged; each 16-lane load then covers one contiguous half of
// every row it touches.  All indexer paths use it, so their scores agree bit
// for bit.
__device__ __forceinline__ intx8 load_fp8_operand(const uint8_t* row, int g) {
  const intx4 lo = *reinterpret_cast<const intx4*>(row + 16 * g);
  const intx4 hi = *reinterpret_cast<const intx4*>(row + 64 + 16 * g);
  return intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// A 16-row x 128-byte FP8 tile in contiguous memory reaches its MFMA
// operand layout through LDS: lane l loads bytes [32l, +32) (four lanes per
// 128-byte row, so loads are fully coalesced), writes them to the wave's LDS
// slot (rows padded to kFp8SlotRow bytes, conflict-free both ways) and reads
// back the load_fp8_operand layout of row l % 16.
constexpr int kFp8SlotRow = 144;
constexpr int kFp8SlotBytes = 16 * kFp8SlotRow;

__device__ __forceinline__ intx8 load_fp8_tile_linear(const uint8_t* tile, int lane) {
  const intx4 lo = *reinterpret_cast<const intx4*>(tile + 32 * lane);
  const intx4 hi = *reinterpret_cast<const intx4*>(tile + 32 * lane + 16);
  return intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ intx8 fp8_tile_operand(uint8_t* slot, const intx8& lin, int lane) {
  uint8_t* wr = slot + (lane >> 2) * kFp8SlotRow + 32 * (lane & 3);
  *reinterpret_cast<intx4*>(wr) = intx4{lin[0], lin[1], lin[2], lin[3]};
  *reinterpret_cast<intx4*>(wr + 16) = intx4{lin[4], lin[5], lin[6], lin[7]};
  return load_fp8_operand(slot + (lane & 15) * kFp8SlotRow, lane >> 4);
}

// max(x, 0) as one integer max on the bit pattern: negative values (sign bit
// set, -0 included) map to +0; used by every indexer path so their scores
// agree bit for bit.
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// This lane's share sum_i w_i * max(0, acc_i) over its 4 MFMA output rows.
__device__ __forceinline__ float relu_weighted(const floatx4& acc, const float (&wv)[4]) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += wv[i] * relu_bits(acc[i]);
  return s;
}
__device__ __forceinline__ float relu_weighted4(const floatx4& acc, const float4 wv) {
  const float w4[4] = {wv.x, wv.y, wv.z, wv.w};
  return relu_weighted(acc, w4);
}

// E8M0 byte -> fp32 scale 2^(b-127); byte 0 is the subnormal 2^-127.
__device__ __forceinline__ float e8m0_to_float(uint32_t b) {
  return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// Reductions across the four 16-lane rows of a wave with the gfx950 lane
// swaps (plain VALU, no LDS round trip).  V_PERMLANE16_SWAP exchanges odd
// rows of one operand with even rows of the other, V_PERMLANE32_SWAP the
// upper half of one with the lower half of the other; with both operands
// equal to x, the two results hold x and its partner row (half) in every
// lane, in one order or the other, so a symmetric op of the two is the
// pairwise reduction.
__device__ __forceinline__ float rows_pair_max(float x) {        // over lanes l, l ^ 16
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_max(float x) {           // over lanes l, l ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inclusive prefix sum over the wave: DPP row shifts within each 16-lane row,
// then the totals of the rows below (read from lanes 15, 31, 47).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
  const uint32_t r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
                 r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Workgroup barrier that orders LDS only.  A plain __syncthreads() also
// waits for every global load in flight, which would drain prefetched data
// at each barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Physical row of logical entry t of a sequence: page table lookup.
__device__ __forceinline__ int64_t entry_row(const int32_t* __restrict__ pt_row, int t, int lg_ps) {
  int page = pt_row[t >> lg_ps];
  return ((int64_t)page << lg_ps) + (t & ((1 << lg_ps) - 1));
}

}  // namespace csa2
