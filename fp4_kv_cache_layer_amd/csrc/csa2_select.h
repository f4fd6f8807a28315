// Device helpers shared by the indexer scan and the Top-K select (gfx950).
// Include after csa2_device.h and csa2_internal.h.
#pragma once

namespace csa2 {

// Canonical score of one 16-entry tile for the query whose indexer heads are
// the A operand a (head weights wv of this lane's four output rows), from the
// tile's B operand b (lane (g, r): entry r's bytes in the load_fp8_operand
// layout of group g): every lane returns the score of entry lane % 16 (a zero
// score as +0).  The scan, the select's repair and the pruning threshold all
// score through it, so an entry scored anywhere has exactly the scan's bits.
__device__ __forceinline__ float operand_score(const intx8& a, const float (&wv)[4], const intx8& b) {
  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
  const float part = halves_sum(rows_pair_sum(relu_weighted(acc, wv)));
  uint32_t u32 = __float_as_uint(part);
  if ((u32 << 1) == 0) u32 = 0;                       // -0 -> +0
  return __uint_as_float(u32);
}

// The same from the tile's 128-byte rows loaded linearly (lin), which reach
// the operand layout through the wave's LDS slot.
__device__ __forceinline__ float tile_score(const intx8& a, const float (&wv)[4], uint8_t* slot, const intx8& lin,
                                            int lane) {
  return operand_score(a, wv, fp8_tile_operand(slot, lin, lane));
}

// Candidates a 2,048-entry chunk keeps: its top L entries (and the ties of
// the L-th key's 22-bit prefix), L = 4 x the chunk's expected share of the
// query's Top-k, at least 16.  A chunk with more of the Top-k than that is
// caught and rescored by the final select.
__device__ __forceinline__ int scan_local_rank(int k, int vis) {
  const int64_t share = ((int64_t)k * kScanChunk + vis - 1) / vis;
  return (int)min<int64_t>(kScanChunk, max<int64_t>(16, 4 * share));
}

// Search over a descending-ordered histogram h[0..nb) (nb <= 2048): the
// largest digit d* whose suffix count reaches need (1 <= need <= total), and
// the count strictly above it, written to result[0..1].  One wave does the
// search; the workgroup barrier at the end publishes the result.  Callers
// have h complete (a barrier) first.
__device__ inline void find_digit(const uint32_t* h, int nb, uint32_t need, uint32_t* result) {
  if ((threadIdx.x >> 6) == 0) {
    const int lane = threadIdx.x & 63;
    if (nb == kHistBins) {
      // Lane l sums the digits [base, base + 32), base = nb - 32 (l + 1)
      // (descending positions 32l .. 32l+31), reading its eight 16-byte
      // pieces in a lane-rotated order so the wave's reads spread over the
      // banks; a wave scan finds the lane L whose range holds d*.  Then lanes
      // 0..31 take one digit each of L's range, descending, and a second scan
      // finds d* itself.
      const int base = nb - 32 * (lane + 1);
      uint32_t mine = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint4 w = *reinterpret_cast<const uint4*>(h + base + 4 * ((j + lane) & 7));
        mine += (w.x + w.y) + (w.z + w.w);
      }
      const uint32_t x = wave_incl_sum(mine);
      const uint64_t hm = __builtin_amdgcn_ballot_w64(x - mine < need && need <= x);
      const int L = __builtin_ctzll(hm);
      const uint32_t run0 = __builtin_amdgcn_readlane(x - mine, L);
      const int dig = nb - 1 - 32 * L - lane;                 // lanes 0..31: L's digits, descending
      const uint32_t hv = h[lane < 32 ? dig : 0];
      const uint32_t c = lane < 32 ? hv : 0u;
      const uint32_t y = wave_incl_sum(c) + run0;
      const uint64_t dm = __builtin_amdgcn_ballot_w64(lane < 32 && need <= y && y - c < need);
      const int L2 = __builtin_ctzll(dm);
      const uint32_t above = __builtin_amdgcn_readlane(y - c, L2);
      if (lane == 0) {
        result[0] = (uint32_t)(nb - 1 - 32 * L - L2);
        result[1] = above;
      }
    } else {
      const int per = (nb + 63) >> 6;
      const int p0 = min(nb, lane * per), p1 = min(nb, p0 + per);
      uint32_t mine = 0;
      for (int p = p0; p < p1; ++p) mine += h[nb - 1 - p];
      const uint32_t x = wave_incl_sum(mine);
      const uint32_t excl = x - mine;
      if (excl < need && need <= x) {
        uint32_t run = excl;
        for (int p = p0; p < p1; ++p) {
          const uint32_t c = h[nb - 1 - p];
          if (need <= run + c) { result[0] = (uint32_t)(nb - 1 - p); result[1] = run; break; }
          run += c;
        }
      }
    }
  }
  lds_barrier();
}

}  // namespace csa2
