// hadamard.hpp -- blockwise Walsh-Hadamard smoothing in registers.
//
// Each quantization block of B elements is transformed by the Sylvester-
// ordered Walsh-Hadamard matrix, as butterflies (a, b) -> (a + b, a - b) of
// stride 1, 2, ..., B/2 in that order (the same binary32 operations in the
// same order as the definition, so the result is bit-identical to it).  The
// stride picks which bit of the element's index within the block pairs the
// two operands; with the data spread over the wave, low index bits are the
// element within the lane, then the lane, then the row.  A cross-lane stage
// reads the partner lane's value (ds_swizzle up to 16 lanes apart,
// ds_bpermute for 32) and each lane computes fma(own, +-1, partner):
// the product is exact, so this is fl(own + partner) in the lower lane and
// fl(partner - own) in the upper one.  All lanes of the wave must be active.
#pragma once

#include "device.hpp"

namespace lowbit {

// v[lane ^ D], D = 1 .. 32: ds_swizzle in bit-mask mode (and 0x1F, xor D)
// within each half-wave, ds_bpermute across the halves.  DPP: partners 1, 2
// and 8 apart by DPP moves instead (quad_perm, and row_ror:8, which within a
// row of 16 lanes is lane ^ 8), and 16 apart by v_permlane16_swap (in
// lane_butterfly): vector-ALU moves in place of LDS-pipe swizzles, which pays
// where the vector ALU has room (the 4-bit B128 decompress of 64 Mi
// elements: 58.2 -> 54.8 us) and not where it is the bound (the stochastic
// compress: 8 % slower).  Partners 4 apart stay on ds_swizzle (two DPP row
// shifts under bank masks measured 1 us slower).
template <int D, bool DPP>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (DPP && D == 1) return dpp_f32<0xB1>(v);        // quad_perm [1,0,3,2]
  else if constexpr (DPP && D == 2) return dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  else if constexpr (DPP && D == 8) return dpp_f32<0x128>(v);  // row_ror:8
  else if constexpr (D <= 16) return swizzle_f32<0x1F | (D << 10)>(v);
  else return __int_as_float(__builtin_amdgcn_ds_bpermute((lane_id() ^ 32) << 2, __float_as_int(v)));
}

// One cross-lane stage (partners D lanes apart) on the N values of the lane.
template <int D, int N, bool DPP>
__device__ __forceinline__ void lane_butterfly(float* v) {
  const float sg = (lane_id() & D) ? -1.0f : 1.0f;
  if constexpr (DPP && D == 16) {
    // v_permlane16_swap of the value with itself: every lane receives the
    // lower row's value (a) and the upper row's (b) of its pair of rows;
    // a + b in the lower row, a - b in the upper one, as fma(b, +-1, a)
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const auto ab = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j]),
                                                       __float_as_uint(v[j]), false, false);
      v[j] = __builtin_fmaf(__uint_as_float(ab[1]), sg, __uint_as_float(ab[0]));
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float p = xor_lane<D, DPP>(v[j]);
      v[j] = __builtin_fmaf(v[j], sg, p);
    }
  }
}

// All cross-lane stages for blocks of LANES consecutive lanes (LANES <= 64).
template <int LANES, int N, bool DPP>
__device__ __forceinline__ void lane_stages(float* v) {
  if constexpr (LANES > 1) lane_butterfly<1, N, DPP>(v);
  if constexpr (LANES > 2) lane_butterfly<2, N, DPP>(v);
  if constexpr (LANES > 4) lane_butterfly<4, N, DPP>(v);
  if constexpr (LANES > 8) lane_butterfly<8, N, DPP>(v);
  if constexpr (LANES > 16) lane_butterfly<16, N, DPP>(v);
  if constexpr (LANES > 32) lane_butterfly<32, N, DPP>(v);
}

// Transform blocks laid out as v[row][elem] per lane: block-local index
// k = ((row % ROWS_PER_BLOCK) * LANES + lane % LANES) * N + elem, where
// N values per lane are contiguous, LANES lanes per row of the block
// (a power of two <= 64) and the block spans ROWS_PER_BLOCK rows.  Then
// multiply by the exact power of two `scale`.
template <int ROWS, int N, int LANES, int ROWS_PER_BLOCK, bool DPP = false>
__device__ __forceinline__ void hadamard_rows(float (&v)[ROWS][N], float scale) {
  // strides 1 .. N/2: within the lane
#pragma unroll
  for (int h = 1; h < N; h <<= 1)
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
      for (int j = 0; j < N; ++j)
        if ((j & h) == 0) {
          const float a = v[r][j], b = v[r][j + h];
          v[r][j] = a + b;
          v[r][j + h] = a - b;
        }
  // strides N .. N*LANES/2: across lanes
#pragma unroll
  for (int r = 0; r < ROWS; ++r) lane_stages<LANES, N, DPP>(v[r]);
  // larger strides: across the rows of the block
#pragma unroll
  for (int m = 1; m < ROWS_PER_BLOCK; m <<= 1)
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
      if ((r & m) == 0)
#pragma unroll
        for (int j = 0; j < N; ++j) {
          const float a = v[r][j], b = v[r + m][j];
          v[r][j] = a + b;
          v[r + m][j] = a - b;
        }
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int j = 0; j < N; ++j) v[r][j] = v[r][j] * scale;
}

// 2^-floor(L/2) (forward) and 2^-ceil(L/2) (inverse) for B = 2^L
template <int LOG2B>
constexpr float hadamard_forward_scale() { return 1.0f / (float)(1 << (LOG2B / 2)); }
template <int LOG2B>
constexpr float hadamard_inverse_scale() { return 1.0f / (float)(1 << ((LOG2B + 1) / 2)); }

}  // namespace lowbit
