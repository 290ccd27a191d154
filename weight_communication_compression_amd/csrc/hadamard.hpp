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
// within each half-wave, ds_bpermute across the halves
template <int D>
__device__ __forceinline__ float xor_lane(float v) {
  // (ds_swizzle uses the LDS pipe and leaves the vector ALU to the
  // butterflies: DPP moves for partners 1 and 2 apart measured 8 % slower on
  // the stochastic compress)
  if constexpr (D <= 16) return swizzle_f32<0x1F | (D << 10)>(v);
  else return __int_as_float(__builtin_amdgcn_ds_bpermute((lane_id() ^ 32) << 2, __float_as_int(v)));
}

// One cross-lane stage (partners D lanes apart) on the N values of the lane.
template <int D, int N>
__device__ __forceinline__ void lane_butterfly(float* v) {
  const float sg = (lane_id() & D) ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float p = xor_lane<D>(v[j]);
    v[j] = __builtin_fmaf(v[j], sg, p);
  }
}

// All cross-lane stages for blocks of LANES consecutive lanes (LANES <= 64).
template <int LANES, int N>
__device__ __forceinline__ void lane_stages(float* v) {
  if constexpr (LANES > 1) lane_butterfly<1, N>(v);
  if constexpr (LANES > 2) lane_butterfly<2, N>(v);
  if constexpr (LANES > 4) lane_butterfly<4, N>(v);
  if constexpr (LANES > 8) lane_butterfly<8, N>(v);
  if constexpr (LANES > 16) lane_butterfly<16, N>(v);
  if constexpr (LANES > 32) lane_butterfly<32, N>(v);
}

// Transform blocks laid out as v[row][elem] per lane: block-local index
// k = ((row % ROWS_PER_BLOCK) * LANES + lane % LANES) * N + elem, where
// N values per lane are contiguous, LANES lanes per row of the block
// (a power of two <= 64) and the block spans ROWS_PER_BLOCK rows.  Then
// multiply by the exact power of two `scale`.
template <int ROWS, int N, int LANES, int ROWS_PER_BLOCK>
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
  for (int r = 0; r < ROWS; ++r) lane_stages<LANES, N>(v[r]);
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
