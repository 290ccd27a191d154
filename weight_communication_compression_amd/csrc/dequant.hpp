// dequant.hpp -- decompress kernels: codes + scales -> binary32, and the
// weight-difference apply w_out = to_dtype(w_old + deq).  Lane l decodes word
// r*64 + l of a tile of R rows; a word never straddles a block (B >= 32 >= E),
// so each word needs one scale.
#pragma once

#include "args.hpp"
#include "device.hpp"

namespace lowbit {

constexpr int kDequantRows = 2;   // words per lane per loop trip

template <int BITS>
__device__ __forceinline__ void decode_word(uint32_t word, float s, float* d) {
  using G = Grid<BITS>;
  constexpr int E = G::E;
  if constexpr (BITS == 1) {
#pragma unroll
    for (int j = 0; j < E; ++j) d[j] = ((word >> j) & 1u) ? s : -s;
  } else {
    const uint32_t tw = word ^ G::FLIP;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int q = (int)(tw << (32 - BITS * (j + 1))) >> (32 - BITS);
      d[j] = (float)q * s;            // exact
    }
  }
}

// APPLY: 0 = decompress to binary32; 1 = weight-difference apply.
template <int BITS, int APPLY, int DT>
__global__ __launch_bounds__(kBlockThreads) void dequant_kernel(DequantArgs a) {
  constexpr int E = Grid<BITS>::E;
  constexpr int TILE_W = kWave * kDequantRows;             // words per tile
  const int lane = lane_id();
  const int64_t wave = (int64_t)blockIdx.x * (kBlockThreads / kWave) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const int64_t n = a.n;
  const int64_t nwords = (n + E - 1) / E;
  const int64_t ntiles = (nwords + TILE_W - 1) / TILE_W;

  for (int64_t tile = wave; tile < ntiles; tile += nwaves) {
    const int64_t wt0 = tile * TILE_W;
    const bool full = (wt0 + TILE_W) * E <= n;
    uint32_t word[kDequantRows];
    uint32_t s16[kDequantRows];
#pragma unroll
    for (int r = 0; r < kDequantRows; ++r) {
      const int64_t w = wt0 + r * kWave + lane;
      word[r] = 0;
      s16[r] = 0;
      if (full || w < nwords) {
        word[r] = a.codes[w];
        s16[r] = a.scales[(w * E) >> a.log2b];
      }
    }
    float wo[kDequantRows][E];
    if constexpr (APPLY) {
#pragma unroll
      for (int r = 0; r < kDequantRows; ++r) {
        const int64_t i0 = (wt0 + r * kWave + lane) * E;
        if (full) load_vec<DT, E>(a.w_old, i0, wo[r]);
        else load_tail<DT, E>(a.w_old, i0, n, wo[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kDequantRows; ++r) {
      const int64_t i0 = (wt0 + r * kWave + lane) * E;
      float d[E];
      decode_word<BITS>(word[r], f16_bits_to_f32(s16[r]), d);
      if constexpr (!APPLY) {
        if (full) store_vec_f32<E>(a.y, i0, d);
        else store_tail_f32<E>(a.y, i0, n, d);
      } else {
        float w[E];
#pragma unroll
        for (int j = 0; j < E; ++j) w[j] = wo[r][j] + d[j];
        if constexpr (DT == kF32) {
          if (full) store_vec_f32<E>(static_cast<float*>(a.w_out), i0, w);
          else store_tail_f32<E>(static_cast<float*>(a.w_out), i0, n, w);
        } else {
          uint16_t* out = static_cast<uint16_t*>(a.w_out) + i0;
          if (full) {
            uint32_t pk[E / 2];
#pragma unroll
            for (int k = 0; k < E / 2; ++k)
              pk[k] = f32_to_bf16_rne(w[2 * k]) | (f32_to_bf16_rne(w[2 * k + 1]) << 16);
            if constexpr (E == 4) {
              *reinterpret_cast<uint2*>(out) = make_uint2(pk[0], pk[1]);
            } else {
#pragma unroll
              for (int k = 0; k < E / 8; ++k)
                reinterpret_cast<uint4*>(out)[k] =
                    make_uint4(pk[4 * k], pk[4 * k + 1], pk[4 * k + 2], pk[4 * k + 3]);
            }
          } else {
#pragma unroll
            for (int j = 0; j < E; ++j)
              if (i0 + j < n) out[j] = (uint16_t)f32_to_bf16_rne(w[j]);
          }
        }
      }
    }
  }
}

// Plain binary32 copy with the codec kernels' launch shape (measurement aid).
__global__ __launch_bounds__(kBlockThreads) void copy_kernel(const float* x, float* y, int64_t n) {
  const int64_t nvec = n / 4;
  const int64_t stride = (int64_t)gridDim.x * kBlockThreads;
  const float4* xv = reinterpret_cast<const float4*>(x);
  float4* yv = reinterpret_cast<float4*>(y);
  int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  for (; i + stride < nvec; i += 2 * stride) {
    float4 a = xv[i];
    float4 b = xv[i + stride];
    yv[i] = a;
    yv[i + stride] = b;
  }
  if (i < nvec) yv[i] = xv[i];
  const int64_t t = nvec * 4 + (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  if (t < n) y[t] = x[t];
}

}  // namespace lowbit
