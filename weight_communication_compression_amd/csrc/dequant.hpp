// dequant.hpp -- decompress kernels: codes + scales -> binary32, the
// weight-difference apply w_out = to_dtype(w_old + deq), and the decompress
// with inverse Hadamard smoothing.
//
// Element-centric layout: a "row" is 64 * EPL consecutive elements and lane l
// of a wave decodes elements EPL*l .. EPL*l + EPL-1 of it (EPL = 4 for the
// decompress, 8 for the apply), so every binary32 or bfloat16 store of the
// wave is one fully coalesced access at any bitwidth.  The codes of a lane are
// consecutive bits of one packed word (two for 8 codes of 8 bits; lanes
// sharing a word read the same address, served by the cache), and blocks are
// at least 32 elements, so each lane needs one scale.
#pragma once

#include "args.hpp"
#include "device.hpp"
#include "hadamard.hpp"

namespace lowbit {

// rows per lane per loop trip, and elements per lane per row (decompress:
// 4, a 16-byte binary32 store; apply: 8, a 16-byte bfloat16 load and store).
// Decompress rows: measured on the 64 Mi bucket inside the whole-path step
// (codes written by the compress just before), 2 rows per wave take the four
// decompresses from 201 to 184 us against 8 rows (4 rows: 200 us, 1 row:
// slower); with the Infinity Cache flushed first, 2 rows is 12 % faster at
// 8 bits and 5 % slower at 1 and 2 bits.
constexpr int kDeqRows = 2;
constexpr int kApplyRows = 2;
constexpr int kDeqEpl = 4;
constexpr int kApplyEpl = 8;
template <int BITS, int APPLY>
constexpr int dequant_rows() { return APPLY ? kApplyRows : kDeqRows; }
template <int APPLY>
constexpr int dequant_epl() { return APPLY ? kApplyEpl : kDeqEpl; }
constexpr int kDeqRow = kWave * 4;              // elements per row at 4 per lane

// Decode the N codes in bits [off, off + N*b) of `word` with scale s
// (N * b <= 32).
template <int BITS, int N>
__device__ __forceinline__ void decode_n(uint32_t word, int off, float s, float* d) {
  using G = Grid<BITS>;
  const uint32_t piece = word >> off;
  if constexpr (BITS == 1) {
#pragma unroll
    for (int j = 0; j < N; ++j) d[j] = signed_scale(piece, j, s);
  } else {
    const uint32_t tw = piece ^ G::FLIP;        // fields become two's-complement q
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int q = (int)(tw << (32 - BITS * (j + 1))) >> (32 - BITS);
      d[j] = (float)q * s;                      // exact
    }
  }
}

template <int BITS>
__device__ __forceinline__ void decode4(uint32_t word, int off, float s, float* d) {
  decode_n<BITS, 4>(word, off, s, d);
}

// One trip of the decompress / apply: rows base .. base + rows - 1.  GUARD:
// the trip may reach past n (the last one only); the others load and store
// unguarded.
template <int BITS, int APPLY, int DT, bool GUARD>
__device__ __forceinline__ void dequant_trip(const DequantArgs& a, int64_t base) {
  constexpr int E = Grid<BITS>::E;              // codes per word
  constexpr int kDequantRows = dequant_rows<BITS, APPLY>();
  constexpr int EPL = dequant_epl<APPLY>();
  constexpr int ROW = kWave * EPL;
  constexpr int NW = EPL * BITS > 32 ? EPL * BITS / 32 : 1;   // words per lane
  constexpr int LOG2ROW = EPL == 8 ? 9 : 8;
  const int lane = lane_id();
  const int64_t n = a.n;
  uint32_t word[kDequantRows][NW];
  uint32_t s16[kDequantRows];
  float wo[kDequantRows][EPL];
  const uint32_t lo = (uint32_t)EPL * (uint32_t)lane;       // lane's element within a row
#pragma unroll
  for (int r = 0; r < kDequantRows; ++r) {
    const int64_t r0 = (base + r) * ROW;                    // row start (wave-uniform)
#pragma unroll
    for (int k = 0; k < NW; ++k) word[r][k] = 0;
    s16[r] = 0;
    if (!GUARD || r0 + lo < n) {
      const uint32_t* cw = a.codes + r0 / E;
      // word k holds elements lo + k*E ..: a tail lane of several words
      // reads only those that hold an element below n
#pragma unroll
      for (int k = 0; k < NW; ++k)
        if (!GUARD || k == 0 || r0 + lo + (uint32_t)(k * E) < n) word[r][k] = cw[lo / E + k];
      // blocks of >= ROW elements cover the whole row: one scale per row
      s16[r] = a.log2b >= LOG2ROW ? a.scales[r0 >> a.log2b]
                                  : (a.scales + (r0 >> a.log2b))[lo >> a.log2b];
      if constexpr (APPLY) {
        if (!GUARD || r0 + lo + EPL <= n) load_vec<DT, EPL>(a.w_old, r0, lo, wo[r]);
        else load_tail<DT, EPL>(a.w_old, r0, lo, n - r0, wo[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kDequantRows; ++r) {
    const int64_t r0 = (base + r) * ROW;
    if (GUARD && r0 + lo >= n) continue;
    float d[EPL];
    const float s = f16_bits_to_f32(s16[r]);
    if constexpr (NW == 1) {
      decode_n<BITS, EPL>(word[r][0], (int)(lo % E) * BITS, s, d);
    } else {
#pragma unroll
      for (int k = 0; k < NW; ++k) decode_n<BITS, E>(word[r][k], 0, s, d + k * E);
    }
    const bool full = !GUARD || r0 + lo + EPL <= n;
    if constexpr (!APPLY) {
      if (full) store_vec_f32<EPL>(a.y, r0, lo, d);
      else store_tail_f32<EPL>(a.y, r0, lo, n - r0, d);
    } else {
      float w[EPL];
#pragma unroll
      for (int j = 0; j < EPL; ++j) w[j] = wo[r][j] + d[j];
      if constexpr (DT == kF32) {
        if (full) store_vec_f32<EPL>(static_cast<float*>(a.w_out), r0, lo, w);
        else store_tail_f32<EPL>(static_cast<float*>(a.w_out), r0, lo, n - r0, w);
      } else {
        const int64_t e0 = r0 + lo;
        uint16_t* out = static_cast<uint16_t*>(a.w_out) + r0 + lo;
        if (full) {
          uint32_t pk[EPL / 2];
#pragma unroll
          for (int k = 0; k < EPL / 2; ++k)
            pk[k] = f32_to_bf16_rne(w[2 * k]) | (f32_to_bf16_rne(w[2 * k + 1]) << 16);
          store_stream_words<EPL / 2>(reinterpret_cast<uint32_t*>(out), pk);
        } else {
#pragma unroll
          for (int j = 0; j < EPL; ++j)
            if (e0 + j < n) out[j] = (uint16_t)f32_to_bf16_rne(w[j]);
        }
      }
    }
  }
}

// APPLY: 0 = decompress to binary32; 1 = weight-difference apply.  Element-
// centric: a row is 64 * EPL consecutive elements, lane l decodes elements
// EPL*l .. EPL*l + EPL - 1 (their codes are EPL*b consecutive bits of one
// word, or two words for 8 codes of 8 bits); blocks are >= 32 elements, so
// each lane needs one scale.
// Workgroup size of the decompress / apply of BITS-bit codes.  2-bit
// decompress of the 64 Mi bucket: 256 threads take it from 52.8 to 50.1 us
// with the Infinity Cache flushed first and from 47.7 to 50.3 us inside the
// whole-path step; 128 threads elsewhere (256 costs 1-4 us in the step at the
// other widths).  Rows per trip for 2 bits: 4 and 8 were slower both ways.
template <int BITS, int APPLY>
constexpr int deq_threads() { return BITS == 2 && !APPLY ? 256 : kDeqThreads; }

template <int BITS, int APPLY, int DT>
__global__ __launch_bounds__((deq_threads<BITS, APPLY>())) void dequant_kernel(DequantArgs a) {
  constexpr int THREADS = deq_threads<BITS, APPLY>();
  constexpr int kDequantRows = dequant_rows<BITS, APPLY>();
  constexpr int ROW = kWave * dequant_epl<APPLY>();
  static_assert(ROW == 256 || ROW == 512, "rows of 256 or 512 elements");
  const int64_t wave = global_wave_id<THREADS>();
  const int64_t nwaves = (int64_t)gridDim.x * (THREADS / kWave);
  const int64_t nrows = (a.n + ROW - 1) / ROW;
  const int64_t ntrips = (nrows + kDequantRows - 1) / kDequantRows;
  for_each_trip(wave, ntrips, nwaves, [&](int64_t t) __attribute__((always_inline)) {
    const int64_t base = t * kDequantRows;
    // wave-uniform: every trip but the last lies inside the buffer
    if ((base + kDequantRows) * ROW <= a.n) dequant_trip<BITS, APPLY, DT, false>(a, base);
    else dequant_trip<BITS, APPLY, DT, true>(a, base);
  });
}

// Decompress followed by the inverse blockwise Walsh-Hadamard transform
// (blocks of B = 2^LOG2B elements).  Same element-centric layout (rows of
// 256, 4 elements per lane); a trip of max(8, B/256) rows
// holds whole blocks, so the transform runs in registers: elements within
// the lane, then lanes, then rows.  Loads and stores are guarded, the
// transform is not (every lane of the wave takes part in the exchanges;
// lanes past the end hold values that are not stored).  Rows per trip,
// measured on the 64 Mi bucket at 4 bits, B = 128, with the exchanges on
// ds_swizzle: 1 row 83 us, 2: 65, 4: 63, 8: 60.6, 16: 75 (more rows keep more
// exchanges in flight per wave until the register footprint costs
// occupancy); with DPP / permlane exchanges (flushed caches): 8 rows 56.9,
// 4 rows 54.8 us.
constexpr int kHsDeqRows = 4;
constexpr bool kHsDeqDpp = true;      // cross-lane partners by DPP moves where possible
// workgroup size: 256 threads 53.8 us against 55.2 (128) and 55.0 (64)
constexpr int kHsDeqThreads = 256;
template <int LOG2B>
constexpr int hadamard_rows_per_trip() {
  return (1 << LOG2B) > kHsDeqRows * kDeqRow ? (1 << LOG2B) / kDeqRow : kHsDeqRows;
}

// Code words and scales of one trip (rows base .. base + rows - 1).  GUARD:
// the trip may reach past n (the last one only).
template <int BITS, int LOG2B, bool GUARD>
__device__ __forceinline__ void hadamard_dequant_load(const DequantArgs& a, int64_t base,
                                                      uint32_t* word, uint32_t* s16) {
  constexpr int E = Grid<BITS>::E;
  constexpr int kHadamardRows = hadamard_rows_per_trip<LOG2B>();
  const uint32_t lo = 4u * (uint32_t)lane_id();
#pragma unroll
  for (int r = 0; r < kHadamardRows; ++r) {
    const int64_t r0 = (base + r) * kDeqRow;
    word[r] = 0;
    s16[r] = 0;
    if (!GUARD || r0 + lo < a.n) {
      word[r] = (a.codes + r0 / E)[lo / E];
      s16[r] = LOG2B >= 8 ? a.scales[r0 >> LOG2B] : (a.scales + (r0 >> LOG2B))[lo >> LOG2B];
    }
  }
}

// Decode, inverse-transform and store one loaded trip.
template <int BITS, int LOG2B, bool GUARD>
__device__ __forceinline__ void hadamard_dequant_finish(const DequantArgs& a, int64_t base,
                                                        const uint32_t* word,
                                                        const uint32_t* s16) {
  constexpr int E = Grid<BITS>::E;
  constexpr int B = 1 << LOG2B;
  constexpr int kHadamardRows = hadamard_rows_per_trip<LOG2B>();
  constexpr int LANES = B >= kDeqRow ? kWave : B / 4;
  constexpr int ROWS_PER_BLOCK = B >= kDeqRow ? B / kDeqRow : 1;
  const int64_t n = a.n;
  const int64_t nfull = n & ~(int64_t)(B - 1);   // elements in whole blocks
  const uint32_t lo = 4u * (uint32_t)lane_id();
  float d[kHadamardRows][4];
#pragma unroll
  for (int r = 0; r < kHadamardRows; ++r)
    decode4<BITS>(word[r], (int)(lo % E) * BITS, f16_bits_to_f32(s16[r]), d[r]);
  hadamard_rows<kHadamardRows, 4, LANES, ROWS_PER_BLOCK, kHsDeqDpp>(d,
                                                                    hadamard_inverse_scale<LOG2B>());
  // a partial last block is decompressed untransformed: its lanes decode
  // their values again (only a trip that reaches past the whole blocks)
  if ((base + kHadamardRows) * kDeqRow > nfull) {
#pragma unroll
    for (int r = 0; r < kHadamardRows; ++r) {
      const int64_t i = (base + r) * kDeqRow + lo;
      if (i >= nfull)
        decode4<BITS>(word[r], (int)(lo % E) * BITS, f16_bits_to_f32(s16[r]), d[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < kHadamardRows; ++r) {
    const int64_t r0 = (base + r) * kDeqRow;
    if (!GUARD || r0 + lo + 4 <= n) store_vec_f32<4>(a.y, r0, lo, d[r]);
    else if (r0 + lo < n) store_tail_f32<4>(a.y, r0, lo, n - r0, d[r]);
  }
}

template <int BITS, int LOG2B>
__global__ __launch_bounds__(kHsDeqThreads) void hadamard_dequant_kernel(DequantArgs a) {
  constexpr int B = 1 << LOG2B;
  constexpr int R = hadamard_rows_per_trip<LOG2B>();
  static_assert(B <= R * kDeqRow, "a block must fit in one trip");
  const int64_t wave = global_wave_id<kHsDeqThreads>();
  const int64_t nwaves = (int64_t)gridDim.x * (kHsDeqThreads / kWave);
  const int64_t nrows = (a.n + kDeqRow - 1) / kDeqRow;
  const int64_t ntrips = (nrows + R - 1) / R;
  for_each_trip(wave, ntrips, nwaves, [&](int64_t t) __attribute__((always_inline)) {
    uint32_t word[R], s16[R];
    // wave-uniform: every trip but the last lies inside the buffer
    if ((t + 1) * R * kDeqRow <= a.n) {
      hadamard_dequant_load<BITS, LOG2B, false>(a, t * R, word, s16);
      hadamard_dequant_finish<BITS, LOG2B, false>(a, t * R, word, s16);
    } else {
      hadamard_dequant_load<BITS, LOG2B, true>(a, t * R, word, s16);
      hadamard_dequant_finish<BITS, LOG2B, true>(a, t * R, word, s16);
    }
  });
}

// Decompress with the inverse transform for blocks of 4096 elements: one
// workgroup of kHsBigWaves waves per block, each wave 4 rows of 256 (16
// values per lane).  A wave transforms its 1024 elements in registers
// (strides 1 .. 512: in the lane, across lanes, across its rows), then the
// strides 1024 and 2048 pair the waves w and w ^ 1, then w and w ^ 2, through
// LDS: every lane writes its 16 values, the workgroup synchronizes, and each
// lane reads the values at the same position of the partner wave and keeps
// fma(own, +-1, partner) as the lane exchanges do; then the scale, then the
// stores.  The same binary32 operations in the same stage order as the
// one-wave trip, which at this block size holds 64 values per lane (252
// VGPRs, two waves per SIMD).  Whole blocks only: the caller decompresses a
// partial last block with hadamard_dequant_kernel.  `nblocks` whole blocks;
// a workgroup takes block blockIdx.x and, where the grid was capped, every
// gridDim.x-th one after it (the whole workgroup alike, so that all its waves
// reach each barrier).
constexpr int kHsBigWaves = 4;
template <int BITS>
__device__ __forceinline__ void hadamard_dequant_big_block(const DequantArgs& a, int64_t blk);
template <int BITS>
__global__ __launch_bounds__(kHsBigWaves * kWave) void hadamard_dequant_big_kernel(DequantArgs a,
                                                                                  int64_t nblocks) {
  for (int64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x)   // workgroup-uniform
    hadamard_dequant_big_block<BITS>(a, blk);
}
template <int BITS>
__device__ __forceinline__ void hadamard_dequant_big_block(const DequantArgs& a, int64_t blk) {
  constexpr int E = Grid<BITS>::E;
  constexpr int RW = 4;                                   // rows per wave
  constexpr int LOG2B = 12;
  static_assert(kHsBigWaves * RW * kDeqRow == (1 << LOG2B), "one block per workgroup");
  __shared__ float xch[kHsBigWaves][RW * 4][kWave];
  const int wv = (int)(threadIdx.x >> 6);
  const int lane = lane_id();
  const uint32_t lo = 4u * (uint32_t)lane;
  const int64_t row0 = blk * (kHsBigWaves * RW) + wv * RW;   // the wave's first row
  uint32_t word[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) word[r] = (a.codes + (row0 + r) * kDeqRow / E)[lo / E];
  const float s = f16_bits_to_f32(a.scales[blk]);
  float d[RW][4];
#pragma unroll
  for (int r = 0; r < RW; ++r) decode4<BITS>(word[r], (int)(lo % E) * BITS, s, d[r]);
  hadamard_rows<RW, 4, kWave, RW, kHsDeqDpp>(d, 1.0f);   // strides 1 .. 512 (x 1: exact)
#pragma unroll
  for (int m = 1; m < kHsBigWaves; m <<= 1) {             // strides 1024, 2048
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) xch[wv][r * 4 + j][lane] = d[r][j];
    __syncthreads();
    const float sg = (wv & m) ? -1.0f : 1.0f;
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) d[r][j] = __builtin_fmaf(d[r][j], sg, xch[wv ^ m][r * 4 + j][lane]);
    __syncthreads();
  }
  constexpr float scale = hadamard_inverse_scale<LOG2B>();
#pragma unroll
  for (int r = 0; r < RW; ++r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) d[r][j] = d[r][j] * scale;
    store_vec_f32<4>(a.y, (row0 + r) * kDeqRow, lo, d[r]);
  }
}

// Plain binary32 copy with the codec kernels' launch shape (measurement aid):
// one float4 per thread and trip.
__global__ __launch_bounds__(kBlockThreads) void copy_kernel(const float* x, float* y, int64_t n) {
  const int64_t nvec = n / 4;
  const int64_t stride = (int64_t)gridDim.x * kBlockThreads;
  const float4* xv = reinterpret_cast<const float4*>(x);
  float4* yv = reinterpret_cast<float4*>(y);
  for (int64_t i = logical_block() * kBlockThreads + threadIdx.x; i < nvec; i += stride)
    yv[i] = xv[i];
  const int64_t t = nvec * 4 + (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  if (t < n) y[t] = x[t];
}

// Measurement aid with the error-feedback compress's memory pattern and none
// of its arithmetic: y[i] = fl(y[i] + x[i]) in place for binary32 x and y, each
// wave taking one row of 256 consecutive elements (4 per lane: one 16-byte
// load of each stream, one 16-byte streaming store of y), the same trip as
// the 4-bit EF compress's row layout without its code and scale writes.
__global__ __launch_bounds__(kBlockThreads) void add_inplace_kernel(const float* x, float* y,
                                                                    int64_t n) {
  constexpr int E = 4, CHUNK = kWave * E;
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const uint32_t off = (uint32_t)lane_id() * E;
  for (int64_t t0 = global_wave_id() * CHUNK; t0 < n; t0 += nwaves * CHUNK) {   // wave-uniform
    float a[E], b[E];
    if (t0 + CHUNK <= n) {
      load_vec<kF32, E>(x, t0, off, a);
      load_vec<kF32, E>(y, t0, off, b);
#pragma unroll
      for (int j = 0; j < E; ++j) b[j] = b[j] + a[j];
      store_vec_f32<E>(y, t0, off, b);
    } else {
      load_tail<kF32, E>(x, t0, off, n - t0, a);
      load_tail<kF32, E>(y, t0, off, n - t0, b);
#pragma unroll
      for (int j = 0; j < E; ++j) b[j] = b[j] + a[j];
      store_tail_f32<E>(y, t0, off, n - t0, b);
    }
  }
}

// Measurement aid with the compress kernels' memory volume and none of their
// arithmetic: reads n binary32 values and writes ceil(n*BITS/32) words.  A
// wave takes 2048 consecutive values (8 rows of 256, one 16-byte load per lane
// per row, as the 1-bit compress reads) and lane l writes BITS consecutive
// words at word (wave*64 + l)*BITS, word k the XOR of the bit patterns of its
// values 4r + j in [k*32/BITS, (k+1)*32/BITS) (r the row, j the position in
// the lane's four); values past n read as 0 and words past the end are not
// written.
template <int BITS>
__global__ __launch_bounds__(kBlockThreads) void fold_kernel(const float* x, int64_t n,
                                                             uint32_t* out, int64_t nwords) {
  constexpr int ROWS = 8, ROW = kWave * 4, TILE = ROWS * ROW, PER = 32 / BITS;
  const int64_t ntiles = (n + TILE - 1) / TILE;
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const int lane = lane_id();
  for (int64_t tile = global_wave_id(); tile < ntiles; tile += nwaves) {
    const int64_t t0 = tile * TILE;
    uint32_t v[ROWS * 4];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const uint32_t off = (uint32_t)(r * ROW + lane * 4);
      float f[4];
      if (t0 + TILE <= n) load_vec<kF32, 4>(x, t0, off, f);
      else load_tail<kF32, 4>(x, t0, off, n - t0, f);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * r + j] = __float_as_uint(f[j]);
    }
    uint32_t w[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) {
      w[k] = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) w[k] ^= v[k * PER + i];
    }
    const int64_t o = (tile * kWave + lane) * BITS;
    if (o + BITS <= nwords) {
      if constexpr (BITS == 1) store_stream(out + o, w[0]);
      else if constexpr (BITS == 2) store_stream_words<2>(out + o, w);
      else if constexpr (BITS == 4) store_stream_words<4>(out + o, w);
      else {
        store_stream_words<4>(out + o, w);
        store_stream_words<4>(out + o + 4, w + 4);
      }
    } else {
#pragma unroll
      for (int k = 0; k < BITS; ++k)
        if (o + k < nwords) out[o + k] = w[k];
    }
  }
}

}  // namespace lowbit
