// device.hpp -- gfx950 device helpers shared by the codec kernels.
//
// Wave64 only (CDNA4).  Cross-lane reductions use DPP row operations and
// ds_swizzle, never LDS round trips.  Every floating-point step that decides
// a code is a single IEEE binary32 operation: the library is compiled with
// -ffp-contract=off, fp32 denormals preserved, and correctly rounded division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

constexpr int kWave = 64;
constexpr int kBlockThreads = 256;   // threads per workgroup
// the decompress kernels' workgroup size (stores dominate; smaller groups
// start and retire in finer steps)
constexpr int kDeqThreads = 128;
constexpr int kXcds = 8;             // MI355X: 8 XCDs of 32 CUs, one L2 each
constexpr float kMagic = 12582912.0f;           // 1.5 * 2^23
constexpr uint32_t kMagicBits = 0x4B400000u;    // bit pattern of kMagic

// compress modes: plain; error feedback (a = g + e, e <- a - deq); weight
// difference (w_new - w_old); EF21 (d = g - h, h <- h + deq); Hadamard
// smoothing (blockwise Walsh-Hadamard transform, then plain compress)
enum Mode : int { kPlain = 0, kErrorFeedback = 1, kWeightDiff = 2, kEF21 = 3, kHadamard = 4 };
enum DType : int { kF32 = 0, kBF16 = 1 };

template <int BITS>
struct Grid {
  static constexpr int E = 32 / BITS;                               // codes per word
  static constexpr int QMAX = BITS == 1 ? 1 : (1 << (BITS - 1)) - 1;
  static constexpr uint32_t HALF = BITS == 1 ? 0u : (1u << (BITS - 1));
  // the offset bit of every field: xor with it turns offset codes into
  // two's-complement fields
  static constexpr uint32_t FLIP = [] {
    uint32_t f = 0;
    for (int j = 0; j < E; ++j) f |= HALF << (j * BITS);
    return f;
  }();
  // packing constant: word = PACK_BIAS + sum_j bits(q_j + kMagic) << (j*BITS)
  // equals sum_j (q_j + HALF) << (j*BITS) modulo 2^32, because
  // bits(q + kMagic) = kMagicBits + q for |q| < 2^22.
  static constexpr uint32_t PACK_BIAS = [] {
    uint32_t c = 0;
    for (int j = 0; j < E; ++j) c += (HALF - kMagicBits) << (j * BITS);
    return c;
  }();
};

// Per-lane elements a wave loads per loop trip: nearest rounding is light on
// ALU and prefers short trips; stochastic rounding of 8-bit codes (four
// elements per lane and tile) hides its hashing better with more tiles' loads
// in flight.  Measured on the 64 Mi bucket, each compress alone: 8 bits, 16
// elements 61.6 us, 8 elements 65.8 us; 4 bits, 16 elements 55.6 us, 8
// elements 52.8 us (inside the whole-path step 52.0 and 50.1 us).
constexpr int kElemsPerTrip = 8;
constexpr int kSrElemsPerTrip = 16;

// Tiles per loop trip for a kernel whose tile gives each lane PER_LANE
// elements: enough tiles for kElemsPerTrip elements, or with stochastic
// rounding for kSrElemsPerTrip when a tile gives a lane fewer than 8.
template <int PER_LANE, bool SR = false>
constexpr int tiles_per_trip() {
  constexpr int want = SR && PER_LANE < 8 ? kSrElemsPerTrip : kElemsPerTrip;
  return PER_LANE >= want ? 1 : want / PER_LANE;
}

// ---------------------------------------------------------------- lanes --
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Workgroups are dealt to the XCDs round-robin (hardware workgroup b runs on
// XCD b mod 8), and each XCD has its own L2.  Where neighbouring workgroups
// share cache lines (the binary16 scales of several tiles), runs of CHUNK
// consecutive logical workgroups can be given to one XCD: within each whole
// group of 8 * CHUNK workgroups, workgroup b takes logical workgroup
// (b mod 8) * CHUNK + (b / 8) mod CHUNK.  A group is still one contiguous
// stretch of memory, so HBM keeps seeing a single stream; a trailing partial
// group keeps the identity mapping.  The map is a bijection on
// [0, gridDim.x).  CHUNK = 1: the hardware order.
template <int CHUNK = 1>
__device__ __forceinline__ int64_t logical_block() {
  const int64_t b = blockIdx.x;
  if constexpr (CHUNK <= 1) {
    return b;
  } else {
    constexpr int64_t G = (int64_t)kXcds * CHUNK;
    const int64_t whole = ((int64_t)gridDim.x / G) * G;
    if (b >= whole) return b;
    const int64_t r = b % G;
    return b - r + (r % kXcds) * CHUNK + r / kXcds;
  }
}

// A pointer to device memory that is the same in every lane, held in scalar
// registers (as a global-memory pointer, so that loads through it stay
// global loads).
template <typename T>
using global_ptr = const __attribute__((address_space(1))) T*;
template <typename T>
__device__ __forceinline__ global_ptr<T> uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (global_ptr<T>)(((uint64_t)hi << 32) | lo);
}

// Index of this wave in the grid, as a wave-uniform (scalar) value: element
// offsets then split into a scalar base and a 32-bit per-lane offset, and
// loads and stores use the scalar-base addressing mode.  THREADS: the
// kernel's workgroup size; CHUNK: see logical_block.
template <int THREADS = kBlockThreads, int CHUNK = 1>
__device__ __forceinline__ int64_t global_wave_id() {
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  return logical_block<CHUNK>() * (THREADS / kWave) + w;
}

// body(i) for i = first, first + stride, ... below count.  The grid gives
// every wave one trip unless it was capped (more than 2^32 work-items), so
// the first call is kept out of the loop: its addresses are then offsets from
// kernel arguments rather than values carried from iteration to iteration in
// 64-bit vector registers.
template <typename F>
__device__ __forceinline__ void for_each_trip(int64_t first, int64_t count, int64_t stride,
                                              F&& body) {
  if (first < count) body(first);
  for (int64_t i = first + stride; i < count; i += stride) body(i);
}

// DPP moves with every row and bank enabled; every control used here gives
// each lane a source lane inside its row, so no lane keeps an old value and
// none is supplied (mov_dpp: no move of a zero first).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

template <int PATTERN>
__device__ __forceinline__ float swizzle_f32(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), PATTERN));
}

__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Reduce over aligned groups of L consecutive lanes (L a power of two <= 64);
// every lane of a group ends with the group's result.  For the sum, the
// combination order is the adjacent-pairs tree over the lanes: partners
// 1, 2, 4, ... apart (quad_perm for 1 and 2; after those steps half_mirror
// and row_mirror pair lanes with the neighbouring aligned group of 4 and 8;
// swizzle xor 16; the two wave halves last).  Addition is commutative, so
// which side of a pair a lane sees first does not change the bits.
template <int L, bool SUM>
__device__ __forceinline__ float group_reduce(float v) {
  auto op = [](float a, float b) { return SUM ? a + b : fmaxf(a, b); };
  if constexpr (L >= 2) v = op(v, dpp_f32<0xB1>(v));     // quad_perm [1,0,3,2]
  if constexpr (L >= 4) v = op(v, dpp_f32<0x4E>(v));     // quad_perm [2,3,0,1]
  if constexpr (L >= 8) v = op(v, dpp_f32<0x141>(v));    // row_half_mirror
  if constexpr (L >= 16) v = op(v, dpp_f32<0x140>(v));   // row_mirror
  if constexpr (L >= 32) v = op(v, swizzle_f32<0x401F>(v));  // lane ^ 16 within 32
  if constexpr (L >= 64) v = op(readlane_f32(v, 0), readlane_f32(v, 32));
  return v;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// Maximum over aligned groups of L lanes of a non-negative binary32 value,
// taken on the bit patterns: for non-negative floats the unsigned integer
// order is the numeric order, and v_max_u32 folds the DPP move into itself.
template <int L>
__device__ __forceinline__ float group_max_nonneg(float x) {
  uint32_t v = __float_as_uint(x);
  if constexpr (L >= 2) v = max(v, dpp_u32<0xB1>(v));
  if constexpr (L >= 4) v = max(v, dpp_u32<0x4E>(v));
  if constexpr (L >= 8) v = max(v, dpp_u32<0x141>(v));
  if constexpr (L >= 16) v = max(v, dpp_u32<0x140>(v));
  if constexpr (L >= 32)
    v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
  if constexpr (L >= 64)
    v = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
            (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
  return __uint_as_float(v);
}

// 1-bit codes of N <= 32 values: bit j = 1 iff v[j] >= 0 (so -0 gives 1).
// fl(v + 0) turns -0 into +0, so its sign bit is set exactly for v < 0;
// v_alignbit shifts the word left by one and inserts that sign bit, two
// instructions per value and no compare/select.  (A NaN codes by its sign.)
template <int N>
__device__ __forceinline__ uint32_t sign_codes(const float* v) {
  uint32_t w = 0;
#pragma unroll
  for (int j = N - 1; j >= 0; --j)
    w = __builtin_amdgcn_alignbit(w, __float_as_uint(v[j] + 0.0f), 31);
  return ~w & (N == 32 ? 0xFFFFFFFFu : ((1u << N) - 1u));
}

// The 1-bit dequantized value u ? s : -s for bit j of `word`, as a sign flip.
__device__ __forceinline__ float signed_scale(uint32_t word, int j, float s) {
  return __uint_as_float(__float_as_uint(s) ^ (((~word) << (31 - j)) & 0x80000000u));
}

// Adjacent-pairs tree sum of |v[0..N)| within one lane (N a power of two).
template <int N>
__device__ __forceinline__ float lane_abs_tree(const float* v) {
  float t[N];
#pragma unroll
  for (int j = 0; j < N; ++j) t[j] = fabsf(v[j]);
#pragma unroll
  for (int w = N; w > 1; w >>= 1) {
#pragma unroll
    for (int j = 0; j < w / 2; ++j) t[j] = t[2 * j] + t[2 * j + 1];
  }
  return t[0];
}

// Adjacent-pairs tree over N values held in registers.
template <int N>
__device__ __forceinline__ float reg_tree(const float* g) {
  float t[N];
#pragma unroll
  for (int j = 0; j < N; ++j) t[j] = g[j];
#pragma unroll
  for (int w = N; w > 1; w >>= 1) {
#pragma unroll
    for (int j = 0; j < w / 2; ++j) t[j] = t[2 * j] + t[2 * j + 1];
  }
  return t[0];
}

// ---------------------------------------------------------------- scale --
// Smallest binary16 value >= t (t >= 0), saturated to 65504 (0x7BFF); any
// NaN or value above 65504 gives 0x7BFF.  v_cvt_f16_f32 rounds to nearest
// even with fp16 denormals kept; stepping the pattern up by one gives the
// next larger binary16 value.
__device__ __forceinline__ uint32_t f16_round_up(float t) {
  _Float16 h = (_Float16)t;
  uint32_t hb = (uint32_t)__builtin_bit_cast(unsigned short, h);
  hb += ((float)h < t) ? 1u : 0u;
  return hb < 0x7BFFu ? hb : 0x7BFFu;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t hb) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)hb);
}

struct BlockScale {
  uint32_t s16;   // binary16 pattern
  float s;        // its value
  float inv;      // fl(1 / s), or 0 when s == 0
};

// fl(a / Q) for a >= 0: one multiply by fl(1/Q) and one FMA correction.
// Equal to the IEEE quotient for every non-negative finite binary32 a and
// Q in {7, 127} (checked exhaustively on the CPU by the test suite).
template <int Q>
__device__ __forceinline__ float div_by_grid(float a) {
  if constexpr (Q == 1) {
    return a;
  } else {
    constexpr float c = 1.0f / (float)Q;
    const float q0 = a * c;
    const float r = __builtin_fmaf(-q0, (float)Q, a);
    return __builtin_fmaf(r, c, q0);
  }
}

// fl(1 / s) for a binary16 value s >= 0 (0 -> 0).  s has an 11-bit
// significand, so 1/s lies at least 2^-12 ulp from any rounding midpoint, and
// one FMA Newton step from the hardware estimate (within 1 ulp) rounds
// correctly (checked for every binary16 s and every estimate within 2 ulp).
__device__ __forceinline__ float recip_f16_value(float s) {
  const float y0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, y0, 1.0f);
  const float y1 = __builtin_fmaf(e, y0, y0);
  return s != 0.0f ? y1 : 0.0f;
}

// s16 = round-up binary16 of t, its value and reciprocal.
__device__ __forceinline__ BlockScale make_scale(float t) {
  BlockScale r;
  r.s16 = f16_round_up(t);
  r.s = f16_bits_to_f32(r.s16);
  r.inv = recip_f16_value(r.s);
  return r;
}

// ----------------------------------------------------------------- hash --
// MurmurHash3 32-bit finaliser, its steps after the first xor-shift, and
// its steps after the first multiply.
constexpr uint32_t kFmixK1 = 0x85EBCA6Bu;
constexpr uint32_t kFmixK2 = 0xC2B2AE35u;
__device__ __forceinline__ uint32_t fmix32_after_first_multiply(uint32_t h) {
  h ^= h >> 13;
  h *= kFmixK2;
  h ^= h >> 16;
  return h;
}
__device__ __forceinline__ uint32_t fmix32_after_first_step(uint32_t h) {
  return fmix32_after_first_multiply(h * kFmixK1);
}

// The first products (c ^ j) * K1 (mod 2^32) for j = 0 .. N - 1 (N a power
// of two, at most 16) with one add or subtract each instead of a multiply.
// Walking j in Gray-code order, j_k = k ^ (k >> 1), consecutive values differ
// in one bit b; flipping bit b of c ^ j changes the product by +-K1 * 2^b,
// plus when the bit becomes set.  d[b] = (1 - 2 c_b) K1 2^b is the change
// when bit b of j goes from 0 to 1.
// All ones where bit b of x is set, else zero (v_bfe_i32).  Written as one
// instruction the compiler cannot see through, so that a conditional negation
// built on it stays two integer operations instead of a select between two
// constants that it would reload into registers for every use.
__device__ __forceinline__ uint32_t bit_mask(uint32_t x, int b) {
  uint32_t m;
  asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(m) : "v"(x), "i"(b));
  return m;
}

template <int N>
struct GrayProducts {
  static constexpr int LOG2N = N <= 1 ? 0 : N <= 2 ? 1 : N <= 4 ? 2 : N <= 8 ? 3 : 4;
  static_assert((1 << LOG2N) == N && N <= 16, "N a power of two up to 16");
  uint32_t p;                       // the product for the current j
  uint32_t d[LOG2N > 0 ? LOG2N : 1];
  __device__ __forceinline__ explicit GrayProducts(uint32_t c) {
    p = c * kFmixK1;                // j = 0
#pragma unroll
    for (int b = 0; b < LOG2N; ++b) {
      // m: all ones when bit b of c is set; (K ^ m) - m = -K or K
      const uint32_t m = bit_mask(c, b);
      d[b] = ((kFmixK1 << b) ^ m) - m;
    }
  }
  // the j of step k, and the product for it (step k >= 1 follows step k - 1)
  static constexpr int index(int k) { return k ^ (k >> 1); }
  __device__ __forceinline__ void step(int k) {
    const int flip = index(k) ^ index(k - 1);            // one bit
    const int b = flip == 1 ? 0 : flip == 2 ? 1 : flip == 4 ? 2 : 3;
    p = (index(k) & flip) ? p + d[b] : p - d[b];
  }
};
__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
  return fmix32_after_first_step(h ^ (h >> 16));
}

// The stochastic-rounding hash of global element index i starts from
// lo ^ fmix32(hi ^ key), lo and hi the 32-bit halves of i.  For the indices
// base + k (0 <= k < 2^32, base wave-uniform) hi is base's high half or one
// more, so both high-half terms are computed once in scalar registers and
// each lane picks one by the carry out of its low half.
struct HiMix {
  uint32_t lo0, m0, m1;
  __device__ __forceinline__ HiMix(uint64_t base, uint32_t key)
      : lo0((uint32_t)base),
        m0(fmix32((uint32_t)(base >> 32) ^ key)),
        m1(fmix32(((uint32_t)(base >> 32) + 1u) ^ key)) {}
  // lo ^ fmix32(hi ^ key) of index base + k
  __device__ __forceinline__ uint32_t x0(uint32_t k) const {
    const uint32_t lo = lo0 + k;
    return lo ^ (lo < lo0 ? m1 : m0);
  }
};

// floor(y) as an int32 in one instruction (v_cvt_flr_i32_f32; the compiler
// emits v_floor_f32 + v_cvt_i32_f32 for (int)floorf(y)).  Measured on gfx950
// with binary32 denormals kept: negative subnormals give -1 and -0 gives 0,
// as floorf; values beyond the int32 range saturate; NaN gives INT32_MAX.
__device__ __forceinline__ int floor_to_int(float y) {
  int q;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(q) : "v"(y));
  return q;
}

// ---------------------------------------------------------------- loads --
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Element access helpers.  Every address is split into the buffer base plus
// a wave-uniform element offset t0 (scalar registers) and a 32-bit per-lane
// element offset `off`, which maps onto the scalar-base + 32-bit-offset
// addressing mode of global loads and stores.

typedef float f32x4 __attribute__((ext_vector_type(4)));

// A plain compress of binary32 input reads it as a stream (non-temporal
// loads) unless the caller says it reads the input again soon
// (LOWBIT_HINT_INPUT_REUSED).  Every such compress reads its input with
// loads whose 16-byte pieces are consecutive across the wave: the 1-bit
// compress (four elements per lane), the 8-bit one (four elements per lane,
// R rows of them) and the 2- and 4-bit ones through LDS (load_tile_staged).
// Measured on the 64 Mi bucket, each alone after the Infinity Cache was
// cleared: 1 bit 50.6 -> 46.3 us, 8 bits 61.6 -> 59.1 us; but a second
// compress of the same bucket right after one with non-temporal loads finds
// none of it in the Infinity Cache (2-bit compress 49 -> 57 us).  (With a
// lane's own 32- or 64-byte span loaded directly, non-temporal loads cost up
// to 50 %: each load instruction then fetches half lines that the next one
// refetches.)
template <int MODE, int DT, int E, int R>
constexpr bool stream_capable() {
  return (MODE == kPlain || MODE == kHadamard) && DT == kF32 && E >= 4 && R >= 1;
}

// Load E consecutive elements at element t0 + off (16-byte aligned for E >= 8
// in bf16 and E >= 4 in fp32; 8-byte for E == 4 in bf16); NT: non-temporal
// (binary32 only).
template <int DT, int E, bool NT = false>
__device__ __forceinline__ void load_vec(const void* base, int64_t t0, uint32_t off, float* v) {
  if constexpr (DT == kF32) {
    const float* p = static_cast<const float*>(base) + t0;
    const float4* q = reinterpret_cast<const float4*>(p + off);
#pragma unroll
    for (int k = 0; k < E / 4; ++k) {
      if constexpr (NT) {
        const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(q) + k);
        v[4 * k + 0] = t.x;
        v[4 * k + 1] = t.y;
        v[4 * k + 2] = t.z;
        v[4 * k + 3] = t.w;
      } else {
        float4 t = q[k];
        v[4 * k + 0] = t.x;
        v[4 * k + 1] = t.y;
        v[4 * k + 2] = t.z;
        v[4 * k + 3] = t.w;
      }
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(base) + t0;
    if constexpr (E == 4) {
      uint2 t = *reinterpret_cast<const uint2*>(p + off);
      v[0] = bf16_lo(t.x);
      v[1] = bf16_hi(t.x);
      v[2] = bf16_lo(t.y);
      v[3] = bf16_hi(t.y);
    } else {
      const uint4* q = reinterpret_cast<const uint4*>(p + off);
#pragma unroll
      for (int k = 0; k < E / 8; ++k) {
        uint4 t = q[k];
        v[8 * k + 0] = bf16_lo(t.x);
        v[8 * k + 1] = bf16_hi(t.x);
        v[8 * k + 2] = bf16_lo(t.y);
        v[8 * k + 3] = bf16_hi(t.y);
        v[8 * k + 4] = bf16_lo(t.z);
        v[8 * k + 5] = bf16_hi(t.z);
        v[8 * k + 6] = bf16_lo(t.w);
        v[8 * k + 7] = bf16_hi(t.w);
      }
    }
  }
}

// Guarded element-by-element load for a ragged last tile: positions
// off + j >= rem (rem = n - t0, the valid elements from t0 on) read as +0.
template <int DT, int E>
__device__ __forceinline__ void load_tail(const void* base, int64_t t0, uint32_t off, int64_t rem,
                                          float* v) {
#pragma unroll
  for (int j = 0; j < E; ++j) {
    float x = 0.0f;
    if ((int64_t)off + j < rem) {
      if constexpr (DT == kF32) x = (static_cast<const float*>(base) + t0)[off + j];
      else x = __uint_as_float((uint32_t)(static_cast<const uint16_t*>(base) + t0)[off + j] << 16);
    }
    v[j] = x;
  }
}

// Streaming stores: outputs are written once and read by a later kernel, so
// they are stored non-temporally and do not linger as dirty cache lines whose
// write-back the next kernel would pay for (measured on MI355X: a 256 MiB read
// takes 43 us after a non-temporal 256 MiB write, 66 us after a plain one;
// the whole compress/reduce/decompress/EF/weight-difference pass is 12 %
// faster with non-temporal outputs).
__device__ __forceinline__ void store_stream(uint32_t* p, uint32_t v) {
  __builtin_nontemporal_store(v, p);
}

// K = 2 or 4 words (8 or 16 bytes, aligned to that) in one streaming store.
template <int K>
__device__ __forceinline__ void store_stream_words(uint32_t* p, const uint32_t* v) {
  static_assert(K == 2 || K == 4, "8- or 16-byte stores");
  typedef uint32_t vk __attribute__((ext_vector_type(K)));
  vk q;
#pragma unroll
  for (int k = 0; k < K; ++k) q[k] = v[k];
  __builtin_nontemporal_store(q, reinterpret_cast<vk*>(p));
}

template <int E>
__device__ __forceinline__ void store_vec_f32(float* base, int64_t t0, uint32_t off, const float* v) {
  float* p = base + t0 + off;
#pragma unroll
  for (int k = 0; k < E / 4; ++k) {
    const f32x4 q = {v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
    __builtin_nontemporal_store(q, reinterpret_cast<f32x4*>(p) + k);
  }
}

template <int E>
__device__ __forceinline__ void store_tail_f32(float* base, int64_t t0, uint32_t off, int64_t rem,
                                               const float* v) {
#pragma unroll
  for (int j = 0; j < E; ++j)
    if ((int64_t)off + j < rem) (base + t0)[off + j] = v[j];
}

// binary32 -> bfloat16, round to nearest even, by integer arithmetic.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;   // NaN stays NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace lowbit
