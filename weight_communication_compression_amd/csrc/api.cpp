// api.cpp -- the extern "C" entry points of liblowbit (declared in
// include/lowbit.h): argument validation, the stochastic-rounding key, and
// dispatch to the gfx950 kernels.  Invalid arguments are rejected before any
// HIP call; nothing here allocates device memory or keeps any state.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/lowbit.h"
#include "args.hpp"
#include "launch.hpp"

namespace lowbit {

namespace {

constexpr int64_t kMaxN = (int64_t)1 << 48;

bool valid_bits(int32_t b) { return b == 1 || b == 2 || b == 4 || b == 8; }

int log2_block(int32_t B) {
  if (B < 32 || B > 4096 || (B & (B - 1)) != 0) return -1;
  int l = 0;
  while ((1 << l) < B) ++l;
  return l;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// MurmurHash3 32-bit finaliser (host copy for the per-call key).
uint32_t fmix32_host(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

uint32_t seed_key(uint64_t seed) {
  return fmix32_host((uint32_t)seed ^ fmix32_host((uint32_t)(seed >> 32) ^ 0x9E3779B9u));
}

// Common checks of one lowbit_qparams; returns log2(B) or -1.
int check_params(const lowbit_qparams* p) {
  if (!p || !valid_bits(p->bitwidth) || (p->hints & ~LOWBIT_HINT_INPUT_REUSED) != 0) return -1;
  const int lb = log2_block(p->block_size);
  if (lb < 0) return -1;
  if (p->index_offset % (uint64_t)p->block_size != 0) return -1;
  return lb;
}

bool valid_dtype(int dt) { return dt == LOWBIT_F32 || dt == LOWBIT_BF16; }

}  // namespace

}  // namespace lowbit

using namespace lowbit;

extern "C" {

int64_t lowbit_num_words(int64_t n, int32_t bitwidth) {
  if (n < 0 || n > kMaxN || !valid_bits(bitwidth)) return -1;
  return (n * bitwidth + 31) / 32;
}

int64_t lowbit_num_blocks(int64_t n, int32_t block_size) {
  if (n < 0 || n > kMaxN || log2_block(block_size) < 0) return -1;
  return (n + block_size - 1) / block_size;
}

const char* lowbit_status_string(lowbit_status status) {
  switch (status) {
    case LOWBIT_OK: return "ok";
    case LOWBIT_EINVAL: return "invalid argument";
    case LOWBIT_EUNSUPPORTED: return "unsupported combination";
    case LOWBIT_EDEVICE: return "device launch error";
  }
  return "unknown status";
}

const char* lowbit_version(void) { return "lowbit 0.1.0 gfx950"; }

lowbit_status lowbit_quantize_pack(const void* x, lowbit_dtype xt, int64_t n,
                                   const lowbit_qparams* p, uint32_t* codes, uint16_t* scales,
                                   hipStream_t stream) {
  const int lb = check_params(p);
  if (lb < 0 || n < 0 || n > kMaxN || !valid_dtype(xt)) return LOWBIT_EINVAL;
  if (n == 0) return LOWBIT_OK;
  if (!x || !codes || !scales) return LOWBIT_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(scales, 2)) return LOWBIT_EINVAL;
  QuantArgs a{};
  a.x = x;
  a.n = n;
  a.out = TileOut{codes, scales, p->index_offset, seed_key(p->seed)};
  return launch_quantize_plain(p->bitwidth, lb, p->stochastic != 0, (int)xt,
                               (p->hints & LOWBIT_HINT_INPUT_REUSED) == 0, a, stream);
}

lowbit_status lowbit_unpack_dequant(const uint32_t* codes, const uint16_t* scales, int64_t n,
                                    const lowbit_qparams* p, float* y, hipStream_t stream) {
  const int lb = check_params(p);
  if (lb < 0 || n < 0 || n > kMaxN) return LOWBIT_EINVAL;
  if (n == 0) return LOWBIT_OK;
  if (!codes || !scales || !y) return LOWBIT_EINVAL;
  if (!aligned(y, 16) || !aligned(codes, 4) || !aligned(scales, 2)) return LOWBIT_EINVAL;
  DequantArgs a{};
  a.codes = codes;
  a.scales = scales;
  a.n = n;
  a.log2b = lb;
  a.y = y;
  return launch_dequant(p->bitwidth, false, LOWBIT_F32, a, stream);
}

// Hadamard smoothing: whole blocks transformed, a partial last block not.
lowbit_status lowbit_hadamard_quantize_pack(const void* x, lowbit_dtype xt, int64_t n,
                                            const lowbit_qparams* p, uint32_t* codes,
                                            uint16_t* scales, hipStream_t stream) {
  const int lb = check_params(p);
  if (lb < 0 || n < 0 || n > kMaxN || !valid_dtype(xt)) return LOWBIT_EINVAL;
  if (n == 0) return LOWBIT_OK;
  if (!x || !codes || !scales) return LOWBIT_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(scales, 2)) return LOWBIT_EINVAL;
  QuantArgs a{};
  a.x = x;
  a.n = n;
  a.out = TileOut{codes, scales, p->index_offset, seed_key(p->seed)};
  return launch_quantize_hadamard(p->bitwidth, lb, p->stochastic != 0, (int)xt,
                                  (p->hints & LOWBIT_HINT_INPUT_REUSED) == 0, a, stream);
}

lowbit_status lowbit_hadamard_unpack_dequant(const uint32_t* codes, const uint16_t* scales,
                                             int64_t n, const lowbit_qparams* p, float* y,
                                             hipStream_t stream) {
  const int lb = check_params(p);
  if (lb < 0 || n < 0 || n > kMaxN) return LOWBIT_EINVAL;
  if (n == 0) return LOWBIT_OK;
  if (!codes || !scales || !y) return LOWBIT_EINVAL;
  if (!aligned(y, 16) || !aligned(codes, 4) || !aligned(scales, 2)) return LOWBIT_EINVAL;
  DequantArgs a{};
  a.codes = codes;
  a.scales = scales;
  a.n = n;
  a.log2b = lb;
  a.y = y;
  return launch_hadamard_dequant(p->bitwidth, a, stream);
}

lowbit_status lowbit_ef_compress(const void* g, lowbit_dtype gt, float* residual, int64_t n,
                                 const lowbit_qparams* p, uint32_t* codes, uint16_t* scales,
                                 hipStream_t stream) {
  const int lb = check_params(p);
  if (lb < 0 || n < 0 || n > kMaxN || !valid_dtype(gt)) return LOWBIT_EINVAL;
  if (n == 0) return LOWBIT_OK;
  if (!g || !residual || !codes || !scales) return LOWBIT_EINVAL;
  if (!aligned(g, 16) || !aligned(residual, 16) || !aligned(codes, 4) || !aligned(scales, 2))
    return LOWBIT_EINVAL;
  QuantArgs a{};
  a.x = g;
  a.resid = residual;
  a.n = n;
  a.out = TileOut{codes, scales, p->index_offset, seed_key(p->seed)};
  return launch_quantize_ef(p->bitwidth, lb, p->stochastic != 0, (int)gt, false, a, stream);
}

}  // extern "C"

namespace {

// Shared body of the two local-reduce entry points (residual == nullptr: no
// stage-2 error feedback).
lowbit_status reduce_common(const uint32_t* const* peer_codes, const uint16_t* const* peer_scales,
                            int32_t npeers, int64_t n, const lowbit_qparams* in_p,
                            const lowbit_qparams* out_p, float* residual, bool want_residual,
                            uint32_t* out_codes, uint16_t* out_scales, float* out_sum,
                            hipStream_t stream) {
  const int lb_in = check_params(in_p);
  const int lb = check_params(out_p);
  if (lb_in < 0 || lb < 0 || n < 0 || n > kMaxN) return LOWBIT_EINVAL;
  if (npeers < 1 || npeers > kMaxPeers) return LOWBIT_EINVAL;
  const int bi = in_p->bitwidth, bo = out_p->bitwidth;
  const bool mixed = bi != bo;
  if (mixed && !((bi == 8 && (bo == 4 || bo == 2)) || (bi == 4 && bo == 2)))
    return LOWBIT_EUNSUPPORTED;
  if (n == 0) return LOWBIT_OK;
  if (!peer_codes || !peer_scales || !out_codes || !out_scales) return LOWBIT_EINVAL;
  if (want_residual && (!residual || !aligned(residual, 16))) return LOWBIT_EINVAL;
  if (!aligned(out_codes, 4) || !aligned(out_scales, 2) || (out_sum && !aligned(out_sum, 16)))
    return LOWBIT_EINVAL;
  // a lane loads b_in/b_out input words as one vector
  const uintptr_t in_align = mixed ? (uintptr_t)(4 * (bi / bo)) : 4;
  ReduceArgs a{};
  for (int p = 0; p < npeers; ++p) {
    if (!peer_codes[p] || !peer_scales[p] || !aligned(peer_codes[p], in_align) ||
        !aligned(peer_scales[p], 2))
      return LOWBIT_EINVAL;
    a.codes[p] = peer_codes[p];
    a.scales[p] = peer_scales[p];
  }
  a.npeers = npeers;
  a.in_log2b = lb_in;
  a.n = n;
  a.out_sum = out_sum;
  a.resid = residual;
  a.out = TileOut{out_codes, out_scales, out_p->index_offset, seed_key(out_p->seed)};
  const bool sr = out_p->stochastic != 0;
  // the peers' code words are streamed unless the caller reads them again
  const bool si = (in_p->hints & LOWBIT_HINT_INPUT_REUSED) == 0;
  if (mixed) return launch_reduce_mixed(bi, bo, lb, sr, want_residual, si, a, stream);
  return want_residual ? launch_reduce_same_ef(bo, lb, sr, si, a, stream)
                       : launch_reduce_same(bo, lb, sr, si, a, stream);
}

}  // namespace

extern "C" {

lowbit_status lowbit_reduce_requant(const uint32_t* const* peer_codes,
                                    const uint16_t* const* peer_scales, int32_t npeers, int64_t n,
                                    const lowbit_qparams* in_p, const lowbit_qparams* out_p,
                                    uint32_t* out_codes, uint16_t* out_scales, float* out_sum,
                                    hipStream_t stream) {
  return reduce_common(peer_codes, peer_scales, npeers, n, in_p, out_p, nullptr, false, out_codes,
                       out_scales, out_sum, stream);
}

lowbit_status lowbit_reduce_requant_ef(const uint32_t* const* peer_codes,
                                       const uint16_t* const* peer_scales, int32_t npeers,
                                       int64_t n, const lowbit_qparams* in_p,
                                       const lowbit_qparams* out_p, float* residual,
                                       uint32_t* out_codes, uint16_t* out_scales, float* out_sum,
                                       hipStream_t stream) {
  return reduce_common(peer_codes, peer_scales, npeers, n, in_p, out_p, residual, true, out_codes,
                       out_scales, out_sum, stream);
}

lowbit_status lowbit_ef21_compress(const void* g, lowbit_dtype gt, float* state, int64_t n,
                                   const lowbit_qparams* p, uint32_t* codes, uint16_t* scales,
                                   hipStream_t stream) {
  const int lb = check_params(p);
  if (lb < 0 || n < 0 || n > kMaxN || !valid_dtype(gt)) return LOWBIT_EINVAL;
  if (n == 0) return LOWBIT_OK;
  if (!g || !state || !codes || !scales) return LOWBIT_EINVAL;
  if (!aligned(g, 16) || !aligned(state, 16) || !aligned(codes, 4) || !aligned(scales, 2))
    return LOWBIT_EINVAL;
  QuantArgs a{};
  a.x = g;
  a.resid = state;
  a.n = n;
  a.out = TileOut{codes, scales, p->index_offset, seed_key(p->seed)};
  return launch_quantize_ef21(p->bitwidth, lb, p->stochastic != 0, (int)gt, false, a, stream);
}

lowbit_status lowbit_wdiff_compress(const void* w_new, const void* w_old, lowbit_dtype wt,
                                    int64_t n, const lowbit_qparams* p, uint32_t* codes,
                                    uint16_t* scales, hipStream_t stream) {
  const int lb = check_params(p);
  if (lb < 0 || n < 0 || n > kMaxN || !valid_dtype(wt)) return LOWBIT_EINVAL;
  if (n == 0) return LOWBIT_OK;
  if (!w_new || !w_old || !codes || !scales) return LOWBIT_EINVAL;
  if (!aligned(w_new, 16) || !aligned(w_old, 16) || !aligned(codes, 4) || !aligned(scales, 2))
    return LOWBIT_EINVAL;
  QuantArgs a{};
  a.x = w_new;
  a.x2 = w_old;
  a.n = n;
  a.out = TileOut{codes, scales, p->index_offset, seed_key(p->seed)};
  return launch_quantize_wdiff(p->bitwidth, lb, p->stochastic != 0, (int)wt, false, a, stream);
}

lowbit_status lowbit_wdiff_apply(const void* w_old, const uint32_t* codes, const uint16_t* scales,
                                 int64_t n, const lowbit_qparams* p, void* w_out, lowbit_dtype wt,
                                 hipStream_t stream) {
  const int lb = check_params(p);
  if (lb < 0 || n < 0 || n > kMaxN || !valid_dtype(wt)) return LOWBIT_EINVAL;
  if (n == 0) return LOWBIT_OK;
  if (!w_old || !codes || !scales || !w_out) return LOWBIT_EINVAL;
  if (!aligned(w_old, 16) || !aligned(w_out, 16) || !aligned(codes, 4) || !aligned(scales, 2))
    return LOWBIT_EINVAL;
  DequantArgs a{};
  a.codes = codes;
  a.scales = scales;
  a.n = n;
  a.log2b = lb;
  a.w_old = w_old;
  a.w_out = w_out;
  return launch_dequant(p->bitwidth, true, (int)wt, a, stream);
}

lowbit_status lowbit_copy_f32(const float* x, float* y, int64_t n, hipStream_t stream) {
  if (n < 0 || n > kMaxN) return LOWBIT_EINVAL;
  if (n == 0) return LOWBIT_OK;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return LOWBIT_EINVAL;
  return launch_copy(x, y, n, stream);
}

lowbit_status lowbit_add_inplace_f32(const float* x, float* y, int64_t n, hipStream_t stream) {
  if (n < 0 || n > kMaxN) return LOWBIT_EINVAL;
  if (n == 0) return LOWBIT_OK;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return LOWBIT_EINVAL;
  return launch_add_inplace(x, y, n, stream);
}

lowbit_status lowbit_xor_streams_u32(const uint32_t* const* streams, int32_t nstreams,
                                     int64_t nwords, uint32_t* out, hipStream_t stream) {
  if (nstreams < 1 || nstreams > kMaxPeers || nwords < 0 || nwords > kMaxN) return LOWBIT_EINVAL;
  if (nwords == 0) return LOWBIT_OK;
  if (!streams || !out || !aligned(out, 4)) return LOWBIT_EINVAL;
  XorArgs a{};
  for (int p = 0; p < nstreams; ++p) {
    if (!streams[p] || !aligned(streams[p], 4)) return LOWBIT_EINVAL;
    a.streams[p] = streams[p];
  }
  a.out = out;
  a.nwords = nwords;
  a.nstreams = nstreams;
  return launch_xor_streams(a, stream);
}

lowbit_status lowbit_stream_probe_u32(int32_t op, const uint32_t* src, uint32_t* dst,
                                     int64_t nwords, uint32_t value, int32_t waves,
                                     int32_t nontemporal, hipStream_t stream) {
  if (op < LOWBIT_PROBE_READ || op > LOWBIT_PROBE_COPY) return LOWBIT_EINVAL;
  if (nwords < 0 || nwords > kMaxN || nwords % 1024 != 0 || waves < 0) return LOWBIT_EINVAL;
  if (nwords == 0) return LOWBIT_OK;
  if (!dst || !aligned(dst, 16)) return LOWBIT_EINVAL;
  if (op != LOWBIT_PROBE_WRITE && (!src || !aligned(src, 16))) return LOWBIT_EINVAL;
  ProbeArgs a{};
  a.src = src;
  a.dst = dst;
  a.value = value;
  return launch_stream_probe(op, a, nwords, waves, nontemporal != 0, stream);
}

lowbit_status lowbit_fold_f32(const float* x, int64_t n, int32_t bitwidth, uint32_t* out,
                              hipStream_t stream) {
  if (n < 0 || n > kMaxN) return LOWBIT_EINVAL;
  if (bitwidth != 1 && bitwidth != 2 && bitwidth != 4 && bitwidth != 8) return LOWBIT_EINVAL;
  if (n == 0) return LOWBIT_OK;
  if (!x || !out || !aligned(x, 16) || !aligned(out, 16)) return LOWBIT_EINVAL;
  return launch_fold(x, n, bitwidth, out, stream);
}

}  // extern "C"
