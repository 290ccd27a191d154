// decompress, weight-difference apply and the measurement copy and add kernels
#include "launch.hpp"
#include "dequant.hpp"

namespace lowbit {

template <int BITS, int APPLY, int DT>
static lowbit_status launch_d(const DequantArgs& a, hipStream_t s) {
  constexpr int ROWS = dequant_rows<APPLY>();
  constexpr int ROW = kWave * dequant_epl<APPLY>();
  const int64_t nrows = (a.n + ROW - 1) / ROW;
  const int64_t ntrips = (nrows + ROWS - 1) / ROWS;
  hipLaunchKernelGGL((dequant_kernel<BITS, APPLY, DT>), dim3(grid_for_tiles<kDeqThreads>(ntrips)),
                     dim3(kDeqThreads), 0, s, a);
  return launch_status();
}

template <int BITS>
static lowbit_status launch_d_b(bool apply, int dt, const DequantArgs& a, hipStream_t s) {
  if (!apply) return launch_d<BITS, 0, kF32>(a, s);
  return dt == kF32 ? launch_d<BITS, 1, kF32>(a, s) : launch_d<BITS, 1, kBF16>(a, s);
}

lowbit_status launch_dequant(int bits, bool apply, int dt, const DequantArgs& a, hipStream_t s) {
  switch (bits) {
    case 1: return launch_d_b<1>(apply, dt, a, s);
    case 2: return launch_d_b<2>(apply, dt, a, s);
    case 4: return launch_d_b<4>(apply, dt, a, s);
    case 8: return launch_d_b<8>(apply, dt, a, s);
  }
  return LOWBIT_EUNSUPPORTED;
}

template <int BITS, int LOG2B>
static lowbit_status launch_hd(const DequantArgs& a, hipStream_t s) {
  const int64_t nrows = (a.n + kDeqRow - 1) / kDeqRow;
  constexpr int ROWS = hadamard_rows_per_trip<LOG2B>();
  // one wave per LOWBIT_HS_DEQ_TRIPS trips
  const int64_t waves = (nrows + ROWS * LOWBIT_HS_DEQ_TRIPS - 1) / (ROWS * LOWBIT_HS_DEQ_TRIPS);
  hipLaunchKernelGGL((hadamard_dequant_kernel<BITS, LOG2B>),
                     dim3(grid_for_tiles<kDeqThreads>(waves)), dim3(kDeqThreads), 0, s, a);
  return launch_status();
}

template <int BITS>
static lowbit_status launch_hd_b(const DequantArgs& a, hipStream_t s) {
  switch (a.log2b) {
    case 5: return launch_hd<BITS, 5>(a, s);
    case 6: return launch_hd<BITS, 6>(a, s);
    case 7: return launch_hd<BITS, 7>(a, s);
    case 8: return launch_hd<BITS, 8>(a, s);
    case 9: return launch_hd<BITS, 9>(a, s);
    case 10: return launch_hd<BITS, 10>(a, s);
    case 11: return launch_hd<BITS, 11>(a, s);
    case 12: return launch_hd<BITS, 12>(a, s);
  }
  return LOWBIT_EUNSUPPORTED;
}

lowbit_status launch_hadamard_dequant(int bits, const DequantArgs& a, hipStream_t s) {
  switch (bits) {
    case 1: return launch_hd_b<1>(a, s);
    case 2: return launch_hd_b<2>(a, s);
    case 4: return launch_hd_b<4>(a, s);
    case 8: return launch_hd_b<8>(a, s);
  }
  return LOWBIT_EUNSUPPORTED;
}

lowbit_status launch_copy(const float* x, float* y, int64_t n, hipStream_t s) {
  const int64_t nvec = n / 4;
  int64_t blocks = (nvec + kCopyUnroll * kBlockThreads - 1) / (kCopyUnroll * kBlockThreads);
  int64_t cap = (int64_t)1 << 30;
  if (LOWBIT_BLOCKS_PER_CU > 0) cap = (int64_t)device_cu_count() * LOWBIT_BLOCKS_PER_CU;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kBlockThreads), 0, s, x, y, n);
  return launch_status();
}

lowbit_status launch_add_inplace(const float* x, float* y, int64_t n, hipStream_t s) {
  const int64_t waves = (n + 4 * kWave - 1) / (4 * kWave);
  hipLaunchKernelGGL(add_inplace_kernel, dim3(grid_for_tiles(waves)), dim3(kBlockThreads), 0, s,
                     x, y, n);
  return launch_status();
}

lowbit_status launch_fold(const float* x, int64_t n, int bits, uint32_t* out, hipStream_t s) {
  const int64_t tiles = (n + 2047) / 2048;
  const int64_t nwords = (n * bits + 31) / 32;
  const dim3 grid(grid_for_tiles(tiles)), block(kBlockThreads);
  switch (bits) {
    case 1: hipLaunchKernelGGL(fold_kernel<1>, grid, block, 0, s, x, n, out, nwords); break;
    case 2: hipLaunchKernelGGL(fold_kernel<2>, grid, block, 0, s, x, n, out, nwords); break;
    case 4: hipLaunchKernelGGL(fold_kernel<4>, grid, block, 0, s, x, n, out, nwords); break;
    case 8: hipLaunchKernelGGL(fold_kernel<8>, grid, block, 0, s, x, n, out, nwords); break;
    default: return LOWBIT_EUNSUPPORTED;
  }
  return launch_status();
}

}  // namespace lowbit
