// decompress, weight-difference apply and the measurement copy and add kernels
#include "launch.hpp"
#include "dequant.hpp"

namespace lowbit {

template <int BITS, int APPLY, int DT>
static lowbit_status launch_d(const DequantArgs& a, hipStream_t s) {
  constexpr int ROWS = dequant_rows<BITS, APPLY>();
  constexpr int ROW = kWave * dequant_epl<APPLY>();
  const int64_t nrows = (a.n + ROW - 1) / ROW;
  const int64_t ntrips = (nrows + ROWS - 1) / ROWS;
  constexpr int THREADS = deq_threads<BITS, APPLY>();
  return launch(&dequant_kernel<BITS, APPLY, DT>, grid_for_tiles<THREADS>(ntrips), THREADS, s, a);
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
  if constexpr (LOG2B == 12) {
    // whole blocks: a workgroup each; a partial last block: the one-wave trip
    // on the remainder (as a buffer of its own, which starts on a block)
    const int64_t nfull = a.n >> LOG2B;
    lowbit_status st = LOWBIT_OK;
    if (nfull > 0)
      st = launch(&hadamard_dequant_big_kernel<BITS>,
                  grid_blocks(nfull * kHsBigWaves, kHsBigWaves * kWave), kHsBigWaves * kWave, s,
                  a, nfull);
    const int64_t done = nfull << LOG2B;
    if (st != LOWBIT_OK || done == a.n) return st;
    DequantArgs rest = a;
    rest.codes = a.codes + done / Grid<BITS>::E;
    rest.scales = a.scales + nfull;
    rest.y = a.y + done;
    rest.n = a.n - done;
    return launch(&hadamard_dequant_kernel<BITS, LOG2B>, 1, kHsDeqThreads, s, rest);
  }
  const int64_t nrows = (a.n + kDeqRow - 1) / kDeqRow;
  constexpr int ROWS = hadamard_rows_per_trip<LOG2B>();
  const int64_t waves = (nrows + ROWS - 1) / ROWS;   // one trip per wave
  return launch(&hadamard_dequant_kernel<BITS, LOG2B>, grid_for_tiles<kHsDeqThreads>(waves),
                kHsDeqThreads, s, a);
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
  return launch(&copy_kernel, grid_blocks((nvec + 63) / 64, kBlockThreads), kBlockThreads, s, x, y,
                n);
}

lowbit_status launch_add_inplace(const float* x, float* y, int64_t n, hipStream_t s) {
  const int64_t waves = (n + 4 * kWave - 1) / (4 * kWave);
  return launch(&add_inplace_kernel, grid_for_tiles(waves), kBlockThreads, s, x, y, n);
}

lowbit_status launch_fold(const float* x, int64_t n, int bits, uint32_t* out, hipStream_t s) {
  const int64_t tiles = (n + 2047) / 2048;
  const int64_t nwords = (n * bits + 31) / 32;
  const int64_t grid = grid_for_tiles(tiles);
  switch (bits) {
    case 1: return launch(&fold_kernel<1>, grid, kBlockThreads, s, x, n, out, nwords);
    case 2: return launch(&fold_kernel<2>, grid, kBlockThreads, s, x, n, out, nwords);
    case 4: return launch(&fold_kernel<4>, grid, kBlockThreads, s, x, n, out, nwords);
    case 8: return launch(&fold_kernel<8>, grid, kBlockThreads, s, x, n, out, nwords);
  }
  return LOWBIT_EUNSUPPORTED;
}

}  // namespace lowbit
