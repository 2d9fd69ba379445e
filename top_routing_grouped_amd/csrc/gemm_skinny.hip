// Steps 6-7 of the layer for batches with few rows per expert (decode-sized
// batches): the grouped GEMMs become weight streams.
//
// Same arithmetic as the tiled kernels in gemm.hip (the SonicMoE article's
// gathered up-projection with a SwiGLU epilogue, §3, §6.2, §6.3, and the
// down-projection), but with a handful of rows per expert almost every byte
// moved is weight: the work is bound by reading each active expert's
// weights once from HBM, so the kernel is organised around that stream.
//
// * The body (gemm_stream.hpp) runs here on 4 waves, one workgroup per
//   expert and block of 256 weight columns; experts without rows exit at
//   once, so only active experts' weights are read.  Measured at the decode
//   size (T=64, d=4096, E=256, n=512) with cached copies: the weight stream
//   ran at 4.7-4.9 TB/s whether or not the MFMAs ran and for 3 to 8 stages,
//   i.e. bound by the memory system for these strided 512-byte row pieces
//   (128-column blocks: 4.5-4.75 TB/s).  The weight copies carry the
//   non-temporal hint (each weight is read once per launch): that lifted the
//   up projection from 374 to 305 us at this size.
// * Rows are taken in passes of 64, or 32 when the batch averages at most 16
//   rows per expert (a smaller token tile leaves more LDS to weights).
#include "gemm_stream.hpp"

namespace moe {
namespace {

constexpr int kSkinnyCols = 256;   // weight columns per workgroup (128-column blocks were slower)
constexpr int kSkinnyWaves = 4;

// ROWS rows per pass: 64, or 32 for batches with at most 16 rows per expert
// on average (a smaller token tile leaves more LDS to weights).
template <int ROWS, int COLS>
using SkinnyGeo = wstream::Geo<ROWS, COLS, kSkinnyWaves>;

template <bool UP, int ROWS, int COLS>
__global__ __launch_bounds__(64 * kSkinnyWaves, 1) void skinny_gemm_bf16(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, uint16_t* __restrict__ C, int64_t T, int Kd, int N,
    int64_t rows_max) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  wstream::stream_block<UP, ROWS, COLS, kSkinnyWaves>(A, perm, offsets, B0, B1, C, T, Kd, N,
                                                      rows_max, 1 << 30, (int)blockIdx.y,
                                                      (int)blockIdx.x, smem);
}

template <bool UP, int ROWS>
hipError_t launch_rows(const Problem& p, const uint16_t* A, const int32_t* perm,
                       const int32_t* offsets, const uint16_t* B0, const uint16_t* B1,
                       uint16_t* C, hipStream_t s) {
  constexpr int kCols = kSkinnyCols;
  auto* kern = skinny_gemm_bf16<UP, ROWS, kCols>;
  constexpr int kLds = SkinnyGeo<ROWS, kCols>::kLds;
  const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (err != hipSuccess) return err;
  const int N = UP ? p.n : p.d;
  const int Kd = UP ? p.d : p.n;
  const int cols = UP ? kCols / 2 : kCols;
  const dim3 grid((unsigned)((N + cols - 1) / cols), (unsigned)p.E);
  hipLaunchKernelGGL(kern, grid, dim3(SkinnyGeo<ROWS, kCols>::kThreads), (size_t)kLds, s, A, perm, offsets, B0, B1, C,
                     p.T, Kd, N, p.rows_max);
  return hipGetLastError();
}

template <bool UP>
hipError_t launch_skinny(const Problem& p, const uint16_t* A, const int32_t* perm,
                         const int32_t* offsets, const uint16_t* B0, const uint16_t* B1,
                         uint16_t* C, hipStream_t s) {
  if (p.T * (int64_t)p.K <= 16 * (int64_t)p.E)
    return launch_rows<UP, 32>(p, A, perm, offsets, B0, B1, C, s);
  return launch_rows<UP, 64>(p, A, perm, offsets, B0, B1, C, s);
}

}  // namespace

hipError_t launch_gemm_up_skinny(const Problem& p, const void* X, const int32_t* perm,
                                 const int32_t* offsets, const void* W_gate, const void* W_up,
                                 void* H, hipStream_t s) {
  return launch_skinny<true>(p, (const uint16_t*)X, perm, offsets, (const uint16_t*)W_gate,
                             (const uint16_t*)W_up, (uint16_t*)H, s);
}

hipError_t launch_gemm_down_skinny(const Problem& p, const void* H, const int32_t* offsets,
                                   const void* W_down, void* O, hipStream_t s) {
  return launch_skinny<false>(p, (const uint16_t*)H, nullptr, offsets, (const uint16_t*)W_down,
                              nullptr, (uint16_t*)O, s);
}

}  // namespace moe
