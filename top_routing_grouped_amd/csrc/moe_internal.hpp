// Internal declarations of the MI355X MoE layer library: kernel launchers
// and the small device helpers they share.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace moe {

// Problem as the launchers see it (validated on the host beforehand).
struct Problem {
  int64_t T;          // tokens
  int d, E, K, n;     // width, experts, experts per token, expert FFN width
  bool bf16;          // element type of X, weights, H, O, Y (else fp32)
  int64_t C;          // per-expert cap
  int64_t rows_max;   // upper bound on kept assignments: min(T*K, E*C)
};

// Token block of the permutation kernels (one workgroup of threads, one
// token per thread).
constexpr int kPermuteBlock = 256;

// Tile rows of the grouped GEMMs (shared by both GEMMs so one tile table
// serves both).
constexpr int kGemmBM = 256;

inline int64_t permute_blocks(int64_t T) { return (T + kPermuteBlock - 1) / kPermuteBlock; }

// Upper bound on row tiles over all experts: sum_e ceil(c_e/BM) with
// sum_e c_e <= rows_max.
inline int64_t max_row_tiles(const Problem& p, int bm) {
  return (p.rows_max + (int64_t)p.E * (bm - 1)) / bm;
}

// Tile table layout: int4 header {count, 0, 0, 0}, then one int4 per row
// tile {expert | tiles_of_expert << 8, row_begin, row_end, first_tile_of_expert}.
// An expert's row tiles are consecutive entries.  The packed word is read as
// uint32: expert < 256 and tiles_of_expert <= 2^23 (T*K < 2^31).
__host__ __device__ inline int tile_expert(uint32_t w) { return (int)(w & 255u); }
__host__ __device__ inline int tile_expert_tiles(uint32_t w) { return (int)(w >> 8); }

inline size_t tile_table_bytes(const Problem& p) {
  return (size_t)(max_row_tiles(p, kGemmBM) + 1) * 4 * sizeof(int32_t);
}

// ---------------------------------------------------------------- launchers
hipError_t launch_route(const Problem& p, const void* X, const void* W_r, const float* bias,
                        float* logits, int32_t* ids, float* gates, hipStream_t s);

hipError_t launch_histogram(const Problem& p, const int32_t* ids, int32_t* blockcnt,
                            hipStream_t s);
// table may be NULL; when given, the scan also writes the grouped-GEMM tile table.
hipError_t launch_scan(const Problem& p, const int32_t* blockcnt, int32_t* blockbase,
                       int32_t* raw, int32_t* counts, int32_t* offsets, int32_t* table,
                       hipStream_t s);
hipError_t launch_scatter(const Problem& p, const int32_t* ids, const int32_t* blockbase,
                          const int32_t* offsets, int32_t* perm, int32_t* inv_slot,
                          hipStream_t s);
hipError_t launch_tile_table(const Problem& p, const int32_t* offsets, int32_t* table,
                             hipStream_t s);

hipError_t launch_gemm_up(const Problem& p, const void* X, const int32_t* perm,
                          const int32_t* table, const void* W_gate, const void* W_up, void* H,
                          hipStream_t s);
hipError_t launch_gemm_down(const Problem& p, const void* H, const int32_t* table,
                            const void* W_down, void* O, hipStream_t s);

hipError_t launch_combine(const Problem& p, const void* O, const float* gates,
                          const int32_t* inv_slot, void* Y, hipStream_t s);

}  // namespace moe

// ---------------------------------------------------------------- device helpers
#ifdef __HIPCC__
namespace moe {
namespace dev {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// Workgroup barrier without the memory fence that __syncthreads adds (the
// fence would also wait for in-flight global->LDS prefetches).  The memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace dev
}  // namespace moe
#endif
