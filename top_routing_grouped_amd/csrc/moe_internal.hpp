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
  int sel = 0;        // top-K selection: 0 sorted lanes + row maxima, 1 threshold bisection
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
// 16-column blocks per router wave: the padded expert range is 32*route_nbw.
inline int route_nbw(int E) {
  const int n = (E + 31) / 32;
  return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 8;
}

// Router k split for small batches (bf16, E % 8 == 0): up to 16 workgroups
// per 64-token block so that the blocks fill the chip, at least two 64-deep
// k-steps each.  1 = no split.
inline int route_ksplit(const Problem& p) {
  if (!p.bf16 || p.E % 8 != 0) return 1;
  const int64_t blocks = (p.T + 63) / 64;
  const int64_t kt = p.d / 64;
  int64_t k = 256 / (blocks > 0 ? blocks : 1);
  if (k > 16) k = 16;
  if (k > kt / 2) k = kt / 2;
  return k > 1 ? (int)k : 1;
}
// Bytes of the router's split-k partial scores (0 when there is no split).
inline size_t route_partial_bytes(const Problem& p) {
  const int ks = route_ksplit(p);
  if (ks <= 1) return 0;
  return (size_t)ks * (size_t)p.T * (size_t)(32 * route_nbw(p.E)) * sizeof(float);
}

// Per-block expert counts written by the router for the fused permutation:
// tokens per count block (the selecting workgroup's token block: 64, or 16
// for the split-k finish at more than 64 padded experts), blocks, and the
// row length of the expert-major array blockcnt[E][ld] (a multiple of 4, so
// that rows can be read as 16-byte vectors).  `split` says whether the
// router may split k (moe_route_ws / moe_forward).
inline int route_count_block(const Problem& p, bool split) {
  return (split && route_ksplit(p) > 1 && route_nbw(p.E) >= 4) ? 16 : 64;
}
inline int64_t route_count_blocks(const Problem& p, bool split) {
  const int cb = route_count_block(p, split);
  return (p.T + cb - 1) / cb;
}
inline int64_t route_count_ld(const Problem& p, bool split) {
  return (route_count_blocks(p, split) + 3) / 4 * 4;
}
inline size_t route_count_bytes(const Problem& p, bool split) {
  return (size_t)p.E * (size_t)route_count_ld(p, split) * sizeof(int32_t);
}

// partial: route_partial_bytes(p) of workspace, or NULL (no k split).
// blockcnt (or NULL): receives the per-block expert counts described above.
hipError_t launch_route(const Problem& p, const void* X, const void* W_r, const float* bias,
                        float* logits, int32_t* ids, float* gates, float* partial, hipStream_t s,
                        int32_t* blockcnt = nullptr);
// The fp32 scores X W1 and X W2 of the same bf16 tokens in one launch (no
// bias, no selection); both widths must be multiples of 8 and at most 256.
// When the token blocks alone would leave CUs idle, each axis wider than 128
// is computed by two groups of workgroups (128 columns each).  zero
// (optional): zero_n int32s that the launch also clears.
bool route_pair_supported(int E1, int E2);
hipError_t launch_logits_pair(int64_t T, int d, int E1, int E2, const void* X, const void* W1,
                              const void* W2, float* logits1, float* logits2, hipStream_t s,
                              int32_t* zero = nullptr, int zero_n = 0);

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
// The whole permutation in one workgroup when permute_blocks(p.T) == 1
// (outputs identical to histogram + scan + scatter; table may be NULL).
hipError_t launch_permute_one_block(const Problem& p, const int32_t* ids, int32_t* raw,
                                   int32_t* counts, int32_t* offsets, int32_t* table,
                                   int32_t* perm, int32_t* inv, hipStream_t s);

// The whole permutation after a router that wrote per-block expert counts
// (blockcnt, cb tokens per block, row length ld): one launch of 256-token
// workgroups, each reducing the counts of the blocks before it (no global
// atomics) and ranking its own tokens with an LDS bitmask.  Outputs are
// those of histogram + scan + scatter.  With T <= 256 blockcnt is not read
// (may be NULL).  table may be NULL.
constexpr int kFusedPermuteTokens = 256;
hipError_t launch_permute_fused(const Problem& p, const int32_t* ids, const int32_t* blockcnt,
                                int cb, int64_t ld, int32_t* raw, int32_t* counts,
                                int32_t* offsets, int32_t* table, int32_t* perm, int32_t* inv,
                                hipStream_t s);

// Static device scratch of the allocation-free permutation entry point
// (permute.hip): its address on the current device, looked up once per
// device with hipGetSymbolAddress and kept.
constexpr size_t kNoallocScratchBytes = (size_t)2 << 20;
hipError_t noalloc_scratch(void** out);

// Hpre (bf16 only, may be NULL): also store the pre-activations [rows][2n]
// (x W_gate | x W_up) for the backward.  stream_rows (bf16 only, 0 or
// 1..kMaxStreamRows, needs offsets; not with Hpre): the experts with at most
// that many rows are computed by weight-streaming blocks in the same launch
// instead of by their (single, mostly empty) tile.
constexpr int kMaxStreamRows = 64;
hipError_t launch_gemm_up(const Problem& p, const void* X, const int32_t* perm,
                          const int32_t* table, const void* W_gate, const void* W_up, void* H,
                          hipStream_t s, void* Hpre = nullptr, const int32_t* offsets = nullptr,
                          int stream_rows = 0);
hipError_t launch_gemm_down(const Problem& p, const void* H, const int32_t* table,
                            const void* W_down, void* O, hipStream_t s,
                            const int32_t* offsets = nullptr, int stream_rows = 0);

// Weight-streaming grouped GEMMs for few rows per expert (one workgroup per
// expert and column block; no tile table).
hipError_t launch_gemm_up_skinny(const Problem& p, const void* X, const int32_t* perm,
                                 const int32_t* offsets, const void* W_gate, const void* W_up,
                                 void* H, hipStream_t s);
hipError_t launch_gemm_down_skinny(const Problem& p, const void* H, const int32_t* offsets,
                                   const void* W_down, void* O, hipStream_t s);

// Which grouped-GEMM kernels a bf16 problem runs: the tiled ones, or the
// weight-streaming ones when the batch averages at most kSkinnyRows rows per
// expert (T*K <= kSkinnyRows*E), unless a flag forces one of them.
constexpr int64_t kSkinnyRows = 64;
inline bool use_skinny(const Problem& p, uint32_t flags, uint32_t tiled_flag, uint32_t skinny_flag) {
  if (!p.bf16) return false;
  if (flags & tiled_flag) return false;
  if (flags & skinny_flag) return true;
  return p.T * (int64_t)p.K <= kSkinnyRows * p.E;
}

hipError_t launch_combine(const Problem& p, const void* O, const float* gates,
                          const int32_t* inv_slot, void* Y, hipStream_t s);

// ---------------------------------------------------------------- atomic experts
// Layer of N = Nr*Nc rank-1 experts with a Cartesian-product router (bf16).
struct OmniProblem {
  int64_t T;
  int d, Nr, Nc, K;
};
struct OmniRouteWs {
  float* p_r;           // [T][Nr] raw axis logits
  float* p_c;           // [T][Nc]
  int32_t* ids1;        // [T] scratch of the projection launches
  float* gates1;        // [T]
};
struct OmniPermuteWs {
  int32_t* cursor;      // [N] fill position of each expert's segment
  int32_t* tmp_tk;      // [T*K] entries in arrival order
};
size_t omni_route_ws_bytes(const OmniProblem& p, OmniRouteWs* w, unsigned char* base);
size_t omni_permute_ws_bytes(const OmniProblem& p, OmniPermuteWs* w, unsigned char* base);
// counts (optional): the selection also counts each expert's entries into
// it (cleared first), so that the permutation can skip its own count
// (launch_omni_permute with counted = true).  tpos (optional, with counts):
// [T*K], each entry's place in its expert's arrival order, which lets the
// permutation place entries without atomics.
hipError_t launch_omni_route(const OmniProblem& p, const void* X, const void* W_r, const void* W_c,
                             float* ls_r, float* ls_c, int32_t* ids, float* gates,
                             const OmniRouteWs& w, hipStream_t s, int32_t* counts = nullptr,
                             int32_t* tpos = nullptr);
hipError_t launch_omni_permute(const OmniProblem& p, const int32_t* ids, int32_t* counts,
                               int32_t* offsets, int32_t* perm, int32_t* inv,
                               const OmniPermuteWs& w, hipStream_t s, bool counted = false,
                               const int32_t* tpos = nullptr);
hipError_t launch_omni_experts(const OmniProblem& p, const void* X, const void* W_in,
                               const void* W_out, const int32_t* ids, const float* gates,
                               const int32_t* offsets, const int32_t* perm, const int32_t* inv,
                               float* a, void* Y, hipStream_t s);

// Tile-aware token rounding of permute's metadata, in place (counts, offsets,
// perm_token, inv_slot); M = kGemmBM.
struct RoundWs {
  uint32_t* key;        // [rows] bit pattern of each old slot's gate
  int32_t* slot_tk;     // [rows] flat (token, k) index of each old slot
  int32_t* rank;        // [rows] rank of a surviving slot inside its expert, or -1
  int32_t* old_total;   // [1]    kept rows before the rounding
};
size_t round_ws_bytes(const Problem& p, RoundWs* w, unsigned char* base);
hipError_t launch_round(const Problem& p, const int32_t* ids, const float* gates, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* inv, const RoundWs& w,
                        hipStream_t s);

// ---------------------------------------------------------------- backward (bf16)
// Scratch of the backward, carved from the caller's workspace.
struct BackwardWs {
  float* gs;           // [rows] gate of each kept slot
  float* dS_part;      // [rows][ceil(n/256)] per-tile shares of dS = <dA', A>
  uint16_t* dH;        // [rows][2n] (dHg | dHu)
  uint16_t* gA;        // [rows][n]  g * silu(Hg) * Hu
  uint16_t* dXs;       // [rows][d]  input gradient per slot
  uint16_t* dl;        // [T][Epad]  router-logit gradient (zeros off the selected experts)
  uint16_t* W_rT;      // [E][d]
  uint32_t* zero;      // kZeroBytes of zeros (copy source past a group's end)
  float* dWr_part;     // [ksplit][d][Epad] split-k partials of dW_r
};
constexpr int kZeroBytes = 256;
int bwd_router_ksplit(const Problem& p);
// Bytes of the backward scratch; with base != NULL also carves it into *w.
size_t backward_ws_bytes(const Problem& p, BackwardWs* w, unsigned char* base);
hipError_t launch_zero_grads(const Problem& p, float* dW_r, float* dW_gate, float* dW_up,
                             float* dW_down, hipStream_t s);
hipError_t launch_backward(const Problem& p, const void* X, const void* W_r, const void* W_gate,
                           const void* W_up, const void* W_down, const void* dY,
                           const int32_t* ids, const float* gates, const int32_t* inv,
                           const int32_t* perm, const int32_t* offsets, const int32_t* table,
                           const void* Hpre, void* dX, float* dW_r, float* dW_gate, float* dW_up,
                           float* dW_down, const BackwardWs& w, hipStream_t s);

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

// 1 / (1 + e^-z) with the hardware exp2 and reciprocal (about 1 ulp each;
// a quotient written with '/' or __fdividef compiles to the full IEEE
// division sequence, several times the instructions and registers).
// z -> -inf gives 1/inf = 0.
__device__ __forceinline__ float sigmoid(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Workgroup barrier without the memory fence that __syncthreads adds (the
// fence would also wait for in-flight global->LDS prefetches).  The memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// 16-byte global -> LDS copy per lane; LDS destination = M0 + 16*lane, so a
// wave fills 1 KB at lds_addr (wave-uniform).  Issued through asm so the
// compiler does not treat later LDS reads as aliasing the copy (it would wait
// for every copy in flight); completion is awaited with explicit s_waitcnt
// vmcnt.  The asm has no register outputs; s_nop covers the M0-write ->
// LDS-DMA hazard.  M0 is written only by these copies in the kernels that
// use them, so clobbering it is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_addr)
               : "memory", "m0");
}
// The same copy with the non-temporal hint, for data read once (a stream
// through the cache should not evict what other workgroups re-read).
__device__ __forceinline__ void lds_copy16_stream(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(g), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace dev
}  // namespace moe
#endif
