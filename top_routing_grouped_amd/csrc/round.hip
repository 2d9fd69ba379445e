// Tile-aware token rounding of the expert-major metadata (SonicMoE article
// §6.5: routing aware of the grouped GEMM's row tile, so that per-expert
// counts sit on tile multiples and fewer padded rows are computed).
//
// Rule (the page gives none; this is the reading the library documents):
// an expert with c >= M kept rows and c mod M < M/2 keeps M*floor(c/M) of
// them, dropping its lowest-gate assignments (equal gates: the larger token
// first); other experts are left alone.  M = kGemmBM, the tiled GEMM's row
// tile.  Dropped assignments become inv_slot = -1 exactly like capacity
// drops, and each expert's surviving slots keep ascending token order.
//
// Four launches over metadata that moe_permute wrote:
//   keys     one thread per (token, k): a kept entry writes its gate's bit
//            pattern and its (token, k) index at its slot (coalesced reads);
//   select   one workgroup per expert: reads its segment's keys (cached in
//            LDS), finds the D-th smallest by a 4-pass radix select on the
//            bit patterns (non-negative floats order as their bits; each
//            pass an LDS histogram and a scan of its 256 bins), then
//            one ordered sweep with wave-ballot prefix counts gives each
//            surviving slot its rank inside the segment; writes the count;
//   offsets  one workgroup: exclusive scan of the new counts;
//   scatter  one thread per old slot: moves survivors to their new slot and
//            rewrites inv_slot (the new slot, or -1).
// Deterministic: no atomics on global memory, LDS histograms only count.
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kCacheKeys = 15360;        // segment gates kept in LDS (60 KB; static LDS stays below 64 KB)

__device__ __forceinline__ int rounded(int c) {
  return (c >= kGemmBM && (c % kGemmBM) < kGemmBM / 2) ? c - c % kGemmBM : c;
}

// Exclusive prefix count of `flag` over the workgroup's 256 threads, and the
// total: a ballot per wave, then the 4 wave totals through LDS.
__device__ int wg_count_prefix(bool flag, int* lds, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) lds[w] = __popcll(m);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int j = 0; j < kThreads / 64; ++j) {
    const int v = lds[j];
    tot += v;
    before += j < w ? v : 0;
  }
  __syncthreads();                      // lds is reused by the next call
  *total = tot;
  return before + in_wave;
}

// Exclusive scan of one value per thread over the 256 threads; returns the
// prefix, *total the sum.  Every thread calls it.  Shuffles inside a wave,
// then the 4 wave totals through LDS.
__device__ int wg_exscan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    x += lane >= o ? y : 0;
  }
  if (lane == 63) lds[w] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int j = 0; j < kThreads / 64; ++j) {
    const int t = lds[j];
    tot += t;
    before += j < w ? t : 0;
  }
  __syncthreads();                      // lds is reused by the next call
  *total = tot;
  return before + x - v;
}

__global__ __launch_bounds__(kThreads) void round_keys_kernel(const float* __restrict__ gates,
                                                              const int32_t* __restrict__ inv,
                                                              uint32_t* __restrict__ key,
                                                              int32_t* __restrict__ slot_tk,
                                                              int64_t TK) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= TK) return;
  const int s = inv[i];
  if (s < 0) return;
  key[s] = __float_as_uint(gates[i]);
  slot_tk[s] = (int32_t)i;
}

__global__ __launch_bounds__(kThreads) void round_select_kernel(
    int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const uint32_t* __restrict__ key, int32_t* __restrict__ rank) {
  __shared__ uint32_t keys[kCacheKeys];
  __shared__ int hist[256];
  __shared__ int red[kThreads / 64];
  __shared__ int bcast[2];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const int off = offsets[e];
  const int c = offsets[e + 1] - off;
  const int r = rounded(c);
  const int D = c - r;                            // assignments to drop (0 <= D < M/2)
  if (tid == 0) counts[e] = r;
  if (D == 0) {
    for (int i = tid; i < c; i += kThreads) rank[off + i] = i;
    return;
  }
  const bool cached = c <= kCacheKeys;
  if (cached)
    for (int i = tid; i < c; i += kThreads) keys[i] = key[off + i];
  __syncthreads();
  auto key_at = [&](int i) -> uint32_t { return cached ? keys[i] : key[off + i]; };

  // radix select: the D-th smallest key (1-based), 8 bits per pass
  uint32_t prefix = 0, mask = 0;
  int want = D, ties = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < c; i += kThreads) {
      const uint32_t k = key_at(i);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
    }
    __syncthreads();
    // the bin holding the want-th key: the one thread whose prefix range
    // [excl, excl + hist) contains it
    int unused = 0;
    const int h = hist[tid];
    const int excl = wg_exscan(h, red, &unused);
    if (excl < want && want <= excl + h) {
      bcast[0] = tid;
      bcast[1] = want - excl;
    }
    __syncthreads();
    const int b = bcast[0];
    want = bcast[1];
    ties = hist[b];
    prefix |= (uint32_t)b << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  // prefix = the threshold key v; keys below it are dropped, and of the
  // `ties` keys equal to it the last `want` (largest slots) are dropped too
  const int keep_ties = ties - want;
  int tie_base = 0, kept_base = 0;
  for (int i0 = 0; i0 < c; i0 += kThreads) {
    const int i = i0 + tid;
    const uint32_t k = i < c ? key_at(i) : 0u;
    const bool is_tie = i < c && k == prefix;
    int tie_total = 0;
    const int tie_idx = tie_base + wg_count_prefix(is_tie, red, &tie_total);
    const bool keep = i < c && (k > prefix || (is_tie && tie_idx < keep_ties));
    int kept_total = 0;
    const int kr = kept_base + wg_count_prefix(keep, red, &kept_total);
    if (i < c) rank[off + i] = keep ? kr : -1;
    tie_base += tie_total;
    kept_base += kept_total;
  }
}

__global__ __launch_bounds__(kThreads) void round_offsets_kernel(const int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ old_total,
                                                                 int E) {
  __shared__ int tmp[kThreads / 64];
  const int tid = threadIdx.x;
  const int before = offsets[E];
  int total = 0;
  const int ex = wg_exscan(tid < E ? counts[tid] : 0, tmp, &total);
  if (tid < E) offsets[tid] = ex;
  if (tid == 0) {
    offsets[E] = total;
    old_total[0] = before;
  }
}

__global__ __launch_bounds__(kThreads) void round_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ slot_tk, const int32_t* __restrict__ old_total,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int64_t rows, int K) {
  const int64_t s = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (s >= rows || s >= old_total[0]) return;
  const int tk = slot_tk[s];
  const int r = rank[s];
  int ns = -1;
  if (r >= 0) {
    ns = offsets[ids[tk]] + r;
    perm[ns] = tk / K;
  }
  inv[tk] = ns;
}

}  // namespace

size_t round_ws_bytes(const Problem& p, RoundWs* w, unsigned char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* ptr = base ? base + off : nullptr;
    off += (bytes + 255) / 256 * 256;
    return ptr;
  };
  const size_t rows = (size_t)(p.rows_max > 0 ? p.rows_max : 1);
  RoundWs ws{};
  ws.key = reinterpret_cast<uint32_t*>(take(rows * 4));
  ws.slot_tk = reinterpret_cast<int32_t*>(take(rows * 4));
  ws.rank = reinterpret_cast<int32_t*>(take(rows * 4));
  ws.old_total = reinterpret_cast<int32_t*>(take(4));
  if (w) *w = ws;
  return off;
}

hipError_t launch_round(const Problem& p, const int32_t* ids, const float* gates, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* inv, const RoundWs& w,
                        hipStream_t s) {
  const int64_t TK = p.T * (int64_t)p.K;
  hipLaunchKernelGGL(round_keys_kernel, dim3((unsigned)((TK + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, gates, inv, w.key, w.slot_tk, TK);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(round_select_kernel, dim3((unsigned)p.E), dim3(kThreads), 0, s, counts,
                     offsets, w.key, w.rank);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(round_offsets_kernel, dim3(1), dim3(kThreads), 0, s, counts, offsets,
                     w.old_total, p.E);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t rows = p.rows_max;
  hipLaunchKernelGGL(round_scatter_kernel, dim3((unsigned)((rows + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, ids, w.rank, w.slot_tk, w.old_total, offsets, perm,
                     inv, rows, p.K);
  return hipGetLastError();
}

}  // namespace moe
