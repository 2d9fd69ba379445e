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
// Three launches over metadata that moe_permute wrote:
//   select   one workgroup per expert: gathers the gate of each of its slots
//            (cached in LDS), finds the D-th smallest gate by a 4-pass radix
//            select on the gates' bit patterns (non-negative floats order as
//            their bits), then one ordered sweep assigns each surviving slot
//            its rank inside the segment; writes the new count, a copy of
//            the segment's perm_token and the slot's expert;
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

// Bit pattern of the gate of (token t, expert e): the entry of t's list that
// holds e (the router lists distinct experts).
__device__ __forceinline__ uint32_t gate_key(const int32_t* ids, const float* gates, int64_t t,
                                             int K, int e) {
  const int32_t* row = ids + t * K;
  int k = 0;
  for (int j = 0; j < K; ++j)
    if (row[j] == e) { k = j; break; }
  return __float_as_uint(gates[t * K + k]);
}

// Exclusive scan of one value per thread over the 256 threads; returns the
// prefix, *total the sum.  Every thread calls it.
__device__ int wg_exscan(int v, int* lds, int* total) {
  const int tid = threadIdx.x;
  lds[tid] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int x = tid >= off ? lds[tid - off] : 0;
    __syncthreads();
    lds[tid] += x;
    __syncthreads();
  }
  const int incl = lds[tid];
  *total = lds[kThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kThreads) void round_select_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ gates,
    int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, int32_t* __restrict__ rank, int32_t* __restrict__ perm_old,
    int32_t* __restrict__ slot_e, int64_t T, int K) {
  __shared__ uint32_t keys[kCacheKeys];
  __shared__ int hist[256];
  __shared__ int scan_tmp[kThreads];
  __shared__ int bcast[2];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const int off = offsets[e];
  const int c = offsets[e + 1] - off;
  const int r = rounded(c);
  const int D = c - r;                            // assignments to drop (0 <= D < M/2)
  const bool cached = c <= kCacheKeys;
  for (int i = tid; i < c; i += kThreads) {
    const int t = perm[off + i];
    perm_old[off + i] = t;
    slot_e[off + i] = e;
    if (D > 0 && cached) keys[i] = gate_key(ids, gates, t, K, e);
  }
  if (tid == 0) counts[e] = r;
  if (D == 0) {
    for (int i = tid; i < c; i += kThreads) rank[off + i] = i;
    return;
  }
  __syncthreads();
  auto key_at = [&](int i) -> uint32_t {
    return cached ? keys[i] : gate_key(ids, gates, perm[off + i], K, e);
  };

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
    if (tid == 0) {
      int cum = 0, b = 0;
      for (; b < 255; ++b) {
        if (cum + hist[b] >= want) break;
        cum += hist[b];
      }
      bcast[0] = b;
      bcast[1] = want - cum;
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
    const int is_tie = (i < c && k == prefix) ? 1 : 0;
    int tie_total = 0;
    const int tie_idx = tie_base + wg_exscan(is_tie, scan_tmp, &tie_total);
    const int keep = (i < c && (k > prefix || (is_tie && tie_idx < keep_ties))) ? 1 : 0;
    int kept_total = 0;
    const int kr = kept_base + wg_exscan(keep, scan_tmp, &kept_total);
    if (i < c) rank[off + i] = keep ? kr : -1;
    tie_base += tie_total;
    kept_base += kept_total;
  }
}

__global__ __launch_bounds__(kThreads) void round_offsets_kernel(const int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ old_total,
                                                                 int E) {
  __shared__ int tmp[kThreads];
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
    const int32_t* __restrict__ perm_old, const int32_t* __restrict__ slot_e,
    const int32_t* __restrict__ old_total, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int64_t rows, int K) {
  const int64_t s = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (s >= rows || s >= old_total[0]) return;
  const int e = slot_e[s];
  const int t = perm_old[s];
  const int r = rank[s];
  int k = 0;
  for (int j = 0; j < K; ++j)
    if (ids[(int64_t)t * K + j] == e) { k = j; break; }
  int ns = -1;
  if (r >= 0) {
    ns = offsets[e] + r;
    perm[ns] = t;
  }
  inv[(int64_t)t * K + k] = ns;
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
  ws.rank = reinterpret_cast<int32_t*>(take(rows * 4));
  ws.perm_old = reinterpret_cast<int32_t*>(take(rows * 4));
  ws.slot_e = reinterpret_cast<int32_t*>(take(rows * 4));
  ws.old_total = reinterpret_cast<int32_t*>(take(4));
  if (w) *w = ws;
  return off;
}

hipError_t launch_round(const Problem& p, const int32_t* ids, const float* gates, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* inv, const RoundWs& w,
                        hipStream_t s) {
  hipLaunchKernelGGL(round_select_kernel, dim3((unsigned)p.E), dim3(kThreads), 0, s, ids, gates,
                     counts, offsets, perm, w.rank, w.perm_old, w.slot_e, p.T, p.K);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(round_offsets_kernel, dim3(1), dim3(kThreads), 0, s, counts, offsets,
                     w.old_total, p.E);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t rows = p.rows_max;
  hipLaunchKernelGGL(round_scatter_kernel, dim3((unsigned)((rows + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, ids, w.rank, w.perm_old, w.slot_e, w.old_total,
                     offsets, perm, inv, rows, p.K);
  return hipGetLastError();
}

}  // namespace moe
