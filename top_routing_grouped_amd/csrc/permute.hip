// Steps 3-5 of the layer: expert-major metadata from the [T, K] top-K ids.
//
// SonicMoE article §11 lists the metadata a grouped GEMM consumes (tokens per
// expert, expert-major slot -> token, token-major entry -> expert-major slot)
// and the counting / prefix-sum / scatter-index steps that build it;
// "算子与编译器：MoE 路由与稀疏 Kernel" §3 names counting and prefix sums as
// the core of the permutation and §4 the per-expert capacity; the OmniMoE page
// (§2.3, §3.3) orders the (token, expert) work by (expert, token).
//
// Three launches, none with atomics on global memory:
//   histogram  one workgroup per block of 256 tokens counts that block's
//              choices per expert in LDS -> blockcnt[block][expert];
//   scan       one workgroup scans blockcnt over blocks (per expert, token
//              order) -> blockbase, raw counts, capped counts, offsets, and
//              optionally the grouped-GEMM tile table;
//   scatter    one workgroup per block rebuilds the block's per-expert token
//              bitmask in LDS; a token's rank inside its expert is blockbase
//              plus the popcount of the mask bits below it, so the rank is
//              the token-order rank without any ordering atomics; kept
//              entries (rank < C) write perm_token and inv_slot.
// With at most 256 tokens (one block) the three steps run in one workgroup
// and one launch (decode batches: 18 -> 10 us at T = 64).
#include "moe_internal.hpp"

#include <mutex>

// Scratch of the allocation-free entry point (moe_permute_noalloc): the
// per-block histogram, block bases and raw counts that moe_permute keeps in
// the caller's workspace.  Each GPU the library runs on holds its own copy
// at its own address until the process ends.  In host code this name is
// only a stand-in for the symbol; the device address comes from
// noalloc_scratch() below and is the only form ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[moe::kNoallocScratchBytes];

namespace moe {

hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

namespace {

constexpr int kB = kPermuteBlock;        // tokens per block (== threads)
constexpr int kWords = kB / 32;          // bitmask words per expert
constexpr int kScanThreads = 1024;
constexpr int kChunk = 8;                // ids loaded per round trip

__global__ __launch_bounds__(kB) void histogram_kernel(const int32_t* __restrict__ ids,
                                                       int32_t* __restrict__ blockcnt, int64_t T,
                                                       int E, int K) {
  __shared__ int cnt[256];
  for (int e = threadIdx.x; e < E; e += kB) cnt[e] = 0;
  __syncthreads();
  const int64_t tb = (int64_t)blockIdx.x * kB;
  const int64_t ntok = (T - tb < kB) ? (T - tb) : kB;
  const int64_t nid = ntok * K;
  const int32_t* base = ids + tb * K;
  // kChunk independent loads per round trip (a load feeding a branch is
  // otherwise waited for before the next one is issued)
  for (int64_t j0 = 0; j0 < nid; j0 += (int64_t)kB * kChunk) {
    int ee[kChunk];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int64_t j = j0 + threadIdx.x + (int64_t)kB * c;
      ee[c] = j < nid ? base[j] : -1;
    }
#pragma unroll
    for (int c = 0; c < kChunk; ++c)
      if (ee[c] >= 0 && ee[c] < E) atomicAdd(&cnt[ee[c]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kB) blockcnt[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// Exclusive scan over the first n (<= 256) threads' values; all threads of
// the block must call it.  Returns the exclusive prefix; *total gets the sum.
__device__ int block_exscan256(int v, int n, int* lds, int* total) {
  const int tid = threadIdx.x;
  if (tid < 256) lds[tid] = (tid < n) ? v : 0;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int x = 0;
    if (tid < 256 && tid >= off) x = lds[tid - off];
    __syncthreads();
    if (tid < 256) lds[tid] += x;
    __syncthreads();
  }
  const int incl = (tid < 256) ? lds[tid] : 0;
  *total = lds[255];
  __syncthreads();
  return incl - ((tid < n) ? v : 0);
}

// Row tiles of one expert: rows [off, off+cnt) cut into BM-row pieces.
__device__ void write_tiles(int e, int off, int cnt, int start, int64_t max_tiles,
                            int32_t* __restrict__ table) {
  const int nt = (cnt + kGemmBM - 1) / kGemmBM;
  for (int i = 0; i < nt; ++i) {
    const int64_t idx = (int64_t)start + i;
    if (idx >= max_tiles) break;
    int32_t* ent = table + 4 * (idx + 1);
    const int rb = off + i * kGemmBM;
    const int re = (rb + kGemmBM < off + cnt) ? rb + kGemmBM : off + cnt;
    ent[0] = (int32_t)((uint32_t)e | ((uint32_t)nt << 8));
    ent[1] = rb;
    ent[2] = re;
    ent[3] = start;
  }
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const int32_t* __restrict__ blockcnt, int32_t* __restrict__ blockbase,
    int32_t* __restrict__ raw, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ table, int64_t max_tiles, int NB, int E, int64_t C) {
  __shared__ int part[kScanThreads];
  __shared__ int tmp[256];
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  const int P = kScanThreads / Ep;            // block ranges per expert
  const int tid = threadIdx.x;
  const int e = tid % Ep, q = tid / Ep;
  const int per = (NB + P - 1) / P;
  const int b0 = q * per;
  const int b1 = (b0 + per < NB) ? b0 + per : NB;
  int s = 0;
  if (e < E)
    for (int b = b0; b < b1; ++b) s += blockcnt[(int64_t)b * E + e];
  part[tid] = s;
  __syncthreads();
  if (tid < Ep && e < E) {                    // q == 0: scan the P partial sums
    int run = 0;
    for (int qq = 0; qq < P; ++qq) {
      const int v = part[qq * Ep + e];
      part[qq * Ep + e] = run;
      run += v;
    }
    raw[e] = run;
    tmp[e] = run;                             // carried to the expert scan
  }
  __syncthreads();
  if (e < E) {
    int run = part[tid];
    for (int b = b0; b < b1; ++b) {
      const int64_t at = (int64_t)b * E + e;
      const int v = blockcnt[at];
      blockbase[at] = run;
      run += v;
    }
  }
  // counts, offsets (exclusive scan over experts), tile table
  int kept = 0;
  if (tid < E) {
    const int r = tmp[tid];
    kept = ((int64_t)r < C) ? r : (int)C;
  }
  __syncthreads();
  int total = 0;
  const int off = block_exscan256(kept, E, tmp, &total);
  if (tid < E) {
    counts[tid] = kept;
    offsets[tid] = off;
  }
  if (tid == 0) offsets[E] = total;
  if (table) {
    const int nt = (tid < E) ? (kept + kGemmBM - 1) / kGemmBM : 0;
    int ntiles = 0;
    const int start = block_exscan256(nt, E, tmp, &ntiles);
    if (tid < E) write_tiles(tid, off, kept, start, max_tiles, table);
    if (tid == 0) {
      table[0] = (int64_t)ntiles < max_tiles ? ntiles : (int)max_tiles;
      table[1] = table[2] = table[3] = 0;
    }
  }
}

__global__ __launch_bounds__(kB) void scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ blockbase,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int64_t T, int E, int K, int64_t C) {
  __shared__ uint32_t bits[256 * kWords];
  for (int j = threadIdx.x; j < E * kWords; j += kB) bits[j] = 0u;
  __syncthreads();
  const int tid = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * kB + tid;
  const bool valid = t < T;
  const int w = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  // a token's ids in chunks of kChunk independent loads, then per chunk the
  // block bases and offsets of those experts (independent again)
  if (valid)
    for (int k0 = 0; k0 < K; k0 += kChunk) {
      int ee[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; ++c) ee[c] = (k0 + c < K) ? ids[t * K + k0 + c] : -1;
#pragma unroll
      for (int c = 0; c < kChunk; ++c)
        if (ee[c] >= 0 && ee[c] < E) atomicOr(&bits[ee[c] * kWords + w], bit);
    }
  __syncthreads();
  if (!valid) return;
  for (int k0 = 0; k0 < K; k0 += kChunk) {
    int ee[kChunk], bb[kChunk], oo[kChunk];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) ee[c] = (k0 + c < K) ? ids[t * K + k0 + c] : -1;
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const bool ok = ee[c] >= 0 && ee[c] < E;
      bb[c] = ok ? blockbase[(int64_t)blockIdx.x * E + ee[c]] : 0;
      oo[c] = ok ? offsets[ee[c]] : 0;
    }
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      if (k0 + c >= K) break;
      const int e = ee[c];
      int32_t slot = -1;
      if (e >= 0 && e < E) {
        const uint32_t* m = bits + e * kWords;
        int below = __popc(m[w] & (bit - 1u));
        for (int ww = 0; ww < w; ++ww) below += __popc(m[ww]);
        const int64_t rank = (int64_t)bb[c] + below;
        if (rank < C) {
          slot = (int32_t)(oo[c] + rank);
          perm[slot] = (int32_t)t;
        }
      }
      inv[t * K + k0 + c] = slot;
    }
  }
}

// All tokens in one block (T <= 256, decode-sized batches): the three steps
// above in one workgroup, with the same definitions -- counts from an LDS
// histogram, the block's base ranks all zero, ranks from the expert's token
// bitmask -- so the outputs are those of the three-launch path, in one
// launch instead of three.
__global__ __launch_bounds__(kB) void permute_one_block_kernel(
    const int32_t* __restrict__ ids, int32_t* __restrict__ raw, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ table, int64_t max_tiles,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int64_t T, int E, int K, int64_t C) {
  __shared__ uint32_t bits[256 * kWords];
  __shared__ int cnt[256];
  __shared__ int offs[256];
  __shared__ int tmp[256];
  const int tid = threadIdx.x;
  for (int j = tid; j < E * kWords; j += kB) bits[j] = 0u;
  if (tid < 256) cnt[tid] = 0;
  __syncthreads();
  const bool valid = tid < T;
  const int w = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  if (valid)
    for (int k0 = 0; k0 < K; k0 += kChunk) {
      int ee[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; ++c) ee[c] = (k0 + c < K) ? ids[(int64_t)tid * K + k0 + c] : -1;
#pragma unroll
      for (int c = 0; c < kChunk; ++c)
        if (ee[c] >= 0 && ee[c] < E) {
          atomicAdd(&cnt[ee[c]], 1);
          atomicOr(&bits[ee[c] * kWords + w], bit);
        }
    }
  __syncthreads();
  const int r = (tid < E) ? cnt[tid] : 0;
  const int kept = ((int64_t)r < C) ? r : (int)C;
  int total = 0;
  const int off = block_exscan256(kept, E, tmp, &total);
  if (tid < E) {
    raw[tid] = r;
    counts[tid] = kept;
    offsets[tid] = off;
    offs[tid] = off;
  }
  if (tid == 0) offsets[E] = total;
  if (table) {
    const int nt = (tid < E) ? (kept + kGemmBM - 1) / kGemmBM : 0;
    int ntiles = 0;
    const int start = block_exscan256(nt, E, tmp, &ntiles);
    if (tid < E) write_tiles(tid, off, kept, start, max_tiles, table);
    if (tid == 0) {
      table[0] = (int64_t)ntiles < max_tiles ? ntiles : (int)max_tiles;
      table[1] = table[2] = table[3] = 0;
    }
  }
  __syncthreads();                            // offs complete
  if (!valid) return;
  for (int k0 = 0; k0 < K; k0 += kChunk) {
    int ee[kChunk];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) ee[c] = (k0 + c < K) ? ids[(int64_t)tid * K + k0 + c] : -1;
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      if (k0 + c >= K) break;
      const int e = ee[c];
      int32_t slot = -1;
      if (e >= 0 && e < E) {
        const uint32_t* m = bits + e * kWords;
        int below = __popc(m[w] & (bit - 1u));
        for (int ww = 0; ww < w; ++ww) below += __popc(m[ww]);
        if ((int64_t)below < C) {
          slot = (int32_t)(offs[e] + below);
          perm[slot] = tid;
        }
      }
      inv[(int64_t)tid * K + k0 + c] = slot;
    }
  }
}

__global__ __launch_bounds__(256) void tile_table_kernel(const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ table,
                                                         int64_t max_tiles, int64_t rows_max,
                                                         int E) {
  __shared__ int tmp[256];
  const int tid = threadIdx.x;
  int off = 0, cnt = 0;
  if (tid < E) {
    off = offsets[tid];
    int end = offsets[tid + 1];
    if (off < 0) off = 0;
    if ((int64_t)end > rows_max) end = (int)rows_max;
    cnt = end > off ? end - off : 0;
  }
  const int nt = (cnt + kGemmBM - 1) / kGemmBM;
  int ntiles = 0;
  const int start = block_exscan256(nt, E, tmp, &ntiles);
  if (tid < E) write_tiles(tid, off, cnt, start, max_tiles, table);
  if (tid == 0) {
    table[0] = (int64_t)ntiles < max_tiles ? ntiles : (int)max_tiles;
    table[1] = table[2] = table[3] = 0;
  }
}

}  // namespace

hipError_t launch_histogram(const Problem& p, const int32_t* ids, int32_t* blockcnt,
                            hipStream_t s) {
  hipLaunchKernelGGL(histogram_kernel, dim3((unsigned)permute_blocks(p.T)), dim3(kB), 0, s, ids,
                     blockcnt, p.T, p.E, p.K);
  return hipGetLastError();
}

hipError_t launch_scan(const Problem& p, const int32_t* blockcnt, int32_t* blockbase,
                       int32_t* raw, int32_t* counts, int32_t* offsets, int32_t* table,
                       hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, blockcnt, blockbase, raw,
                     counts, offsets, table, max_row_tiles(p, kGemmBM), (int)permute_blocks(p.T),
                     p.E, p.C);
  return hipGetLastError();
}

hipError_t launch_scatter(const Problem& p, const int32_t* ids, const int32_t* blockbase,
                          const int32_t* offsets, int32_t* perm, int32_t* inv_slot,
                          hipStream_t s) {
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)permute_blocks(p.T)), dim3(kB), 0, s, ids,
                     blockbase, offsets, perm, inv_slot, p.T, p.E, p.K, p.C);
  return hipGetLastError();
}

hipError_t launch_permute_one_block(const Problem& p, const int32_t* ids, int32_t* raw,
                                   int32_t* counts, int32_t* offsets, int32_t* table,
                                   int32_t* perm, int32_t* inv, hipStream_t s) {
  hipLaunchKernelGGL(permute_one_block_kernel, dim3(1), dim3(kB), 0, s, ids, raw, counts, offsets,
                     table, max_row_tiles(p, kGemmBM), perm, inv, p.T, p.E, p.K, p.C);
  return hipGetLastError();
}

hipError_t launch_tile_table(const Problem& p, const int32_t* offsets, int32_t* table,
                             hipStream_t s) {
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(256), 0, s, offsets, table,
                     max_row_tiles(p, kGemmBM), p.rows_max, p.E);
  return hipGetLastError();
}

}  // namespace moe
