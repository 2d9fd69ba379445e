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
// the block (at least 256) must call it.  Returns the exclusive prefix (0 for threads from
// 256 on); *total gets the sum.  Each of the first four waves scans its 64
// values with lane shuffles, then adds the totals of the waves before it
// (two barriers, where a scan through LDS in 8 rounds took 18).
__device__ int block_exscan256(int v, int n, int* lds, int* total) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int own = (tid < n) ? v : 0;
  int x = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (wv < 4 && lane == 63) lds[wv] = x;
  __syncthreads();
  int base = 0;
  for (int j = 0; j < wv && j < 4; ++j) base += lds[j];
  *total = ((lds[0] + lds[1]) + lds[2]) + lds[3];
  __syncthreads();                      // the caller may reuse lds
  return (wv < 4) ? x + base - own : 0;
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

// First table entry of each expert's row tiles.  The grouped GEMMs give each
// XCD a contiguous range of the table, so in expert order the most loaded
// experts of a skewed router would all fall to the first XCDs (the Zipf-biased
// layer: the nine experts capped at 640 rows on two of eight).  Instead the
// experts, sorted by tile count (descending; ties by id), are dealt in a snake
// over 8 lanes (0..7, 7..0, ...), and the table lists lane 0's experts, then
// lane 1's, ...: every XCD's range gets a similar mix of heavy and light
// experts, heavy ones first, while each expert's tiles stay contiguous.
// All threads of the workgroup (at least 256) must call it; threads below E
// pass their expert's tile count and get its first entry; *ntiles = total.
__device__ int tile_starts(int nt, int E, int* cnt_s, int* ord_s, int* pref_s, int* tmp,
                           int* ntiles) {
  const int tid = threadIdx.x;
  if (tid < 256) {
    cnt_s[tid] = (tid < E) ? nt : 0;
    ord_s[tid] = -1;
  }
  __syncthreads();
  int key = 0;
  if (tid < E) {
    int rank = 0;
    for (int j = 0; j < E; ++j) {
      const int c = cnt_s[j];
      rank += (c > nt) || (c == nt && j < tid);
    }
    const int round = rank >> 3, pos = rank & 7;
    const int lane = (round & 1) ? 7 - pos : pos;
    key = lane * 32 + round;                  // rounds <= 32 for E <= 256
    ord_s[key] = tid;
  }
  __syncthreads();
  const int v = (tid < 256 && ord_s[tid] >= 0) ? cnt_s[ord_s[tid]] : 0;
  const int pref = block_exscan256(v, 256, tmp, ntiles);
  if (tid < 256) pref_s[tid] = pref;
  __syncthreads();
  return (tid < E) ? pref_s[key] : 0;
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const int32_t* __restrict__ blockcnt, int32_t* __restrict__ blockbase,
    int32_t* __restrict__ raw, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ table, int64_t max_tiles, int NB, int E, int64_t C) {
  __shared__ int part[kScanThreads];
  __shared__ int tmp[256];
  __shared__ int tcnt_s[256], tord_s[256], tpref_s[256];   // tile_starts scratch
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
    const int start = tile_starts(nt, E, tcnt_s, tord_s, tpref_s, tmp, &ntiles);
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
  __shared__ int tcnt_s[256], tord_s[256], tpref_s[256];   // tile_starts scratch
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
    const int start = tile_starts(nt, E, tcnt_s, tord_s, tpref_s, tmp, &ntiles);
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

// The fused permutation (after a router that wrote per-block expert counts).
// One workgroup of 1024 threads per 256 tokens:
//   1. every wave sums whole rows of the router's expert-major counts
//      blockcnt[E][ld] (64 lanes x 16-byte loads = 256 blocks per load, eight
//      rows in flight), split at this workgroup's first token: base[e] =
//      assignments to e from earlier tokens, total[e] = all of them;
//   2. counts = min(total, C), offsets = exclusive scan (workgroup 0 writes
//      raw counts, counts, offsets and the tile table);
//   3. the first 256 threads (one token each) set bits in an LDS bitmask per
//      expert (256 bits = 8 words), an 8-lane scan turns the words' popcounts
//      into exclusive prefixes, and a token's rank inside expert e is base[e]
//      plus the prefix of its word plus the popcount of the lower bits of its
//      word.  A workgroup's kept tokens of expert e fill one contiguous run of
//      slots, so (for K <= 32) the tokens are staged in LDS by expert and each
//      run is stored by consecutive lanes instead of one 4-byte store per
//      (token, k) to a random slot.
// Same definitions as histogram + scan + scatter, so the same outputs.
constexpr int kFT = kFusedPermuteTokens;   // tokens per workgroup
constexpr int kFThreads = 1024;
constexpr int kFWords = kFT / 32;
constexpr int kFRows = 8;                  // rows of counts in flight per wave
constexpr int kFStageK = 32;               // largest K whose slots are staged in LDS

// Sum over the 64 lanes of a wave, returned to every lane: DPP steps inside
// each 16-lane row (lane pairs, quads, half-row mirror, row mirror), then the
// four row sums read out with readlane (no LDS round trips).
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ int wave_sum(int x) {
  x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);   // row_half_mirror
  x += dpp_mov<0x140>(x);   // row_mirror
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
         __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}

__global__ __launch_bounds__(kFThreads) void permute_fused_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ blockcnt, int cb, int64_t ld,
    int64_t nbc, int32_t* __restrict__ raw, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ table, int64_t max_tiles,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int64_t T, int E, int K, int64_t C) {
  __shared__ uint32_t bits[256 * kFWords];
  __shared__ int pre[256 * kFWords];
  __shared__ int base_s[256];
  __shared__ int tot_s[256];
  __shared__ int offs_s[256];
  __shared__ int lst_s[256];                // start of each expert's run in stage[]
  __shared__ int tmp[256];
  __shared__ int tcnt_s[256], tord_s[256], tpref_s[256];   // tile_starts scratch
  __shared__ int stage[kFT * kFStageK];     // kept tokens, grouped by expert
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  constexpr int kWaves = kFThreads / 64;
  const int64_t t0 = (int64_t)blockIdx.x * kFT;
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  for (int j = tid; j < Ep * kFWords; j += kFThreads) bits[j] = 0u;

  // 1. counts of the blocks before this workgroup, and of all blocks, per expert
  if (gridDim.x > 1) {
    using i4 = int __attribute__((ext_vector_type(4)));
    const int64_t bfirst = t0 / cb;           // a multiple of 4
    const int64_t nchunk = (nbc + 255) / 256;
    for (int e0 = wave; e0 < E; e0 += kWaves * kFRows) {
      int bef[kFRows], tot[kFRows];
#pragma unroll
      for (int r = 0; r < kFRows; ++r) bef[r] = tot[r] = 0;
      for (int64_t c = 0; c < nchunk; ++c) {
        const int64_t q = c * 256 + 4 * lane;
        i4 v[kFRows];
#pragma unroll
        for (int r = 0; r < kFRows; ++r) {
          const int e = e0 + kWaves * r;
          v[r] = (e < E && q < nbc) ? *reinterpret_cast<const i4*>(blockcnt + (int64_t)e * ld + q)
                                    : i4{0, 0, 0, 0};
        }
#pragma unroll
        for (int r = 0; r < kFRows; ++r)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int x = (q + j < nbc) ? v[r][j] : 0;   // entries past nbc are not counts
            tot[r] += x;
            if (q + j < bfirst) bef[r] += x;
          }
      }
#pragma unroll
      for (int r = 0; r < kFRows; ++r) {
        const int e = e0 + kWaves * r;
        const int sb = wave_sum(bef[r]), st = wave_sum(tot[r]);
        if (lane == 0 && e < E) {
          base_s[e] = sb;
          tot_s[e] = st;
        }
      }
    }
  } else if (tid < 256) {
    base_s[tid] = 0;
  }

  // 3a. bitmask of this workgroup's tokens per expert
  const int64_t t = t0 + tid;
  const bool valid = tid < kFT && t < T;
  const int w = (tid >> 5) & (kFWords - 1);
  const uint32_t bit = 1u << (tid & 31);
  __syncthreads();                            // bits zeroed
  // the first kChunk ids stay in registers for the ranking pass
  int e_first[kChunk];
#pragma unroll
  for (int c = 0; c < kChunk; ++c) e_first[c] = (valid && c < K) ? ids[t * K + c] : -1;
  if (valid)
    for (int k0 = 0; k0 < K; k0 += kChunk) {
      int ee[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; ++c)
        ee[c] = (k0 == 0) ? e_first[c] : ((k0 + c < K) ? ids[t * K + k0 + c] : -1);
#pragma unroll
      for (int c = 0; c < kChunk; ++c)
        if (ee[c] >= 0 && ee[c] < E) atomicOr(&bits[ee[c] * kFWords + w], bit);
    }
  __syncthreads();
  // 3b. exclusive prefix of the words' popcounts, per expert (8-lane segments)
  for (int j = tid; j < Ep * kFWords; j += kFThreads) {
    const int c = __popc(bits[j]);
    int x = c;
#pragma unroll
    for (int off = 1; off < kFWords; off <<= 1) {
      const int y = __shfl_up(x, off, kFWords);
      if ((j & (kFWords - 1)) >= off) x += y;
    }
    pre[j] = x - c;
  }
  __syncthreads();
  int mytot = 0, mine = 0;                    // mine: this workgroup's assignments to expert tid
  if (tid < E) {
    mine = pre[tid * kFWords + kFWords - 1] + __popc(bits[tid * kFWords + kFWords - 1]);
    mytot = (gridDim.x > 1) ? tot_s[tid] : mine;
  }
  const bool staged = K <= kFStageK;
  if (staged) {
    int nst = 0;
    const int ls = block_exscan256(mine, E, tmp, &nst);
    if (tid < E) lst_s[tid] = ls;
  }

  // 2. capped counts, offsets (and, in workgroup 0, the metadata and tile table)
  int kept = 0;
  if (tid < E) kept = ((int64_t)mytot < C) ? mytot : (int)C;
  int total = 0;
  const int off = block_exscan256(kept, E, tmp, &total);
  if (tid < E) offs_s[tid] = off;
  if (blockIdx.x == 0) {
    if (tid < E) {
      raw[tid] = mytot;
      counts[tid] = kept;
      offsets[tid] = off;
    }
    if (tid == 0) offsets[E] = total;
    if (table) {
      const int nt = (tid < E) ? (kept + kGemmBM - 1) / kGemmBM : 0;
      int ntiles = 0;
      const int start = tile_starts(nt, E, tcnt_s, tord_s, tpref_s, tmp, &ntiles);
      if (tid < E) write_tiles(tid, off, kept, start, max_tiles, table);
      if (tid == 0) {
        table[0] = (int64_t)ntiles < max_tiles ? ntiles : (int)max_tiles;
        table[1] = table[2] = table[3] = 0;
      }
    }
  }
  __syncthreads();                            // base_s, offs_s, lst_s complete

  // 3c. ranks and slots (perm_token through the staging runs, or directly)
  if (valid)
    for (int k0 = 0; k0 < K; k0 += kChunk) {
      int ee[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; ++c)
        ee[c] = (k0 == 0) ? e_first[c] : ((k0 + c < K) ? ids[t * K + k0 + c] : -1);
      int32_t slot[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        const int e = ee[c];
        slot[c] = -1;
        if (k0 + c < K && e >= 0 && e < E) {
          const int jw = e * kFWords + w;
          const int within = pre[jw] + __popc(bits[jw] & (bit - 1u));
          const int64_t rank = (int64_t)base_s[e] + within;
          if (rank < C) {
            slot[c] = (int32_t)(offs_s[e] + rank);
            if (staged) stage[lst_s[e] + within] = (int32_t)t;
            else perm[slot[c]] = (int32_t)t;
          }
        }
      }
      if ((K & 3) == 0 && k0 + kChunk <= K) {   // whole 16-byte pieces of the token's row
        using i4 = int __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int c = 0; c < kChunk; c += 4)
          *reinterpret_cast<i4*>(inv + t * K + k0 + c) = i4{slot[c], slot[c + 1], slot[c + 2], slot[c + 3]};
      } else {
#pragma unroll
        for (int c = 0; c < kChunk; ++c)
          if (k0 + c < K) inv[t * K + k0 + c] = slot[c];
      }
    }
  if (!staged) return;
  __syncthreads();
  // each expert's kept run: consecutive lanes store consecutive slots
  for (int e = wave; e < E; e += kWaves) {
    const int n = pre[e * kFWords + kFWords - 1] + __popc(bits[e * kFWords + kFWords - 1]);
    const int64_t room = C - (int64_t)base_s[e];          // ranks below C are kept
    const int nk = room <= 0 ? 0 : (room < n ? (int)room : n);
    const int64_t dst = (int64_t)offs_s[e] + base_s[e];
    for (int i = lane; i < nk; i += 64) perm[dst + i] = stage[lst_s[e] + i];
  }
}

__global__ __launch_bounds__(256) void tile_table_kernel(const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ table,
                                                         int64_t max_tiles, int64_t rows_max,
                                                         int E) {
  __shared__ int tmp[256];
  __shared__ int tcnt_s[256], tord_s[256], tpref_s[256];   // tile_starts scratch
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
  const int start = tile_starts(nt, E, tcnt_s, tord_s, tpref_s, tmp, &ntiles);
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

hipError_t launch_permute_fused(const Problem& p, const int32_t* ids, const int32_t* blockcnt,
                                int cb, int64_t ld, int32_t* raw, int32_t* counts,
                                int32_t* offsets, int32_t* table, int32_t* perm, int32_t* inv,
                                hipStream_t s) {
  const int64_t nwg = (p.T + kFT - 1) / kFT;
  if (nwg > 1 && (blockcnt == nullptr || kFT % cb != 0 || (kFT / cb) % 4 != 0))
    return hipErrorInvalidValue;
  const int64_t nbc = (p.T + cb - 1) / cb;
  hipLaunchKernelGGL(permute_fused_kernel, dim3((unsigned)nwg), dim3(kFThreads), 0, s, ids, blockcnt, cb,
                     ld, nbc, raw, counts, offsets, table, max_row_tiles(p, kGemmBM), perm, inv,
                     p.T, p.E, p.K, p.C);
  return hipGetLastError();
}

hipError_t launch_tile_table(const Problem& p, const int32_t* offsets, int32_t* table,
                             hipStream_t s) {
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(256), 0, s, offsets, table,
                     max_row_tiles(p, kGemmBM), p.rows_max, p.E);
  return hipGetLastError();
}

}  // namespace moe
