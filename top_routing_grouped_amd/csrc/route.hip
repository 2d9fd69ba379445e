// Steps 1-2 of the layer: router logits, softmax + top-K, renormalised gates.
//
// Router scores l = X W_r (+ b) ([P2] "Routing-Free 与 OmniMoE" §1.1: a
// token goes Router -> softmax -> TopK), selection of the K best experts with
// K a run-time value ([P4] "AI芯片如何支持MoE架构" §4.3), gates renormalised
// over the selected experts.
//
// One workgroup = 64 tokens, 16x16x32 bf16 MFMA, waves in a 2 x (NW/2) grid
// over (32 tokens) x (a slice of the padded expert range): 4 waves below 128
// padded experts, 8 from 128 on.  For E % 8 == 0 the X tile (64 tokens x
// 64 k) and the W_r tile (64 k x E, natural [k][e] layout) of each k-step go
// global -> LDS with global_load_lds_dwordx4 through four stages whose
// completion is counted with explicit vmcnt waits; the W_r tile
// is read with the gfx950 transpose load (ds_read_b64_tr_b16), so the weights
// need no transpose in memory, and both tiles are XOR-swizzled so that every
// fragment read is bank-conflict free.  (Other E use a register-staged
// variant.)  The 64 x E fp32 scores (+ bias) land in LDS, then each 16-lane
// DPP row selects the top K of its tokens on order-preserving int32 keys:
// integer max / min reductions need no NaN canonicalisation, and folding
// -0.0 into +0.0 before keying makes the two zeros tie (then the lower id
// wins, as the oracle rules).  The selection is either K rounds of row
// maxima over lanes sorted once (default) or the threshold bisection of
// [P4] §4.3 (MOE_FLAG_TOPK_THRESHOLD); both give the same ids, order and
// gates.  The fp32 router uses fp32 MFMA (32x32x2) on LDS-staged slices.
#include "moe_internal.hpp"

namespace moe {
namespace {

using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using i16x4 = short __attribute__((ext_vector_type(4)));
using f32x4 = float __attribute__((ext_vector_type(4)));
using f32x16 = float __attribute__((ext_vector_type(16)));
using u32x4 = uint32_t __attribute__((ext_vector_type(4)));

constexpr int kTok = 64;       // tokens per workgroup
constexpr int kBK = 64;        // k per stage
constexpr int kThreads = 256;

// ---------------------------------------------------------------- selection helpers
__device__ __forceinline__ int sort_key(float f) {
  int b = __float_as_int(f + 0.0f);          // -0.0 -> +0.0
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key_value(int k) {
  return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF));
}
// Every lane of these patterns reads a valid lane of its row, so bound_ctrl
// changes nothing and lets the compiler fold the move into the max/min/add.
template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);
}
// Butterfly over one 16-lane DPP row; every lane of the row ends with the result.
__device__ __forceinline__ int row_max16(int x) {
  x = max(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = max(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = max(x, dpp<0x141>(x));  // row_half_mirror
  x = max(x, dpp<0x140>(x));  // row_mirror
  return x;
}
__device__ __forceinline__ int row_min16(int x) {
  x = min(x, dpp<0xB1>(x));
  x = min(x, dpp<0x4E>(x));
  x = min(x, dpp<0x141>(x));
  x = min(x, dpp<0x140>(x));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(dpp<0xB1>(__float_as_int(x)));
  x += __int_as_float(dpp<0x4E>(__float_as_int(x)));
  x += __int_as_float(dpp<0x141>(__float_as_int(x)));
  x += __int_as_float(dpp<0x140>(__float_as_int(x)));
  return x;
}

// Batcher's odd-even merge network on V inputs (V a power of two), listed
// at compile time: comparator c orders entries lo[c] < hi[c].
template <int V>
struct BatcherNet {
  int lo[V * V] = {}, hi[V * V] = {};
  int n = 0;
  constexpr BatcherNet() {
    for (int p = 1; p < V; p <<= 1)
      for (int k = p; k >= 1; k >>= 1)
        for (int j = k % p; j + k < V; j += 2 * k)
          for (int i = 0; i < k && i < V - j - k; ++i)
            if ((i + j) / (2 * p) == (i + j + k) / (2 * p)) {
              lo[n] = i + j;
              hi[n] = i + j + k;
              ++n;
            }
  }
};

// Sorts v[0..V) into descending order.  The comparator list is a constant
// and the loop over it has a constant trip count, so after unrolling every
// index is a constant and the entries stay in registers.  (Written as nested
// loops over the network's stages, the 16-entry case was not fully unrolled
// in one kernel: the entries were then picked by chains of selects and the
// decode-batch selection took 33 instead of 5 us.)
template <int V>
__device__ __forceinline__ void sort_desc(int64_t* v) {
  constexpr BatcherNet<V> net{};
#pragma unroll
  for (int c = 0; c < net.n; ++c) {
    const int64_t a = v[net.lo[c]], b = v[net.hi[c]];
    const bool sw = b > a;
    v[net.lo[c]] = sw ? b : a;
    v[net.hi[c]] = sw ? a : b;
  }
}

// Top-K of the tokens whose scores sit in LDS (row stride S floats, padded
// columns hold -inf).  Each 16-lane DPP row takes R tokens, so wave w
// handles tokens 4Rw .. 4Rw + 4R - 1 and DPP row q takes tokens 4Rw + Rq + r,
// r < R; lane i of the row holds experts i + 16j.  Each lane first sorts its
// V entries once, as 64-bit values (sort key, 255 - id): one signed order
// ranks the score first, then the lower id.  A round then only looks at the
// lanes' heads: the row maximum of the head keys, the lowest id among the
// heads holding it, and the lane that owns that id pops its head.  (The lowest
// id of the maximum key in a lane is that lane's head, so this is the lowest
// id of the maximum overall, as the oracle rules.)  Rescanning all V entries
// every round takes about twice the VALU instructions; measured, the router
// gains 0.3-0.7 us at E = 128 and is within run-to-run noise (+-3 us of
// 113) at E = 256.  Round results go to ids (global) and, as values,
// back into the token's own LDS row (no longer read) for the gate pass.
template <int V, int R = 4>
__device__ __forceinline__ void topk_from_lds(float* L, int S, int64_t t0, int64_t T, int E, int K,
                                              int32_t* __restrict__ ids, float* __restrict__ gates,
                                              int* cntl = nullptr) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int i = lane & 15;
  // a popped or exhausted entry: below every real key (-inf included)
  constexpr int64_t kRetired = (int64_t)(((uint64_t)0x80000000u) << 32);
  int64_t v[R][V];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float* row = L + (4 * R * w + R * q + r) * S;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int e = i + 16 * j;
      v[r][j] = (int64_t)(((uint64_t)(uint32_t)sort_key(row[e]) << 32) | (uint32_t)(255 - e));
    }
    sort_desc<V>(v[r]);
  }
  int top[R];
  for (int k = 0; k < K; ++k) {
    // the R tokens of a row are independent chains: keep them in one
    // branch-free block so their DPP steps interleave
    int m[R], cand[R];
#pragma unroll
    for (int r = 0; r < R; ++r) m[r] = row_max16((int)(v[r][0] >> 32));
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int head_id = 255 - (int)(uint32_t)v[r][0];
      cand[r] = ((int)(v[r][0] >> 32) == m[r]) ? head_id : 0x7FFFFFFF;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) cand[r] = row_min16(cand[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // ids are distinct within the row, so exactly one lane pops.  The pop
      // is a bitwise blend under an opaque all-ones / all-zeros mask: written
      // as selects, the compiler turned the shift into loads at index j + win
      // and so into compare-and-select chains over every entry (quadratic in
      // V, and at V = 16 the masks spilled to vector lanes).
      const bool win = ((int)(v[r][0] >> 32) == m[r]) && (255 - (int)(uint32_t)v[r][0] == cand[r]);
      int wm32 = win ? -1 : 0;
      asm volatile("" : "+v"(wm32));
      const uint64_t wmask = (uint64_t)(int64_t)wm32;
#pragma unroll
      for (int j = 0; j + 1 < V; ++j)
        v[r][j] = (int64_t)(((uint64_t)v[r][j + 1] & wmask) | ((uint64_t)v[r][j] & ~wmask));
      v[r][V - 1] = (int64_t)(((uint64_t)kRetired & wmask) | ((uint64_t)v[r][V - 1] & ~wmask));
      if (k == 0) top[r] = m[r];
    }
    if (i == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int tl = 4 * R * w + R * q + r;
        L[tl * S + k] = key_value(m[r]);
        if (t0 + tl < T) {
          ids[(t0 + tl) * K + k] = cand[r];
          if (cntl) atomicAdd(&cntl[cand[r]], 1);
        }
      }
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  // gates: softmax over the K selected scores (the full-softmax denominator
  // cancels in the renormalisation).
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int tl = 4 * R * w + R * q + r;
    const float m0 = key_value(top[r]);
    float part = 0.f;
    for (int c = i; c < K; c += 16) part += expf(L[tl * S + c] - m0);
    const float sum = row_sum16(part);
    if (t0 + tl < T) {
      for (int c = i; c < K; c += 16)
        gates[(t0 + tl) * K + c] = expf(L[tl * S + c] - m0) / sum;
    }
  }
}

__device__ __forceinline__ int row_sum16i(int x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

// The same top-K by threshold selection ("AI芯片如何支持MoE架构" §4.3: guess a
// threshold, count the scores above it, raise or lower it), with the same
// token layout as topk_from_lds and exactly its results:
// * the K-th largest key th is found by bisection over the 32-bit
//   order-preserving key: each step tries th | bit and keeps the bit when at
//   least K keys of the token's row reach it (a DPP row sum of per-lane
//   counts).  It starts below the highest bit where the row's largest and
//   smallest keys differ.
// * ties at th, when not all fit, go to the lowest ids: the same bisection
//   over the 8-bit ids of the tied entries.
// * the K winners are compacted into the token's LDS row slot by slot (lane
//   i, slot j is expert i + 16 j, so positions follow ascending ids), and a
//   winner's rank is the number of row keys above its own plus the equal
//   keys at lower positions: the order (score desc, id asc).
template <int V, int R = 4>
__device__ __forceinline__ void topk_threshold_from_lds(float* L, int S, int64_t t0, int64_t T,
                                                        int E, int K, int32_t* __restrict__ ids,
                                                        float* __restrict__ gates, int* cntl) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int i = lane & 15;
  uint32_t uk[R][V];
  float val[R][V];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float* row = L + (4 * R * w + R * q + r) * S;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      val[r][j] = row[i + 16 * j];
      uk[r][j] = (uint32_t)sort_key(val[r][j]) ^ 0x80000000u;
    }
  }
  // threshold: the K-th largest key of each token.  The R tokens of a row
  // run their bisections side by side (independent DPP chains), over the
  // wave's widest range of bits; a token skips the bits above its own range.
  uint32_t th[R];
  int top[R], hb[R];
  int hbw = -1;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int mx = (int)0x80000000, mn = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      mx = max(mx, (int)(uk[r][j] ^ 0x80000000u));
      mn = min(mn, (int)(uk[r][j] ^ 0x80000000u));
    }
    mx = row_max16(mx);
    mn = row_min16(mn);
    top[r] = mx;                              // largest sort key (signed order)
    const uint32_t kmax = (uint32_t)mx ^ 0x80000000u, kmin = (uint32_t)mn ^ 0x80000000u;
    const uint32_t diff = kmax ^ kmin;
    hb[r] = diff ? 31 - __builtin_clz(diff) : -1;
    th[r] = (hb[r] >= 0) ? (kmax & ~((2u << hb[r]) - 1u)) : kmax;
    hbw = max(hbw, hb[r]);
  }
  hbw = max(max(__builtin_amdgcn_readlane(hbw, 0), __builtin_amdgcn_readlane(hbw, 16)),
            max(__builtin_amdgcn_readlane(hbw, 32), __builtin_amdgcn_readlane(hbw, 48)));
  for (int bit = hbw; bit >= 0; --bit) {
    int c[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t cand = th[r] | (1u << bit);
      c[r] = 0;
#pragma unroll
      for (int j = 0; j < V; ++j) c[r] += uk[r][j] >= cand;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) c[r] = row_sum16i(c[r]);
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (bit <= hb[r] && c[r] >= K) th[r] |= 1u << bit;
  }
  // ties at the threshold: the lowest ids first
  int xid[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      gt += uk[r][j] > th[r];
      eq += uk[r][j] == th[r];
    }
    gt = row_sum16i(gt);
    eq = row_sum16i(eq);
    const int need = K - gt;
    int x = 255;                               // every tie taken (the usual case)
    if (need < eq) {
      x = 0;
      for (int bit = 7; bit >= 0; --bit) {
        const int cand = x | (1 << bit);
        int c = 0;
#pragma unroll
        for (int j = 0; j < V; ++j) c += (uk[r][j] == th[r]) && (i + 16 * j < cand);
        if (row_sum16i(c) < need) x = cand;
      }
    }
    xid[r] = x;
  }
  // compact the winners' keys into the token's row, positions in id order
  int pos[R][V];
  __builtin_amdgcn_wave_barrier();             // every lane has read its row entries
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int* row = reinterpret_cast<int*>(L + (4 * R * w + R * q + r) * S);
    int base = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const bool win = uk[r][j] > th[r] || (uk[r][j] == th[r] && i + 16 * j <= xid[r]);
      const uint32_t m = (uint32_t)(__ballot(win) >> (16 * q)) & 0xFFFFu;
      pos[r][j] = win ? base + __popc(m & ((1u << i) - 1u)) : -1;
      if (win) row[pos[r][j]] = (int)(uk[r][j] ^ 0x80000000u);
      base += __popc(m);
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  int rank[R][V];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int* row = reinterpret_cast<const int*>(L + (4 * R * w + R * q + r) * S);
#pragma unroll
    for (int j = 0; j < V; ++j) rank[r][j] = 0;
    for (int c = 0; c < K; ++c) {
      const int kc = row[c];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int mine = (int)(uk[r][j] ^ 0x80000000u);
        rank[r][j] += (kc > mine) || (kc == mine && c < pos[r][j]);
      }
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  // winners in rank order: ids out, scores back into the row for the gates
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int tl = 4 * R * w + R * q + r;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      if (pos[r][j] >= 0) {
        L[tl * S + rank[r][j]] = val[r][j];
        if (t0 + tl < T) {
          ids[(t0 + tl) * K + rank[r][j]] = i + 16 * j;
          if (cntl) atomicAdd(&cntl[i + 16 * j], 1);
        }
      }
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int tl = 4 * R * w + R * q + r;
    const float m0 = key_value(top[r]);
    float part = 0.f;
    for (int c = i; c < K; c += 16) part += expf(L[tl * S + c] - m0);
    const float sum = row_sum16(part);
    if (t0 + tl < T) {
      for (int c = i; c < K; c += 16)
        gates[(t0 + tl) * K + c] = expf(L[tl * S + c] - m0) / sum;
    }
  }
}

// Top-K by the selection the kernel was built for (SEL: 0 sorted lanes and
// K rounds of row maxima, 1 threshold bisection); the results are the same.
// A template parameter, not a run-time branch: compiled into one kernel, the
// bisection's registers made the default selection spill scalar registers.
template <int SEL, int V, int R = 4>
__device__ __forceinline__ void select_topk(float* L, int S, int64_t t0, int64_t T, int E, int K,
                                            int32_t* __restrict__ ids, float* __restrict__ gates,
                                            int* cntl) {
  if constexpr (SEL == 1) topk_threshold_from_lds<V, R>(L, S, t0, T, E, K, ids, gates, cntl);
  else topk_from_lds<V, R>(L, S, t0, T, E, K, ids, gates, cntl);
}

// Shared tail: bias, optional export, selection.
// PREPPED: the caller already added the bias and wrote -inf into the padding.
template <int SEL, int V, bool PREPPED = false>
__device__ __forceinline__ void route_tail(float* L, int S, int64_t t0, int64_t T, int E, int K, int Epad,
                           const float* __restrict__ bias, float* __restrict__ logits,
                           int32_t* __restrict__ ids, float* __restrict__ gates, int* cntl) {
  if (!PREPPED) {
    for (int idx = threadIdx.x; idx < kTok * Epad; idx += kThreads) {
      const int r = idx / Epad, e = idx - (idx / Epad) * Epad;
      float v = L[r * S + e];
      if (e < E) {
        if (bias) v += bias[e];
      } else {
        v = -__builtin_inff();
      }
      L[r * S + e] = v;
    }
    __syncthreads();
  }
  if (logits) {
    for (int idx = threadIdx.x; idx < kTok * E; idx += kThreads) {
      const int r = idx / E, e = idx - (idx / E) * E;
      if (t0 + r < T) logits[(t0 + r) * E + e] = L[r * S + e];
    }
    __syncthreads();  // selection rewrites the rows being exported
  }
  select_topk<SEL, V>(L, S, t0, T, E, K, ids, gates, cntl);
}

// Per-block expert counts for the permutation: the selection above adds each
// chosen expert of the block's tokens to an LDS array (zeroed by
// count_zero before the selection), which is then stored expert-major,
// blockcnt[e * ldc + block] (every expert's entry, zeros included).
__device__ __forceinline__ void count_zero(int* cntl, int nthreads) {
  for (int e = threadIdx.x; e < 256; e += nthreads) cntl[e] = 0;
}
__device__ __forceinline__ void count_store(const int* cntl, int32_t* __restrict__ blockcnt,
                                            int64_t ldc, int64_t block, int E, int nthreads) {
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += nthreads) blockcnt[e * ldc + block] = cntl[e];
}

// ---------------------------------------------------------------- bf16 router (MFMA)
// NBW: 16-column blocks per wave; the padded expert range is 32*NBW.
// The widest expert range (NBW = 8) needs the whole register file: one
// workgroup per CU; narrower ones fit two.
template <int NBW, bool VEC, int SEL>
__global__ __launch_bounds__(kThreads, (NBW >= 8) ? 1 : 2) void route_bf16_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wr, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ gates, int64_t T,
    int d, int E, int K, int32_t* __restrict__ blockcnt, int64_t ldc) {
  constexpr int Epad = 32 * NBW;
  __shared__ int cntl[256];
  // X stages held in registers (prefetch depth); fewer when the weight tile is wide
  constexpr int kPF = (NBW >= 8) ? 4 : 6;
  constexpr int R = Epad + 16;            // bf16 elements per LDS weight row (padded)
  constexpr int S = Epad + 16;            // floats per LDS score row
  constexpr int kStageElems = kBK * R;
  constexpr int kLdsBytes = (2 * kStageElems * 2 > kTok * S * 4) ? 2 * kStageElems * 2 : kTok * S * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
  uint16_t* Bs = reinterpret_cast<uint16_t*>(smem);
  float* L = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int KT = d / kBK;

  // A operand rows (16x16x32: lane -> row lane%16, k chunk lane/16).
  const uint16_t* arow[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    int64_t t = t0 + wm * 32 + rb * 16 + (lane & 15);
    if (t > T - 1) t = T - 1;
    arow[rb] = X + t * (int64_t)d + 8 * (lane >> 4);
  }

  // Weight tile staging: NBW chunks of 8 bf16 per thread per stage, two
  // stages in registers (loaded two k-steps ahead) plus two in LDS.
  constexpr int kChunksPerRow = Epad / 8;
  uint16_t breg[2][NBW][8];
  auto load_b = [&](int slot, int kt) {
#pragma unroll
    for (int c = 0; c < NBW; ++c) {
      const int idx = tid + kThreads * c;
      const int row = idx / kChunksPerRow;
      const int col = (idx % kChunksPerRow) * 8;
      const uint16_t* src = Wr + (int64_t)(kt * kBK + row) * E + col;
      if (VEC) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (col < E) v = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          breg[slot][c][2 * h] = (uint16_t)(v[h] & 0xFFFF);
          breg[slot][c][2 * h + 1] = (uint16_t)(v[h] >> 16);
        }
      } else {
#pragma unroll
        for (int h = 0; h < 8; ++h) breg[slot][c][h] = (col + h < E) ? src[h] : (uint16_t)0;
      }
    }
  };
  auto store_b = [&](int slot, int buf) {
#pragma unroll
    for (int c = 0; c < NBW; ++c) {
      const int idx = tid + kThreads * c;
      const int row = idx / kChunksPerRow;
      const int col = (idx % kChunksPerRow) * 8;
      u32x4 v;
#pragma unroll
      for (int h = 0; h < 4; ++h)
        v[h] = (uint32_t)breg[slot][c][2 * h] | ((uint32_t)breg[slot][c][2 * h + 1] << 16);
      *reinterpret_cast<u32x4*>(Bs + buf * kStageElems + row * R + col) = v;
    }
  };

  f32x4 acc[2][NBW];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 a[kPF][2][2];  // [stage slot][k substep][row block]
  auto load_a = [&](int slot, int kt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        a[slot][ks][rb] = *reinterpret_cast<const bf16x8*>(arow[rb] + kt * kBK + ks * 32);
  };

  // transpose-load lane geometry (16x16x32 B operand: col lane%16, k 8*(lane/16)+j)
  const int g = lane >> 4, s4 = lane & 15;
  const int trow = 8 * g + (s4 >> 2);
  const int tcol = wn * 16 * NBW + 4 * (s4 & 3);

  load_b(0, 0);
  if (KT > 1) load_b(1, 1);
#pragma unroll
  for (int s = 0; s < kPF - 1; ++s)
    if (s < KT) load_a(s, s);
  store_b(0, 0);
  __syncthreads();

  for (int kt0 = 0; kt0 < KT; kt0 += kPF) {
#pragma unroll
    for (int u = 0; u < kPF; ++u) {
      const int kt = kt0 + u;
      if (kt < KT) {
        // weights first: vmcnt retires in issue order, so the wait before
        // store_b then leaves the deeper X prefetch in flight.  kt0 is a
        // multiple of kPF (even), so kt%2 == u%2 at compile time.
        if (kt + 2 < KT) load_b(u % 2, kt + 2);
        if (kt + kPF - 1 < KT) load_a((u + kPF - 1) % kPF, kt + kPF - 1);
        const uint16_t* Bt = Bs + (kt & 1) * kStageElems;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) {
            const uint16_t* p = Bt + (ks * 32 + trow) * R + tcol + nb * 16;
            i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(p));
            i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(p + 4 * R));
            bf16x8 b;
            b = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
              acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][ks][rb], b, acc[rb][nb], 0, 0, 0);
          }
        }
        if (kt + 1 < KT) store_b((u + 1) % 2, (kt + 1) & 1);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
    }
  }

  // scores -> LDS (reusing the weight buffers)
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 32 + rb * 16 + 4 * (lane >> 4) + r;
        const int col = wn * 16 * NBW + nb * 16 + (lane & 15);
        L[row * S + col] = acc[rb][nb][r];
      }
  if (blockcnt) count_zero(cntl, kThreads);
  __syncthreads();
  route_tail<SEL, 2 * NBW>(L, S, t0, T, E, K, Epad, bias, logits, ids, gates,
                           blockcnt ? cntl : nullptr);
  if (blockcnt) count_store(cntl, blockcnt, ldc, blockIdx.x, E, kThreads);
}

// ---------------------------------------------------------------- bf16 router, staged copies
// For E % 8 == 0 (W_r rows are whole 16-byte chunks).  The X tile (64 tokens
// x 64 k, 128-byte rows) and the W_r tile (64 k x Epad, natural [k][e]
// layout) of each k-step go global -> LDS with global_load_lds_dwordx4;
// NST stages keep NST-1 k-steps of copies in flight, and the copies are
// counted with explicit vmcnt waits so no load ever waits on a later one.
// Both tiles are XOR-swizzled at 16-byte granularity so that the X fragment
// reads (ds_read_b128) and the W_r transpose reads are bank-conflict free.

// XOR applied to the 16-byte chunk index of W_r tile row r (CPR chunks per
// row) so that a 16x16x32 transpose read touches every bank equally.
template <int CPR>
__device__ __forceinline__ int wr_swizzle(int r) {
  if (CPR >= 16) return 2 * ((r & 3) + 4 * ((r >> 3) & 1));
  if (CPR == 8) return 2 * (((r >> 1) & 1) + 2 * ((r >> 3) & 1));
  return 2 * ((r >> 3) & 1);
}

template <int NBW>
struct RouteGeo {
  static constexpr int Epad = 32 * NBW;
  // Waves: 4 (2 token halves x 2 expert halves), or 8 (2 x 4) from 128
  // padded experts on.  One workgroup per CU either way; 8 waves put two on
  // each SIMD, so one wave's LDS and barrier waits overlap the other's MFMAs
  // (measured: E = 256, T = 32768, d = 4096: 133 -> 122 us; E = 128: 30 ->
  // 29 us).  Below 128 the W_r tile has too few copies to split over 8 waves.
  static constexpr int NW = (NBW >= 4) ? 8 : 4;
  static constexpr int kThreads = 64 * NW;
  static constexpr int WN = NW / 2;                  // waves along the experts
  static constexpr int CBW = 2 * NBW / WN;           // 16-expert MFMA blocks per wave
  // LDS stages (X tile + W_r tile each).  Four at every width (E = 256: 4 x
  // 40 KB, the whole LDS; 136 instead of 144 us with three at T = 32768,
  // d = 4096); more at E = 128 were slower (five or six: 34-35 against 30 us).
  static constexpr int NST = 4;
  static constexpr int kX = kTok * kBK * 2;          // X tile bytes (8 KB)
  static constexpr int kW = kBK * Epad * 2;          // W_r tile bytes
  static constexpr int kStage = kX + kW;
  static constexpr int S = Epad + 16;                // floats per score row
  // per-block expert counts (256 ints) after the score rows, in the idle stage space
  static constexpr int kCnt = kTok * S * 4;
  static constexpr int kLds = (NST * kStage > kCnt + 1024) ? NST * kStage : kCnt + 1024;
  static_assert(kLds <= 160 * 1024, "one workgroup's LDS");
  static constexpr int kXInstr = kX / 1024 / NW;     // copies per wave per tile
  static constexpr int kWInstr = kW / 1024 / NW;
  static_assert(kXInstr * 1024 * NW == kX && kWInstr * 1024 * NW == kW, "copy split");
  static constexpr int kInstr = kXInstr + kWInstr;
  static constexpr int CPR = Epad / 8;               // 16-byte chunks per W_r tile row
  static constexpr int kWRows = 64 / CPR;            // W_r rows per copy instruction
};

// Wait until at most `pending` stages (INSTR copies each) of this wave are in flight.
template <int INSTR>
__device__ __forceinline__ void wait_stages(int pending) {
  if (pending >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * INSTR) : "memory");
  else if (pending == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(INSTR) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// With ksplit > 1 the k range is split over gridDim.y workgroups per token
// block (for batches too small to fill the chip): each writes its raw fp32
// partial scores to partial[ks][T][Epad]; route_select_kernel adds them and
// finishes.
// Router matrices over the same tokens that share one launch (fp32 scores
// only, no bias or selection): job j takes workgroups j*nblk .. (j+1)*nblk-1,
// multiplying X by E[j] columns of a matrix whose rows (and score rows) are
// ld[j] wide.  n = 0: the launch is one ordinary router.  zero (optional):
// zero_n int32s cleared by the launch, a slice per workgroup.
struct RouteJobs {
  const uint16_t* W[4];
  float* logits[4];
  int E[4];
  int ld[4];
  int n;
  int nblk;
  int32_t* zero;
  int zero_n;
};
template <typename V>
__device__ __forceinline__ V pick4(const V (&a)[4], int j) {
  return j == 0 ? a[0] : j == 1 ? a[1] : j == 2 ? a[2] : a[3];
}

template <int NBW, int SEL>
__global__ __launch_bounds__(RouteGeo<NBW>::kThreads, 1) void route_staged_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wr, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ gates, int64_t T,
    int d, int E, int K, int ksplit, float* __restrict__ partial, RouteJobs jobs,
    int32_t* __restrict__ blockcnt, int64_t ldc) {
  using G = RouteGeo<NBW>;
  constexpr int Epad = G::Epad, NST = G::NST, CPR = G::CPR;
  constexpr int XI = G::kXInstr, WI = G::kWInstr, CBW = G::CBW;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  float* L = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / G::WN, wn = w - (w / G::WN) * G::WN;
  int bx = blockIdx.x;
  int ld = E;                                 // row stride of W_r and of the score rows
  if (jobs.n > 0) {
    const int j = bx / jobs.nblk;
    bx -= j * jobs.nblk;
    Wr = pick4(jobs.W, j);
    logits = pick4(jobs.logits, j);
    E = pick4(jobs.E, j);
    ld = pick4(jobs.ld, j);
    ids = nullptr;
    blockcnt = nullptr;
  }
  if (jobs.zero) {
    const int per = (jobs.zero_n + (int)gridDim.x - 1) / (int)gridDim.x;
    const int z1 = min(jobs.zero_n, ((int)blockIdx.x + 1) * per);
    for (int i = (int)blockIdx.x * per + tid; i < z1; i += G::kThreads) jobs.zero[i] = 0;
  }
  const int64_t t0 = (int64_t)bx * kTok;
  const int KT_all = d / kBK;
  const int kt0 = (int)(((int64_t)blockIdx.y * KT_all) / ksplit);   // this workgroup's k-steps
  const int KT = (int)(((int64_t)(blockIdx.y + 1) * KT_all) / ksplit) - kt0;
  const uint32_t lds_base = (uint32_t)(size_t)(__attribute__((address_space(3))) void*)smem;

  // X copies: instruction j = XI*w + i fills tile rows 8j + lane/8, slot
  // lane%8 holding k chunk slot ^ ((row >> 1) & 7).  Rows past T repeat row T-1.
  const uint16_t* xsrc[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int r = (w * XI + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    int64_t t = t0 + r;
    if (t > T - 1) t = T - 1;
    xsrc[i] = X + t * (int64_t)d + c * 8;
  }
  // W_r copies: instruction j = WI*w + i fills tile rows kWRows*j + lane/CPR,
  // slot lane%CPR holding column chunk slot ^ wr_swizzle(row).  Chunks past E
  // (padding) read chunk 0 of the same row: in bounds, and their scores are
  // replaced by -inf before selection.
  const uint16_t* wsrc[WI];
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int r = (w * WI + i) * G::kWRows + lane / CPR;
    int c = (lane % CPR) ^ wr_swizzle<CPR>(r);
    if (c * 8 >= E) c = 0;
    wsrc[i] = Wr + (int64_t)r * ld + c * 8;
  }
  // Every workgroup reads all of W_r; starting each one at a different
  // k-step (rotated by its position among the workgroups of its XCD) spreads
  // the reads of any moment over all of W_r instead of one 64-row tile.  The
  // sum over k is then taken in a rotated but fixed order per token position.
  // X is read once, with the non-temporal hint, so the stream of token rows
  // does not evict the W_r tiles every workgroup re-reads from L2 (the route
  // takes 30 instead of 38 us at the Qwen3 shape).
  const int rot = (ksplit > 1) ? 0 : (int)((blockIdx.x >> 3) % (unsigned)KT);
  auto issue = [&](int kt) {
    const uint32_t base = lds_base + (uint32_t)((kt % NST) * G::kStage);
    int kk = kt + rot;
    if (kk >= KT) kk -= KT;
    kk += kt0;
#pragma unroll
    for (int i = 0; i < XI; ++i) dev::lds_copy16_stream(xsrc[i] + kk * kBK, base + (w * XI + i) * 1024);
#pragma unroll
    for (int i = 0; i < WI; ++i)
      dev::lds_copy16(wsrc[i] + (int64_t)kk * kBK * ld, base + G::kX + (w * WI + i) * 1024);
  };

  // fragment offsets.  X (16x16x32 A operand): lane -> token row lane%16,
  // k chunk 4*ks + lane/16.  W_r (B operand, transpose read): lane group
  // g = lane/16, s = lane%16 -> tile row 32*ks + 8g + s/4 (+4 for the upper
  // half), column 16*nb + 4*(s%4) of this wave's expert range.
  int xo[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r = wm * 32 + rb * 16 + (lane & 15);
      const int c = 4 * ks + (lane >> 4);
      xo[rb][ks] = r * 128 + ((c ^ ((r >> 1) & 7)) * 16);
    }
  const int g = lane >> 4, s4 = lane & 15;
  int wo[CBW][2][2];
#pragma unroll
  for (int nb = 0; nb < CBW; ++nb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 32 * ks + 8 * g + (s4 >> 2) + 4 * h;
        const int col = wn * 16 * CBW + nb * 16 + 4 * (s4 & 3);
        wo[nb][ks][h] = G::kX + r * (Epad * 2) + (((col >> 3) ^ wr_swizzle<CPR>(r)) * 16) + (col & 7) * 2;
      }

  f32x4 acc[2][CBW];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int nb = 0; nb < CBW; ++nb) acc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < KT) issue(st);
  for (int kt = 0; kt < KT; ++kt) {
    // stage kt landed (own copies), then published to all waves; the barrier
    // also tells every wave that stage kt-1 (the buffer refilled below) is free
    const int issued = (kt + NST - 2 < KT - 1) ? kt + NST - 2 : KT - 1;
    wait_stages<G::kInstr>(issued - kt);
    asm volatile("s_barrier" ::: "memory");
    if (kt + NST - 1 < KT) issue(kt + NST - 1);
    const unsigned char* S = smem + (kt % NST) * G::kStage;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 a[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) a[rb] = *reinterpret_cast<const bf16x8*>(S + xo[rb][ks]);
#pragma unroll
      for (int nb = 0; nb < CBW; ++nb) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(S + wo[nb][ks][0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(S + wo[nb][ks][1]));
        const bf16x8 b = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], b, acc[rb][nb], 0, 0, 0);
      }
    }
  }

  if (ksplit > 1) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int nb = 0; nb < CBW; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t t = t0 + wm * 32 + rb * 16 + 4 * (lane >> 4) + r;
          const int col = wn * 16 * CBW + nb * 16 + (lane & 15);
          if (t < T) partial[((int64_t)blockIdx.y * T + t) * Epad + col] = acc[rb][nb][r];
        }
    return;
  }

  // scores (+ bias; -inf in the padding columns) -> LDS, reusing the stage
  // buffers once every wave is done reading them
  float bcol[CBW];
#pragma unroll
  for (int nb = 0; nb < CBW; ++nb) {
    const int col = wn * 16 * CBW + nb * 16 + (lane & 15);
    bcol[nb] = (col < E) ? (bias ? bias[col] : 0.f) : -__builtin_inff();
  }
  __syncthreads();
  int* cntl = reinterpret_cast<int*>(smem + G::kCnt);
  if (blockcnt) count_zero(cntl, G::kThreads);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int nb = 0; nb < CBW; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 32 + rb * 16 + 4 * (lane >> 4) + r;
        const int col = wn * 16 * CBW + nb * 16 + (lane & 15);
        L[row * G::S + col] = (col < E) ? acc[rb][nb][r] + bcol[nb] : bcol[nb];
      }
  __syncthreads();
  // optional export by every thread, then the selection by every wave
  // (64 / NW tokens each: 16 with 4 waves, 8 with 8)
  if (logits) {
    for (int idx = tid; idx < kTok * E; idx += G::kThreads) {
      const int r = idx / E, e = idx - (idx / E) * E;
      if (t0 + r < T) logits[(t0 + r) * ld + e] = L[r * G::S + e];
    }
    __syncthreads();  // selection rewrites the rows being exported
  }
  if (ids) select_topk<SEL, 2 * NBW, kTok / (4 * G::NW)>(L, G::S, t0, T, E, K, ids, gates,
                                                       blockcnt ? cntl : nullptr);
  if (blockcnt) count_store(cntl, blockcnt, ldc, bx, E, G::kThreads);
}

// Split-k finish, part 1: partial[0] = sum over ks of partial[ks], in ks
// order (a fixed order: the result does not depend on which workgroup of the
// router finished first).  One float4 of scores per thread, spread over as
// many workgroups as the T x Epad scores need.

// Split-k finish: the partial scores of TW tokens per workgroup added in split
// order (a separate summing launch took 4.7 us at the decode size), plus bias
// (-inf in the padding), then the selection by 4 waves of 4R tokens.
// Wide expert ranges (E > 64) take TW = 16 and one token per DPP row, so the
// serial selection chains of a small batch spread over several CUs (decode,
// T = 64, E = 256: the route 30 -> 21 us); narrower ones keep TW = 64, R = 4.
template <int NBW>
struct SelGeo {
  static constexpr int Epad = 32 * NBW, S = Epad + 16;
  static constexpr int TW = (NBW >= 4) ? 16 : kTok;
  static constexpr int R = TW / 16;
  static constexpr int kCnt = TW * S * 4;            // per-block expert counts after the rows
  static constexpr int kLds = kCnt + 1024;
};
template <int NBW, int SEL>
__global__ __launch_bounds__(kThreads) void route_select_kernel(
    const float* __restrict__ scores, const float* __restrict__ bias, float* __restrict__ logits,
    int32_t* __restrict__ ids, float* __restrict__ gates, int64_t T, int E, int K,
    int32_t* __restrict__ blockcnt, int64_t ldc, int ksplit) {
  using G = SelGeo<NBW>;
  constexpr int Epad = G::Epad, S = G::S, TW = G::TW;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* L = reinterpret_cast<float*>(smem);
  int* cntl = reinterpret_cast<int*>(smem + G::kCnt);
  if (blockcnt) count_zero(cntl, kThreads);
  const int64_t t0 = (int64_t)blockIdx.x * TW;
  // Each thread owns one 4-column group and kPer rows of it: all of its
  // 16-byte loads are issued before the first is used (one at a time, the
  // 64 x Epad scores took ~30 us of L2 round trips at Epad = 256).
  using f4 = float __attribute__((ext_vector_type(4)));
  constexpr int kGroups = Epad / 4;                  // 4-column groups per row
  constexpr int kRowStep = kThreads / kGroups;
  constexpr int kPer = TW / kRowStep;                // rows per thread
  static_assert(kRowStep * kGroups == kThreads && kPer * kRowStep == TW, "score split");
  const int c4 = threadIdx.x % kGroups, r0 = threadIdx.x / kGroups;
  float bv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * c4 + j;
    bv[j] = (bias && e < E) ? bias[e] : 0.f;
  }
  // scores[ks][T][Epad] holds the ksplit partial sums; they are added in
  // split order (split 0 first), up to four splits' loads in flight
  f4 v[kPer];
  int64_t roff[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t t = (t0 + r0 + kRowStep * i < T) ? t0 + r0 + kRowStep * i : T - 1;
    roff[i] = t * Epad + 4 * c4;
    v[i] = *reinterpret_cast<const f4*>(scores + roff[i]);
  }
  const int64_t plane = T * Epad;
  for (int ks = 1; ks < ksplit; ks += 4) {
    f4 a[4][kPer];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (ks + u < ksplit) a[u][i] = *reinterpret_cast<const f4*>(scores + (ks + u) * plane + roff[i]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (ks + u < ksplit) v[i] += a[u][i];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    f4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = (4 * c4 + j < E) ? (bias ? v[i][j] + bv[j] : v[i][j]) : -__builtin_inff();
    *reinterpret_cast<f4*>(L + (r0 + kRowStep * i) * S + 4 * c4) = o;
  }
  __syncthreads();
  if (logits) {
    for (int idx = threadIdx.x; idx < TW * E; idx += kThreads) {
      const int r = idx / E, e = idx - (idx / E) * E;
      if (t0 + r < T) logits[(t0 + r) * E + e] = L[r * S + e];
    }
    __syncthreads();  // selection rewrites the rows being exported
  }
  select_topk<SEL, 2 * NBW, G::R>(L, S, t0, T, E, K, ids, gates, blockcnt ? cntl : nullptr);
  if (blockcnt) count_store(cntl, blockcnt, ldc, blockIdx.x, E, kThreads);
}

// ---------------------------------------------------------------- fp32 router (MFMA)
// 64 tokens x Epad scores per workgroup: 32 x 32 blocks (2 token halves x
// Epad/32 expert blocks, dealt to the 4 waves) with v_mfma_f32_32x32x2_f32
// over 32-deep k slices of X and W_r staged in LDS (in the space the score
// rows take afterwards).  A lane supplies X[token lane%32][k lane/32] and
// W_r[k lane/32][expert lane%32] and ends with expert lane%32 of tokens
// 8*(v/4) + 4*(lane/32) + v%4 of its block.
template <int NBW>
struct F32RouteGeo {
  static constexpr int Epad = 32 * NBW, S = Epad + 16, TK = 32;
  static constexpr int kBlocks = 2 * NBW;                 // 32 x 32 score blocks
  static constexpr int kPerWave = (kBlocks + 3) / 4;
  static constexpr int kXs = kTok * (TK + 1);             // floats, padded rows
  static constexpr int kWs = TK * Epad;
  static constexpr int kFloats = (kTok * S > kXs + kWs) ? kTok * S : kXs + kWs;
};
template <int NBW, int SEL>
__global__ __launch_bounds__(kThreads) void route_f32_kernel(
    const float* __restrict__ X, const float* __restrict__ Wr, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ gates, int64_t T,
    int d, int E, int K, int32_t* __restrict__ blockcnt, int64_t ldc) {
  using G = F32RouteGeo<NBW>;
  constexpr int Epad = G::Epad, S = G::S, TK = G::TK;
  __shared__ float L[G::kFloats];
  __shared__ int cntl[256];
  float* Xs = L;                 // [kTok][TK + 1]
  float* Ws = L + G::kXs;        // [TK][Epad]
  if (blockcnt) count_zero(cntl, kThreads);
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  f32x16 acc[G::kPerWave];
#pragma unroll
  for (int b = 0; b < G::kPerWave; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
  for (int k0 = 0; k0 < d; k0 += TK) {
    for (int idx = tid; idx < kTok * TK; idx += kThreads) {
      const int r = idx / TK, c = idx - (idx / TK) * TK;
      Xs[r * (TK + 1) + c] = (t0 + r < T && k0 + c < d) ? X[(t0 + r) * (int64_t)d + k0 + c] : 0.f;
    }
    for (int idx = tid; idx < TK * Epad; idx += kThreads) {
      const int r = idx / Epad, e = idx - (idx / Epad) * Epad;
      Ws[r * Epad + e] = (e < E && k0 + r < d) ? Wr[(int64_t)(k0 + r) * E + e] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < G::kPerWave; ++b) {
      const int blk = w + 4 * b;                 // token half blk & 1, expert block blk >> 1
      if (blk < G::kBlocks) {
        const int tr = 32 * (blk & 1) + (lane & 31), ec = 32 * (blk >> 1) + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < TK; kk += 2)
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(Xs[tr * (TK + 1) + kk + (lane >> 5)],
                                                        Ws[(kk + (lane >> 5)) * Epad + ec], acc[b],
                                                        0, 0, 0);
      }
    }
    __syncthreads();
  }
  // scores to the rows (the staging space is free after the last barrier)
#pragma unroll
  for (int b = 0; b < G::kPerWave; ++b) {
    const int blk = w + 4 * b;
    if (blk < G::kBlocks) {
      const int ec = 32 * (blk >> 1) + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * (blk & 1) + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        L[r * S + ec] = acc[b][v];
      }
    }
  }
  __syncthreads();
  route_tail<SEL, 2 * NBW>(L, S, t0, T, E, K, Epad, bias, logits, ids, gates,
                           blockcnt ? cntl : nullptr);
  if (blockcnt) count_store(cntl, blockcnt, ldc, blockIdx.x, E, kThreads);
}

template <int NBW, int SEL>
hipError_t launch_route_sel(const Problem& p, const void* X, const void* W_r, const float* bias,
                            float* logits, int32_t* ids, float* gates, float* partial,
                            int32_t* blockcnt, hipStream_t s) {
  const int64_t ldc = blockcnt ? route_count_ld(p, partial != nullptr) : 0;
  const dim3 grid((unsigned)((p.T + kTok - 1) / kTok));
  if (p.bf16) {
    if (p.E % 8 == 0) {
      const int ksplit = partial ? route_ksplit(p) : 1;
      auto* kern = route_staged_kernel<NBW, SEL>;
      hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           RouteGeo<NBW>::kLds);
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL(kern, dim3(grid.x, (unsigned)ksplit), dim3(RouteGeo<NBW>::kThreads),
                         (size_t)RouteGeo<NBW>::kLds, s, (const uint16_t*)X, (const uint16_t*)W_r,
                         bias, logits, ids, gates, p.T, p.d, p.E, p.K, ksplit, partial,
                         RouteJobs{}, ksplit > 1 ? nullptr : blockcnt, ldc);
      if (ksplit > 1) {
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        constexpr int kSelLds = SelGeo<NBW>::kLds, TW = SelGeo<NBW>::TW;
        auto* sel = route_select_kernel<NBW, SEL>;
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(sel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kSelLds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(sel, dim3((unsigned)((p.T + TW - 1) / TW)), dim3(kThreads),
                           (size_t)kSelLds, s, partial, bias, logits, ids, gates, p.T, p.E, p.K,
                           blockcnt, ldc, ksplit);
      }
    } else
      hipLaunchKernelGGL((route_bf16_kernel<NBW, false, SEL>), grid, dim3(kThreads), 0, s,
                         (const uint16_t*)X, (const uint16_t*)W_r, bias, logits, ids, gates, p.T,
                         p.d, p.E, p.K, blockcnt, ldc);
  } else {
    hipLaunchKernelGGL((route_f32_kernel<NBW, SEL>), grid, dim3(kThreads), 0, s, (const float*)X,
                       (const float*)W_r, bias, logits, ids, gates, p.T, p.d, p.E, p.K, blockcnt,
                       ldc);
  }
  return hipGetLastError();
}

template <int NBW>
hipError_t launch_route_nbw(const Problem& p, const void* X, const void* W_r, const float* bias,
                            float* logits, int32_t* ids, float* gates, float* partial,
                            int32_t* blockcnt, hipStream_t s) {
  if (p.sel == 1) return launch_route_sel<NBW, 1>(p, X, W_r, bias, logits, ids, gates, partial, blockcnt, s);
  return launch_route_sel<NBW, 0>(p, X, W_r, bias, logits, ids, gates, partial, blockcnt, s);
}

}  // namespace

namespace {
template <int NBW>
hipError_t launch_jobs_nbw(int64_t T, int d, const RouteJobs& jobs, const void* X, hipStream_t s) {
  auto* kern = route_staged_kernel<NBW, 0>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       RouteGeo<NBW>::kLds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3((unsigned)(jobs.n * jobs.nblk), 1), dim3(RouteGeo<NBW>::kThreads),
                     (size_t)RouteGeo<NBW>::kLds, s, (const uint16_t*)X, (const uint16_t*)nullptr,
                     (const float*)nullptr, (float*)nullptr, (int32_t*)nullptr, (float*)nullptr, T,
                     d, 0, 1, 1, (float*)nullptr, jobs, (int32_t*)nullptr, (int64_t)0);
  return hipGetLastError();
}

// Token blocks below which a launch of the two axes leaves CUs idle (one
// workgroup per CU): the axes wider than 128 columns are then cut in two
// halves of their own workgroups.  The atomic-expert router (T = 4096, two
// 256-wide axes): 128 -> 256 workgroups.
constexpr int64_t kRouteFillBlocks = 256;
}  // namespace

bool route_pair_supported(int E1, int E2) {
  return E1 % 8 == 0 && E2 % 8 == 0 && E1 >= 1 && E2 >= 1 && E1 <= 256 && E2 <= 256;
}

hipError_t launch_logits_pair(int64_t T, int d, int E1, int E2, const void* X, const void* W1,
                              const void* W2, float* logits1, float* logits2, hipStream_t s,
                              int32_t* zero, int zero_n) {
  if (!route_pair_supported(E1, E2)) return hipErrorInvalidValue;
  if (T == 0) return hipSuccess;
  RouteJobs jobs{};
  jobs.nblk = (int)((T + kTok - 1) / kTok);
  jobs.zero = zero_n > 0 ? zero : nullptr;
  jobs.zero_n = zero_n;
  const bool halves = 2 * (int64_t)jobs.nblk < kRouteFillBlocks;
  const uint16_t* Ws[2] = {(const uint16_t*)W1, (const uint16_t*)W2};
  float* Ls[2] = {logits1, logits2};
  const int Es[2] = {E1, E2};
  int widest = 0;
  for (int a = 0; a < 2; ++a) {
    const int cut = (halves && Es[a] > 128) ? 128 : Es[a];
    for (int c0 = 0; c0 < Es[a]; c0 += cut) {
      const int w = (Es[a] - c0 < cut) ? Es[a] - c0 : cut;
      jobs.W[jobs.n] = Ws[a] + c0;
      jobs.logits[jobs.n] = Ls[a] + c0;
      jobs.E[jobs.n] = w;
      jobs.ld[jobs.n] = Es[a];
      ++jobs.n;
      widest = w > widest ? w : widest;
    }
  }
  const int nbw = route_nbw(widest);
  if (nbw <= 1) return launch_jobs_nbw<1>(T, d, jobs, X, s);
  if (nbw <= 2) return launch_jobs_nbw<2>(T, d, jobs, X, s);
  if (nbw <= 4) return launch_jobs_nbw<4>(T, d, jobs, X, s);
  return launch_jobs_nbw<8>(T, d, jobs, X, s);
}

hipError_t launch_route(const Problem& p, const void* X, const void* W_r, const float* bias,
                        float* logits, int32_t* ids, float* gates, float* partial,
                        hipStream_t s, int32_t* blockcnt) {
  const int nbw = route_nbw(p.E);
  if (nbw <= 1) return launch_route_nbw<1>(p, X, W_r, bias, logits, ids, gates, partial, blockcnt, s);
  if (nbw <= 2) return launch_route_nbw<2>(p, X, W_r, bias, logits, ids, gates, partial, blockcnt, s);
  if (nbw <= 4) return launch_route_nbw<4>(p, X, W_r, bias, logits, ids, gates, partial, blockcnt, s);
  return launch_route_nbw<8>(p, X, W_r, bias, logits, ids, gates, partial, blockcnt, s);
}

}  // namespace moe
