// Steps 1-2 of the layer: router logits, softmax + top-K, renormalised gates.
//
// Router scores l = X W_r (+ b) ([P2] "Routing-Free 与 OmniMoE" §1.1: a
// token goes Router -> softmax -> TopK), selection of the K best experts with
// K a run-time value ([P4] "AI芯片如何支持MoE架构" §4.3), gates renormalised
// over the selected experts.
//
// One workgroup = 64 tokens, 4 waves in a 2x2 grid over (32 tokens) x (half of
// the padded expert range).  X rows stream from HBM straight into registers
// in the MFMA A-operand layout (16 B per lane, 4 stages in flight); the
// W_r[k0:k0+64, :] tile is staged in LDS in its natural [k][e] layout and
// read with the gfx950 transpose load (ds_read_b64_tr_b16), so the weights
// need no transpose in memory.  The 64 x E fp32 scores land in LDS, then
// each 16-lane DPP row selects the top K of one token per pass (4 tokens per
// row, interleaved for ILP) on order-preserving int32 keys: integer max / min
// reductions need no NaN canonicalisation, and folding -0.0 into +0.0 before
// keying makes the two zeros tie (then the lower id wins, as the oracle rules).
#include "moe_internal.hpp"

namespace moe {
namespace {

using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using i16x4 = short __attribute__((ext_vector_type(4)));
using f32x4 = float __attribute__((ext_vector_type(4)));
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
template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
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

// Top-K of 64 tokens whose scores sit in LDS (row stride S floats, padded
// columns hold -inf).  Wave w handles tokens 16w..16w+15; DPP row q takes
// tokens 16w+4q+r, r = 0..3; lane i of the row holds experts i + 16j.
// Round results go to ids (global) and, as values, back into the token's own
// LDS row (no longer read) for the gate pass.
template <int V>
__device__ void topk_from_lds(float* L, int S, int64_t t0, int64_t T, int E, int K,
                              int32_t* __restrict__ ids, float* __restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int i = lane & 15;
  constexpr int kRetired = (int)0x80000000;
  int key[4][V];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float* row = L + (16 * w + 4 * q + r) * S;
#pragma unroll
    for (int j = 0; j < V; ++j) key[r][j] = sort_key(row[i + 16 * j]);
  }
  int top[4];
  for (int k = 0; k < K; ++k) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int m = key[r][0];
#pragma unroll
      for (int j = 1; j < V; ++j) m = max(m, key[r][j]);
      m = row_max16(m);
      int cand = 0x7FFFFFFF;
#pragma unroll
      for (int j = V - 1; j >= 0; --j) cand = (key[r][j] == m) ? (i + 16 * j) : cand;
      cand = row_min16(cand);
#pragma unroll
      for (int j = 0; j < V; ++j) key[r][j] = (i + 16 * j == cand) ? kRetired : key[r][j];
      if (k == 0) top[r] = m;
      const int tl = 16 * w + 4 * q + r;
      if (i == 0) {
        L[tl * S + k] = key_value(m);
        if (t0 + tl < T) ids[(t0 + tl) * K + k] = cand;
      }
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  // gates: softmax over the K selected scores (the full-softmax denominator
  // cancels in the renormalisation).
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tl = 16 * w + 4 * q + r;
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

// Shared tail: bias, optional export, selection.
template <int V>
__device__ void route_tail(float* L, int S, int64_t t0, int64_t T, int E, int K, int Epad,
                           const float* __restrict__ bias, float* __restrict__ logits,
                           int32_t* __restrict__ ids, float* __restrict__ gates) {
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
  if (logits) {
    for (int idx = threadIdx.x; idx < kTok * E; idx += kThreads) {
      const int r = idx / E, e = idx - (idx / E) * E;
      if (t0 + r < T) logits[(t0 + r) * E + e] = L[r * S + e];
    }
    __syncthreads();  // selection rewrites the rows being exported
  }
  topk_from_lds<V>(L, S, t0, T, E, K, ids, gates);
}

// ---------------------------------------------------------------- bf16 router (MFMA)
// NBW: 16-column blocks per wave; the padded expert range is 32*NBW.
// The widest expert range (NBW = 8) needs the whole register file: one
// workgroup per CU; narrower ones fit two.
template <int NBW, bool VEC>
__global__ __launch_bounds__(kThreads, (NBW >= 8) ? 1 : 2) void route_bf16_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wr, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ gates, int64_t T,
    int d, int E, int K) {
  constexpr int Epad = 32 * NBW;
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
  __syncthreads();
  route_tail<2 * NBW>(L, S, t0, T, E, K, Epad, bias, logits, ids, gates);
}

// ---------------------------------------------------------------- fp32 router (plain FMA)
template <int NBW>
__global__ __launch_bounds__(kThreads) void route_f32_kernel(
    const float* __restrict__ X, const float* __restrict__ Wr, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ gates, int64_t T,
    int d, int E, int K) {
  constexpr int Epad = 32 * NBW;
  constexpr int S = Epad + 16;
  __shared__ float L[kTok * S];
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  for (int idx = threadIdx.x; idx < kTok * Epad; idx += kThreads) {
    const int r = idx / Epad, e = idx - (idx / Epad) * Epad;
    float s = 0.f;
    if (e < E && t0 + r < T) {
      const float* x = X + (t0 + r) * (int64_t)d;
      for (int i = 0; i < d; ++i) s = fmaf(x[i], Wr[(int64_t)i * E + e], s);
    }
    L[r * S + e] = s;
  }
  __syncthreads();
  route_tail<2 * NBW>(L, S, t0, T, E, K, Epad, bias, logits, ids, gates);
}

template <int NBW>
hipError_t launch_route_nbw(const Problem& p, const void* X, const void* W_r, const float* bias,
                            float* logits, int32_t* ids, float* gates, hipStream_t s) {
  const dim3 grid((unsigned)((p.T + kTok - 1) / kTok));
  if (p.bf16) {
    if (p.E % 8 == 0)
      hipLaunchKernelGGL((route_bf16_kernel<NBW, true>), grid, dim3(kThreads), 0, s,
                         (const uint16_t*)X, (const uint16_t*)W_r, bias, logits, ids, gates, p.T,
                         p.d, p.E, p.K);
    else
      hipLaunchKernelGGL((route_bf16_kernel<NBW, false>), grid, dim3(kThreads), 0, s,
                         (const uint16_t*)X, (const uint16_t*)W_r, bias, logits, ids, gates, p.T,
                         p.d, p.E, p.K);
  } else {
    hipLaunchKernelGGL((route_f32_kernel<NBW>), grid, dim3(kThreads), 0, s, (const float*)X,
                       (const float*)W_r, bias, logits, ids, gates, p.T, p.d, p.E, p.K);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const Problem& p, const void* X, const void* W_r, const float* bias,
                        float* logits, int32_t* ids, float* gates, hipStream_t s) {
  const int nbw = (p.E + 31) / 32;
  if (nbw <= 1) return launch_route_nbw<1>(p, X, W_r, bias, logits, ids, gates, s);
  if (nbw <= 2) return launch_route_nbw<2>(p, X, W_r, bias, logits, ids, gates, s);
  if (nbw <= 4) return launch_route_nbw<4>(p, X, W_r, bias, logits, ids, gates, s);
  return launch_route_nbw<8>(p, X, W_r, bias, logits, ids, gates, s);
}

}  // namespace moe
