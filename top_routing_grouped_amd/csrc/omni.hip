// Atomic-expert layer with a Cartesian-product router (the OmniMoE design on
// the page "MoE 的两个上游创新：Routing-Free 与 OmniMoE", part 2):
//
//   §2.1  expert i is two d-vectors: E_i(x) = silu(x . w_in_i) w_out_i
//         (sigma = SiLU; the routing weight plays SwiGLU's gating role);
//   §2.2  i = i_r * N_c + i_c; p_r = x W_r, p_c = x W_c; the score of (i_r, i_c)
//         is ls_r[i_r] + ls_c[i_c] with ls the log-softmax of each axis; the
//         top-K is searched among the top rows and columns of each axis;
//   §2.3  the L*K tasks run expert by expert in (expert, token) order, each
//         expert's vectors read once for all its tokens, and the outputs are
//         summed back per token.
//
// Kernels (after the two axis projections, which reuse the router GEMM):
//   omni_select   one wave per token: log-softmax of both axes (exported),
//                 the top min(K, N_r) rows and min(K, N_c) columns by repeated
//                 wave arg-max on (score, -id) keys, then the top K of the
//                 row+column sums among the pairs (i, j) of axis ranks with
//                 (i+1)(j+1) <= K (a pair with more than K-1 pairs ranked
//                 above it cannot be in the top K); gates = softmax over the
//                 K selected sums.  The pruning is exact: every top-K pair
//                 uses a top-K row and a top-K column.
//   omni_count / omni_scan / omni_scatter / omni_rank
//                 (expert, token) permutation over N = N_r*N_c experts:
//                 counts, exclusive scan, a scatter into each expert's segment
//                 in arrival order, then one wave per expert ranks its entries
//                 by token (distinct keys) so the order is deterministic;
//   omni_expert   one wave per active expert: w_in loaded once, then for each
//                 of its tokens a[s] = silu(x_t . w_in) (fp32 dot, wave sum);
//   omni_combine  one wave per token: y_t = sum_k g_k a[slot] w_out[id_k]
//                 (fp32 in k order, no atomics).
#include "moe_internal.hpp"

namespace moe {
namespace {

using u32x4 = uint32_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxAxis = 256;             // N_r, N_c <= 256: 4 scores per lane
constexpr int kMaxK = 64;
constexpr int kMaxCand = 320;             // >= sum over i = 1..64 of floor(64 / i) = 280

__device__ __forceinline__ uint32_t ord(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unord(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
// key ordering (score desc, id asc) as an unsigned max
__device__ __forceinline__ uint64_t mkkey(float v, uint32_t id) {
  return ((uint64_t)ord(v) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint64_t wave_max64(uint64_t k) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)k, o), hi = __shfl_xor((uint32_t)(k >> 32), o);
    const uint64_t other = ((uint64_t)hi << 32) | lo;
    k = other > k ? other : k;
  }
  return k;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_maxf(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Log-softmax of one axis row (n <= 256 scores, lane holds entries lane + 64 j);
// exports it when `out` is given; returns the lane's values (-inf padding).
__device__ __forceinline__ void axis_log_softmax(const float* p, int n, float* out, float v[4]) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = lane + 64 * j;
    v[j] = i < n ? p[i] : -INFINITY;
    m = fmaxf(m, v[j]);
  }
  m = wave_maxf(m);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += (lane + 64 * j < n) ? __expf(v[j] - m) : 0.f;
  const float lse = m + __logf(wave_sum(s));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = lane + 64 * j;
    if (i < n) {
      v[j] = v[j] - lse;
      if (out) out[i] = v[j];
    }
  }
}

// The top r entries of an axis by (score desc, id asc): lane q < r receives
// the q-th (score, id).
__device__ __forceinline__ void axis_top(const float v[4], int n, int r, float* tv, int* ti) {
  const int lane = threadIdx.x & 63;
  uint64_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = lane + 64 * j;
    key[j] = i < n ? mkkey(v[j], (uint32_t)i) : 0ull;
  }
  for (int q = 0; q < r; ++q) {
    uint64_t best = key[0];
#pragma unroll
    for (int j = 1; j < 4; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max64(best);
    const int id = (int)(0xFFFFFFFFu - (uint32_t)best);
    if (lane == q) {
      *tv = unord((uint32_t)(best >> 32));
      *ti = id;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == id) key[j] = 0ull;     // retire the winner
  }
}

__global__ __launch_bounds__(kThreads) void omni_select_kernel(
    const float* __restrict__ p_r, const float* __restrict__ p_c, float* __restrict__ ls_r,
    float* __restrict__ ls_c, int32_t* __restrict__ ids, float* __restrict__ gates, int64_t T,
    int Nr, int Nc, int K) {
  __shared__ uint64_t cand[kWaves][kMaxCand];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * kWaves + wv;
  if (t >= T) return;                                  // wave-uniform; no block barrier below
  float vr[4], vc[4];
  axis_log_softmax(p_r + t * Nr, Nr, ls_r ? ls_r + t * Nr : nullptr, vr);
  axis_log_softmax(p_c + t * Nc, Nc, ls_c ? ls_c + t * Nc : nullptr, vc);
  const int R = K < Nr ? K : Nr, C = K < Nc ? K : Nc;
  float rv = 0.f, cv = 0.f;
  int ri = 0, ci = 0;
  axis_top(vr, Nr, R, &rv, &ri);
  axis_top(vc, Nc, C, &cv, &ci);
  // candidate pairs (i, j) of axis ranks with (i+1)(j+1) <= K; lane j holds
  // column rank j, row rank i is broadcast
  uint64_t* cl = cand[wv];
  int nc = 0;
  for (int i = 0; i < R; ++i) {
    int jmax = K / (i + 1);
    jmax = jmax < C ? jmax : C;
    const float a = __shfl(rv, i);
    const int ar = __shfl(ri, i);
    if (lane < jmax) cl[nc + lane] = mkkey(a + cv, (uint32_t)(ar * Nc + ci));
    nc += jmax;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // top K of the candidates; lane q receives the q-th
  float sv = 0.f;
  int sid = 0;
  for (int q = 0; q < K; ++q) {
    uint64_t best = 0ull;
    int where = -1;
    for (int c = lane; c < nc; c += 64) {
      const uint64_t k = cl[c];
      if (k > best) { best = k; where = c; }
    }
    const uint64_t top = wave_max64(best);
    if (best == top && where >= 0) cl[where] = 0ull;  // keys are distinct (ids differ)
    if (lane == q) {
      sv = unord((uint32_t)(top >> 32));
      sid = (int)(0xFFFFFFFFu - (uint32_t)top);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // gates: softmax over the K selected sums (lane 0 holds the largest)
  const float s0 = __shfl(sv, 0);
  const float ex = lane < K ? __expf(sv - s0) : 0.f;
  const float z = wave_sum(ex);
  if (lane < K) {
    ids[t * K + lane] = sid;
    gates[t * K + lane] = ex / z;
  }
}

// ---------------------------------------------------------------- permutation
__global__ __launch_bounds__(kThreads) void omni_zero_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(kThreads) void omni_count_kernel(const int32_t* __restrict__ ids,
                                                              int32_t* __restrict__ counts,
                                                              int64_t TK) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < TK) atomicAdd(&counts[ids[i]], 1);
}

// One workgroup of 1024 threads: thread q owns a contiguous run of experts.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void omni_scan_kernel(const int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ cursor,
                                                                 int N) {
  __shared__ int part[kScanThreads];
  const int q = threadIdx.x;
  const int per = (N + kScanThreads - 1) / kScanThreads;
  const int lo = q * per, hi = (lo + per < N) ? lo + per : N;
  int sum = 0;
  for (int e = lo; e < hi; ++e) sum += counts[e];
  part[q] = sum;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int x = q >= off ? part[q - off] : 0;
    __syncthreads();
    part[q] += x;
    __syncthreads();
  }
  int run = part[q] - sum;
  for (int e = lo; e < hi; ++e) {
    offsets[e] = run;
    cursor[e] = run;
    run += counts[e];
  }
  if (q == kScanThreads - 1) offsets[N] = part[q];
}

__global__ __launch_bounds__(kThreads) void omni_scatter_kernel(const int32_t* __restrict__ ids,
                                                                int32_t* __restrict__ cursor,
                                                                int32_t* __restrict__ tmp_tk,
                                                                int64_t TK) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= TK) return;
  const int s = atomicAdd(&cursor[ids[i]], 1);
  tmp_tk[s] = (int32_t)i;
}

// One wave per expert: each entry's final place is its rank among the
// segment's (token*K + k) keys (distinct), i.e. ascending token order.
__global__ __launch_bounds__(kThreads) void omni_rank_kernel(const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ tmp_tk,
                                                             int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ inv, int N,
                                                             int K) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (e >= N) return;
  const int off = offsets[e], c = offsets[e + 1] - off;
  for (int i0 = 0; i0 < c; i0 += 64) {
    const int i = i0 + lane;
    const int mine = i < c ? tmp_tk[off + i] : 0x7FFFFFFF;
    int rank = 0;
    for (int j = 0; j < c; ++j) rank += tmp_tk[off + j] < mine ? 1 : 0;
    if (i < c) {
      perm[off + rank] = mine / K;
      inv[mine] = off + rank;
    }
  }
}

// ---------------------------------------------------------------- experts
// d <= 4096: a lane owns 8-element chunks lane, lane+64, ... of the row.
constexpr int kMaxChunks = 8;

__device__ __forceinline__ void load_row(const uint16_t* row, int nchunk, float* v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int ch = lane + 64 * c;
    if (c * 64 < nchunk) {
      u32x4 q = {0u, 0u, 0u, 0u};
      if (ch < nchunk) q = *reinterpret_cast<const u32x4*>(row + ch * 8);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v[c * 8 + 2 * h] = dev::bf16_bits_to_f32(q[h] & 0xFFFFu);
        v[c * 8 + 2 * h + 1] = dev::bf16_bits_to_f32(q[h] >> 16);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void omni_expert_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W_in,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, float* __restrict__ a,
    int N, int d) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (e >= N) return;
  const int off = offsets[e], c = offsets[e + 1] - off;
  if (c == 0) return;
  const int nchunk = d / 8;
  float w[kMaxChunks * 8];
  load_row(W_in + (int64_t)e * d, nchunk, w);
  for (int s = off; s < off + c; ++s) {
    const int t = __builtin_amdgcn_readfirstlane(perm[s]);
    float x[kMaxChunks * 8];
    load_row(X + (int64_t)t * d, nchunk, x);
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxChunks * 8; ++i)
      if ((i / 8) * 64 < nchunk) dot = fmaf(x[i], w[i], dot);
    dot = wave_sum(dot);
    if (lane == 0) a[s] = dot * dev::sigmoid(dot);
  }
}

__global__ __launch_bounds__(kThreads) void omni_combine_kernel(
    const uint16_t* __restrict__ W_out, const int32_t* __restrict__ ids,
    const float* __restrict__ gates, const int32_t* __restrict__ inv, const float* __restrict__ a,
    uint16_t* __restrict__ Y, int64_t T, int d, int K) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nchunk = d / 8;
  for (int c0 = lane; c0 < nchunk; c0 += 64) {
    float acc[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[v] = 0.f;
    constexpr int KG = 8;                       // rows in flight per group
    for (int k0 = 0; k0 < K; k0 += KG) {
      u32x4 q[KG];
      float coef[KG];
#pragma unroll
      for (int u = 0; u < KG; ++u) {
        const int k = k0 + u < K ? k0 + u : K - 1;
        const int64_t tk = t * K + k;
        coef[u] = k0 + u < K ? gates[tk] * a[inv[tk]] : 0.f;
        q[u] = *reinterpret_cast<const u32x4*>(W_out + (int64_t)ids[tk] * d + c0 * 8);
      }
#pragma unroll
      for (int u = 0; u < KG; ++u)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc[2 * h] = fmaf(coef[u], dev::bf16_bits_to_f32(q[u][h] & 0xFFFFu), acc[2 * h]);
          acc[2 * h + 1] = fmaf(coef[u], dev::bf16_bits_to_f32(q[u][h] >> 16), acc[2 * h + 1]);
        }
    }
    u32x4 out;
#pragma unroll
    for (int h = 0; h < 4; ++h) out[h] = dev::pack_bf16x2(acc[2 * h], acc[2 * h + 1]);
    *reinterpret_cast<u32x4*>(Y + t * (int64_t)d + c0 * 8) = out;
  }
}

}  // namespace

size_t omni_route_ws_bytes(const OmniProblem& p, OmniRouteWs* w, unsigned char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* ptr = base ? base + off : nullptr;
    off += (bytes + 255) / 256 * 256;
    return ptr;
  };
  OmniRouteWs ws{};
  ws.p_r = reinterpret_cast<float*>(take((size_t)p.T * p.Nr * 4));
  ws.p_c = reinterpret_cast<float*>(take((size_t)p.T * p.Nc * 4));
  ws.ids1 = reinterpret_cast<int32_t*>(take((size_t)p.T * 4));
  ws.gates1 = reinterpret_cast<float*>(take((size_t)p.T * 4));
  if (w) *w = ws;
  return off;
}

size_t omni_permute_ws_bytes(const OmniProblem& p, OmniPermuteWs* w, unsigned char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* ptr = base ? base + off : nullptr;
    off += (bytes + 255) / 256 * 256;
    return ptr;
  };
  OmniPermuteWs ws{};
  ws.cursor = reinterpret_cast<int32_t*>(take((size_t)p.Nr * p.Nc * 4));
  ws.tmp_tk = reinterpret_cast<int32_t*>(take((size_t)p.T * p.K * 4));
  if (w) *w = ws;
  return off;
}

hipError_t launch_omni_route(const OmniProblem& p, const void* X, const void* W_r, const void* W_c,
                             float* ls_r, float* ls_c, int32_t* ids, float* gates,
                             const OmniRouteWs& w, hipStream_t s) {
  // the two axis projections: the router GEMM with fp32 logits out (top-1
  // outputs go to scratch)
  Problem q{};
  q.T = p.T;
  q.d = p.d;
  q.K = 1;
  q.n = 64;
  q.bf16 = true;
  q.C = p.T;
  q.rows_max = p.T;
  q.E = p.Nr;
  hipError_t err = launch_route(q, X, W_r, nullptr, w.p_r, w.ids1, w.gates1, nullptr, s);
  if (err != hipSuccess) return err;
  q.E = p.Nc;
  err = launch_route(q, X, W_c, nullptr, w.p_c, w.ids1, w.gates1, nullptr, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(omni_select_kernel, dim3((unsigned)((p.T + kWaves - 1) / kWaves)),
                     dim3(kThreads), 0, s, w.p_r, w.p_c, ls_r, ls_c, ids, gates, p.T, p.Nr, p.Nc,
                     p.K);
  return hipGetLastError();
}

hipError_t launch_omni_permute(const OmniProblem& p, const int32_t* ids, int32_t* counts,
                               int32_t* offsets, int32_t* perm, int32_t* inv,
                               const OmniPermuteWs& w, hipStream_t s) {
  const int N = p.Nr * p.Nc;
  const int64_t TK = p.T * (int64_t)p.K;
  const unsigned gN = (unsigned)((N + kThreads - 1) / kThreads);
  const unsigned gTK = (unsigned)((TK + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(omni_zero_kernel, dim3(gN), dim3(kThreads), 0, s, counts, (int64_t)N);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(omni_count_kernel, dim3(gTK), dim3(kThreads), 0, s, ids, counts, TK);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(omni_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, counts, offsets,
                     w.cursor, N);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(omni_scatter_kernel, dim3(gTK), dim3(kThreads), 0, s, ids, w.cursor,
                     w.tmp_tk, TK);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(omni_rank_kernel, dim3((unsigned)((N + kWaves - 1) / kWaves)),
                     dim3(kThreads), 0, s, offsets, w.tmp_tk, perm, inv, N, p.K);
  return hipGetLastError();
}

hipError_t launch_omni_experts(const OmniProblem& p, const void* X, const void* W_in,
                               const void* W_out, const int32_t* ids, const float* gates,
                               const int32_t* offsets, const int32_t* perm, const int32_t* inv,
                               float* a, void* Y, hipStream_t s) {
  const int N = p.Nr * p.Nc;
  hipLaunchKernelGGL(omni_expert_kernel, dim3((unsigned)((N + kWaves - 1) / kWaves)),
                     dim3(kThreads), 0, s, (const uint16_t*)X, (const uint16_t*)W_in, offsets,
                     perm, a, N, p.d);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(omni_combine_kernel, dim3((unsigned)((p.T + kWaves - 1) / kWaves)),
                     dim3(kThreads), 0, s, (const uint16_t*)W_out, ids, gates, inv, a,
                     (uint16_t*)Y, p.T, p.d, p.K);
  return hipGetLastError();
}

}  // namespace moe
