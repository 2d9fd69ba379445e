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
//                 the top min(K, N_r) rows and min(K, N_c) columns by
//                 (score desc, id asc) -- a bitwise threshold search with
//                 ballot counts, not a sort -- then the top K of the
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

// Order-preserving int32 key of a float: signed order of the key = order of
// the value (the wave max of floats runs as an integer DPP reduction).
__device__ __forceinline__ int skey(float v) {
  const uint32_t b = __float_as_uint(v);
  return (int)((b & 0x80000000u) ? ~b : (b | 0x80000000u)) ^ (int)0x80000000u;
}
__device__ __forceinline__ float unskey(int k) {
  const uint32_t o = (uint32_t)k ^ 0x80000000u;
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);
}
// all-reduce over the wave: within 16-lane rows by DPP, then the 4 rows
__device__ __forceinline__ int wave_max_i(int x) {
  x = max(x, dpp<0xB1>(x));    // quad_perm [1,0,3,2]
  x = max(x, dpp<0x4E>(x));    // quad_perm [2,3,0,1]
  x = max(x, dpp<0x141>(x));   // row_half_mirror
  x = max(x, dpp<0x140>(x));   // row_mirror
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
__device__ __forceinline__ float dppf(float x, int ctrl_sel) {
  const int v = __float_as_int(x);
  return __int_as_float(ctrl_sel == 0 ? dpp<0xB1>(v) : ctrl_sel == 1 ? dpp<0x4E>(v)
                                     : ctrl_sel == 2 ? dpp<0x141>(v) : dpp<0x140>(v));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dppf(x, 0);
  x += dppf(x, 1);
  x += dppf(x, 2);
  x += dppf(x, 3);
  return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48)));
}
__device__ __forceinline__ float wave_maxf(float x) {
  return unskey(wave_max_i(skey(x)));
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

// Unsigned order-preserving key of a float (0 is below every finite value,
// so it marks an empty slot).
__device__ __forceinline__ uint32_t ukey(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unukey(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int wave_count(bool p) { return __popcll(__ballot(p)); }

// Top r (1 <= r <= 64) of the wave's entries -- S slots per lane, entry
// (u, lane) with key k[u] (0 = empty) and a distinct id i[u] < 2^17 -- by
// (key desc, id asc).  Lane q < r receives the q-th key and id.
// Without a sort: the r-th largest key th by a bitwise search with ballot
// counts (over the bits below the common prefix of the largest and the
// smallest non-empty key), the ties at th, when not all are taken, resolved
// by the same search over ids, the winners
// compacted to lanes 0..r-1 through LDS, then each winner's rank counted
// against the others (readlane broadcasts) and the winners placed by rank.
// Ballot counts and the searches run on the scalar unit.
template <int S>
__device__ __forceinline__ void wave_top(const uint32_t* k, const int* id, int r, uint32_t* ok,
                                         int* oi, int* lk, int* li) {
  const int lane = threadIdx.x & 63;
  // th is a non-empty key (r never exceeds the non-empty entries), so it
  // lies in [smallest non-empty key, largest key] and shares their common
  // high bits: the search starts below the highest bit where they differ.
  // Keys are compared as signed ints after flipping the top bit.
  int smax = (int)0x80000000, snot = (int)0x80000000;   // max of s, max of ~s
#pragma unroll
  for (int u = 0; u < S; ++u) {
    const int sk = (int)(k[u] ^ 0x80000000u);
    smax = max(smax, sk);
    if (k[u] != 0u) snot = max(snot, ~sk);
  }
  const uint32_t kmax = (uint32_t)wave_max_i(smax) ^ 0x80000000u;
  const uint32_t kmin = (uint32_t)(~wave_max_i(snot)) ^ 0x80000000u;
  const uint32_t diff = kmax ^ kmin;
  const int top = diff ? 31 - __builtin_clz(diff) : -1;
  uint32_t th = (top >= 0) ? (kmax & ~((2u << top) - 1u)) : kmax;
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = th | (1u << bit);
    int c = 0;
#pragma unroll
    for (int u = 0; u < S; ++u) c += wave_count(k[u] >= cand);
    if (c >= r) th = cand;
  }
  int gt = 0, eq = 0;
#pragma unroll
  for (int u = 0; u < S; ++u) {
    gt += wave_count(k[u] > th);
    eq += wave_count(k[u] == th);
  }
  const int need = r - gt;                       // ties at th to take, lowest ids first
  int x = (1 << 17) - 1;                         // every tie taken (the usual case: th unique)
  if (need < eq) {
    x = 0;                                       // the need-th smallest id among the ties
    for (int bit = 16; bit >= 0; --bit) {
      const int cand = x | (1 << bit);
      int c = 0;
#pragma unroll
      for (int u = 0; u < S; ++u) c += wave_count(k[u] == th && id[u] < cand);
      if (c < need) x = cand;
    }
  }
  // compact the r winners to positions 0..r-1 (slot-major, lane order)
  const uint64_t below = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int u = 0; u < S; ++u) {
    const bool sel = k[u] > th || (k[u] == th && id[u] <= x);
    const uint64_t m = __ballot(sel);
    if (sel) {
      const int pos = base + __popcll(m & below);
      lk[pos] = (int)k[u];
      li[pos] = id[u];
    }
    base += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint32_t mk = lane < r ? (uint32_t)lk[lane] : 0u;
  const int mi = lane < r ? li[lane] : 0x7FFFFFFF;
  int rank = 0;
  for (int q = 0; q < r; ++q) {
    const uint32_t kq = (uint32_t)__builtin_amdgcn_readlane((int)mk, q);
    const int iq = __builtin_amdgcn_readlane(mi, q);
    rank += (kq > mk || (kq == mk && iq < mi)) ? 1 : 0;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < r) {
    lk[64 + rank] = (int)mk;
    li[64 + rank] = mi;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  *ok = lane < r ? (uint32_t)lk[64 + lane] : 0u;
  *oi = lane < r ? li[64 + lane] : 0;
}

__global__ __launch_bounds__(kThreads) void omni_select_kernel(
    const float* __restrict__ p_r, const float* __restrict__ p_c, float* __restrict__ ls_r,
    float* __restrict__ ls_c, int32_t* __restrict__ ids, float* __restrict__ gates, int64_t T,
    int Nr, int Nc, int K) {
  __shared__ int ckey[kWaves][kMaxCand];
  __shared__ int cid[kWaves][kMaxCand];
  __shared__ int tk[kWaves][128];
  __shared__ int ti[kWaves][128];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * kWaves + wv;
  if (t >= T) return;                                  // wave-uniform; no block barrier below
  float vr[4], vc[4];
  axis_log_softmax(p_r + t * Nr, Nr, ls_r ? ls_r + t * Nr : nullptr, vr);
  axis_log_softmax(p_c + t * Nc, Nc, ls_c ? ls_c + t * Nc : nullptr, vc);
  const int R = K < Nr ? K : Nr, C = K < Nc ? K : Nc;
  uint32_t kr[4], kc[4];
  int ir[4], ic[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = lane + 64 * j;
    kr[j] = i < Nr ? ukey(vr[j]) : 0u;
    kc[j] = i < Nc ? ukey(vc[j]) : 0u;
    ir[j] = ic[j] = i;
  }
  uint32_t rk, ck;
  int ri, ci;
  wave_top<4>(kr, ir, R, &rk, &ri, tk[wv], ti[wv]);
  wave_top<4>(kc, ic, C, &ck, &ci, tk[wv], ti[wv]);
  const float rv = unukey(rk), cv = unukey(ck);
  // candidate pairs (i, j) of axis ranks with (i+1)(j+1) <= K; lane j holds
  // column rank j, row rank i is broadcast
  int* cks = ckey[wv];
  int* cis = cid[wv];
  int nc = 0;
  for (int i = 0; i < R; ++i) {
    int jmax = K / (i + 1);
    jmax = jmax < C ? jmax : C;
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rv), i));
    const int ar = __builtin_amdgcn_readlane(ri, i);
    if (lane < jmax) {
      cks[nc + lane] = (int)ukey(a + cv);
      cis[nc + lane] = ar * Nc + ci;
    }
    nc += jmax;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int kPer = (kMaxCand + 63) / 64;
  uint32_t mk[kPer];
  int mi[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = lane + 64 * u;
    mk[u] = c < nc ? (uint32_t)cks[c] : 0u;
    mi[u] = c < nc ? cis[c] : (1 << 17);
  }
  uint32_t sk;
  int sid;
  wave_top<kPer>(mk, mi, K, &sk, &sid, tk[wv], ti[wv]);
  const float sv = unukey(sk);
  // gates: softmax over the K selected sums (lane 0 holds the largest)
  const float s0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), 0));
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

// Exclusive scan over N <= 65536 counts in two launches of N/1024
// workgroups: block sums, then each block adds the sums before it and scans
// its own 1024 counts (thread q owns 4 consecutive ones: coalesced 16-byte
// accesses).
constexpr int kScanBlock = 4 * kThreads;
__device__ __forceinline__ void load4(const int32_t* p, int base, int N, int v[4]) {
  if (base + 3 < N) {
    const int4 q = *reinterpret_cast<const int4*>(p + base);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = base + r < N ? p[base + r] : 0;
  }
}
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__global__ __launch_bounds__(kThreads) void omni_blocksum_kernel(const int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ bsum, int N) {
  __shared__ int tmp[kWaves];
  int v[4];
  load4(counts, blockIdx.x * kScanBlock + 4 * threadIdx.x, N, v);
  const int s = wave_sum_i(v[0] + v[1] + v[2] + v[3]);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) bsum[blockIdx.x] = (tmp[0] + tmp[1]) + (tmp[2] + tmp[3]);
}

__global__ __launch_bounds__(kThreads) void omni_scan_kernel(const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ bsum,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ cursor, int N) {
  __shared__ int tmp[kWaves];
  __shared__ int carry_sh;
  const int q = threadIdx.x, lane = q & 63, w = q >> 6;
  const int b = blockIdx.x;
  if (w == 0) {                                   // blocks before this one (b <= 64)
    const int c = wave_sum_i(lane < b ? bsum[lane] : 0);
    if (lane == 0) carry_sh = c;
  }
  const int base = b * kScanBlock + 4 * q;
  int v[4];
  load4(counts, base, N, v);
  const int mine = (v[0] + v[1]) + (v[2] + v[3]);
  int x = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    x += lane >= o ? y : 0;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int before = carry_sh, total = 0;
#pragma unroll
  for (int j = 0; j < kWaves; ++j) {
    total += tmp[j];
    before += j < w ? tmp[j] : 0;
  }
  int o[4];
  o[0] = before + x - mine;
  o[1] = o[0] + v[0];
  o[2] = o[1] + v[1];
  o[3] = o[2] + v[2];
  if (base + 3 < N) {
    *reinterpret_cast<int4*>(offsets + base) = int4{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<int4*>(cursor + base) = int4{o[0], o[1], o[2], o[3]};
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (base + r < N) {
        offsets[base + r] = o[r];
        cursor[base + r] = o[r];
      }
  }
  if (b == (int)gridDim.x - 1 && q == 0) offsets[N] = carry_sh + total;
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
// A lane owns NCH 8-element chunks (lane, lane+64, ...) of a d-row; NCH =
// ceil(d / 512) keeps the registers, and so the waves per SIMD, to what d needs.
template <int NCH>
__device__ __forceinline__ void load_row(const uint16_t* row, int nchunk, u32x4* q) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    q[c] = ch < nchunk ? *reinterpret_cast<const u32x4*>(row + ch * 8) : u32x4{0u, 0u, 0u, 0u};
  }
}
// The same with the non-temporal hint, for the expert tables: w_in rows are
// read once and w_out rows a few times far apart, so caching them only
// evicts the token rows that are re-read (the layer about 4% faster).
template <int NCH>
__device__ __forceinline__ void load_row_nt(const uint16_t* row, int nchunk, u32x4* q) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    q[c] = ch < nchunk ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + ch * 8)) : u32x4{0u, 0u, 0u, 0u};
  }
}
template <int NCH>
__device__ __forceinline__ float dot_rows(const u32x4* a, const float* w) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      s = fmaf(dev::bf16_bits_to_f32(a[c][h] & 0xFFFFu), w[c * 8 + 2 * h], s);
      s = fmaf(dev::bf16_bits_to_f32(a[c][h] >> 16), w[c * 8 + 2 * h + 1], s);
    }
  return s;
}

// One wave per expert: w_in once, then its tokens four at a time (their
// rows loaded together), a[s] = silu(x . w_in).
template <int NCH>
__global__ __launch_bounds__(kThreads) void omni_expert_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W_in,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, float* __restrict__ a,
    int N, int d) {
  constexpr int kTasks = 4;
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (e >= N) return;
  const int off = offsets[e], c = offsets[e + 1] - off;
  if (c == 0) return;
  const int nchunk = d / 8;
  float w[NCH * 8];
  {
    u32x4 q[NCH];
    load_row_nt<NCH>(W_in + (int64_t)e * d, nchunk, q);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        w[ch * 8 + 2 * h] = dev::bf16_bits_to_f32(q[ch][h] & 0xFFFFu);
        w[ch * 8 + 2 * h + 1] = dev::bf16_bits_to_f32(q[ch][h] >> 16);
      }
  }
  for (int s0 = 0; s0 < c; s0 += kTasks) {
    u32x4 x[kTasks][NCH];
#pragma unroll
    for (int u = 0; u < kTasks; ++u) {
      const int s = off + (s0 + u < c ? s0 + u : c - 1);
      const int t = __builtin_amdgcn_readfirstlane(perm[s]);
      load_row<NCH>(X + (int64_t)t * d, nchunk, x[u]);
    }
#pragma unroll
    for (int u = 0; u < kTasks; ++u) {
      const float dot = wave_sum(dot_rows<NCH>(x[u], w));
      if (lane == 0 && s0 + u < c) a[off + s0 + u] = dot * dev::sigmoid(dot);
    }
  }
}

// One wave per token: lane k first loads the token's id and coefficient
// g_k * a[slot] for entry k (so the row loads below depend on nothing but a
// broadcast), then rows go in groups (16 for d <= 1024) with all their
// loads in flight.
template <int NCH>
__global__ __launch_bounds__(kThreads) void omni_combine_kernel(
    const uint16_t* __restrict__ W_out, const int32_t* __restrict__ ids,
    const float* __restrict__ gates, const int32_t* __restrict__ inv, const float* __restrict__ a,
    uint16_t* __restrict__ Y, int64_t T, int d, int K) {
  constexpr int KG = NCH >= 4 ? 32 / NCH : 16;   // 16-byte loads in flight: 16..32 per lane
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nchunk = d / 8;
  int myid = 0;
  float mycoef = 0.f;
  if (lane < K) {
    const int64_t tk = t * K + lane;
    myid = ids[tk];
    mycoef = gates[tk] * a[inv[tk]];
  }
  float acc[NCH * 8];
#pragma unroll
  for (int v = 0; v < NCH * 8; ++v) acc[v] = 0.f;
  for (int k0 = 0; k0 < K; k0 += KG) {
    u32x4 q[KG][NCH];
#pragma unroll
    for (int u = 0; u < KG; ++u) {
      const int k = k0 + u < K ? k0 + u : K - 1;
      const int row = __builtin_amdgcn_readlane(myid, k);
      load_row_nt<NCH>(W_out + (int64_t)row * d, nchunk, q[u]);
    }
#pragma unroll
    for (int u = 0; u < KG; ++u) {
      const int k = k0 + u < K ? k0 + u : K - 1;
      const float cf = k0 + u < K ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mycoef), k)) : 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc[c * 8 + 2 * h] = fmaf(cf, dev::bf16_bits_to_f32(q[u][c][h] & 0xFFFFu), acc[c * 8 + 2 * h]);
          acc[c * 8 + 2 * h + 1] = fmaf(cf, dev::bf16_bits_to_f32(q[u][c][h] >> 16), acc[c * 8 + 2 * h + 1]);
        }
    }
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nchunk) {
      u32x4 out;
#pragma unroll
      for (int h = 0; h < 4; ++h) out[h] = dev::pack_bf16x2(acc[c * 8 + 2 * h], acc[c * 8 + 2 * h + 1]);
      *reinterpret_cast<u32x4*>(Y + t * (int64_t)d + ch * 8) = out;
    }
  }
}

// The router GEMM's problem for one axis (top-1 outputs go to scratch).
Problem axis_problem(const OmniProblem& p, int E) {
  Problem q{};
  q.T = p.T;
  q.d = p.d;
  q.E = E;
  q.K = 1;
  q.n = 64;
  q.bf16 = true;
  q.C = p.T;
  q.rows_max = p.T;
  return q;
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
  ws.bsum = reinterpret_cast<int32_t*>(take(64 * 4));
  if (w) *w = ws;
  return off;
}

hipError_t launch_omni_route(const OmniProblem& p, const void* X, const void* W_r, const void* W_c,
                             float* ls_r, float* ls_c, int32_t* ids, float* gates,
                             const OmniRouteWs& w, hipStream_t s) {
  // the two axis projections: the router GEMM with fp32 logits out.  Both in
  // one launch where the widths allow it (twice the workgroups of one axis,
  // which alone fills a quarter of the chip at T = 4096); otherwise one
  // launch per axis, their top-1 outputs going to scratch.
  // (no k split: its extra selection pass costs more than it saves here)
  hipError_t err;
  if (route_pair_supported(p.Nr, p.Nc)) {
    err = launch_logits_pair(p.T, p.d, p.Nr, p.Nc, X, W_r, W_c, w.p_r, w.p_c, s);
    if (err != hipSuccess) return err;
  } else {
    err = launch_route(axis_problem(p, p.Nr), X, W_r, nullptr, w.p_r, w.ids1, w.gates1, nullptr, s);
    if (err != hipSuccess) return err;
    err = launch_route(axis_problem(p, p.Nc), X, W_c, nullptr, w.p_c, w.ids1, w.gates1, nullptr, s);
    if (err != hipSuccess) return err;
  }
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
  const unsigned nb = (unsigned)((N + kScanBlock - 1) / kScanBlock);
  hipLaunchKernelGGL(omni_blocksum_kernel, dim3(nb), dim3(kThreads), 0, s, counts, w.bsum, N);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(omni_scan_kernel, dim3(nb), dim3(kThreads), 0, s, counts, w.bsum, offsets,
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
  const dim3 eg((unsigned)((N + kWaves - 1) / kWaves));
  const int nch = (p.d + 511) / 512;
  auto run = [&](auto kern) {
    hipLaunchKernelGGL(kern, eg, dim3(kThreads), 0, s, (const uint16_t*)X, (const uint16_t*)W_in,
                       offsets, perm, a, N, p.d);
  };
  if (nch <= 1) run(omni_expert_kernel<1>);
  else if (nch <= 2) run(omni_expert_kernel<2>);
  else if (nch <= 4) run(omni_expert_kernel<4>);
  else run(omni_expert_kernel<8>);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 cg((unsigned)((p.T + kWaves - 1) / kWaves));
  auto comb = [&](auto kern) {
    hipLaunchKernelGGL(kern, cg, dim3(kThreads), 0, s, (const uint16_t*)W_out, ids, gates, inv, a,
                       (uint16_t*)Y, p.T, p.d, p.K);
  };
  if (nch <= 1) comb(omni_combine_kernel<1>);
  else if (nch <= 2) comb(omni_combine_kernel<2>);
  else if (nch <= 4) comb(omni_combine_kernel<4>);
  else comb(omni_combine_kernel<8>);
  return hipGetLastError();
}

}  // namespace moe
