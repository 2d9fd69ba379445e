// Step 8 of the layer: gate-weighted combine back to token order.
//
// Y[t] = sum over k = 0..K-1 with inv_slot[t,k] >= 0 of gates[t,k] * O[inv_slot[t,k]]
// (SonicMoE article §1 for the weighted sum, §6.1 for doing the scatter and
// the sum in one aggregation kernel).  One wave owns one token: it reads the
// token's K expert rows of O with 16-byte loads (the K loads of a chunk are
// independent, so they are all in flight together), accumulates in fp32 in k
// order and writes the row once.  Every output row has exactly one writer,
// so no atomics are needed and the result is deterministic.
#include "moe_internal.hpp"

namespace moe {
namespace {

using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
using f32x4 = float __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTokPerBlock = kThreads / 64;

// bf16, 8 elements per 16-byte chunk.  The token index is wave-uniform; each
// group of 8 slots and gates is read with one vector load and broadcast with
// readlane, so they live in scalar registers.  A lane owns CB chunks of the row
// (64 lanes x CB x 16 bytes = 2048 bf16 with CB = 4) and issues the loads of
// all of them for KG experts at once (KG = 2, 4 or 8: the least >= K) -- one
// memory round trip per token row block -- then accumulates in k order.
// Dropped assignments point their load at a kept row of the same token (no
// extra HBM traffic) and are left out of the sum by a select, so the load
// sequence has no branches.  A group with no kept entry at all issues no
// loads (a wave-uniform branch): pointing them at row 0 of O made that row
// one hot spot in L2 for every token without a kept row.  O is read once
// and Y written once, both with the non-temporal hint (9% faster than cached
// accesses at the Qwen3 shape: the stream does not fill L2).
template <int CB, int KG>
__global__ __launch_bounds__(kThreads) void combine_bf16(const uint16_t* __restrict__ O,
                                                        const float* __restrict__ gates,
                                                        const int32_t* __restrict__ inv,
                                                        uint16_t* __restrict__ Y, int64_t T, int d,
                                                        int K) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)__builtin_amdgcn_readfirstlane(
      (int)(blockIdx.x * kTokPerBlock + (threadIdx.x >> 6)));
  if (t >= T) return;
  const int nchunk = d / 8;
  const int32_t* tinv = inv + t * K;
  const float* tg = gates + t * K;
  for (int c0 = 0; c0 < nchunk; c0 += 64 * CB) {
    int fallback = 0;                         // a kept row of this token (row 0 if none yet)
    float acc[CB][8];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[cb][v] = 0.f;
    int cc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = c0 + 64 * cb + lane;
      cc[cb] = (c < nchunk) ? c : 0;
    }
    for (int k0 = 0; k0 < K; k0 += KG) {
      int sl[KG];
      float gk[KG];
      bool ok[KG];
      {
        // lane u (mod KG) loads entry k0+u (clamped), then every value is
        // broadcast: one memory round trip for the group's metadata
        const int kk = (k0 + (lane & (KG - 1)) < K) ? k0 + (lane & (KG - 1)) : K - 1;
        const int ms = tinv[kk];
        const float mg = tg[kk];
#pragma unroll
        for (int u = 0; u < KG; ++u) {
          sl[u] = __builtin_amdgcn_readlane(ms, u);
          gk[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mg), u));
          ok[u] = (k0 + u < K) && sl[u] >= 0;
        }
      }
      bool any = false;
#pragma unroll
      for (int u = 0; u < KG; ++u) any = any || ok[u];
      if (!any) continue;                     // nothing kept in this group: no loads
#pragma unroll
      for (int u = KG - 1; u >= 0; --u) fallback = ok[u] ? sl[u] : fallback;
#pragma unroll
      for (int u = 0; u < KG; ++u) sl[u] = ok[u] ? sl[u] : fallback;
      u32x4 o[KG][CB];
#pragma unroll
      for (int u = 0; u < KG; ++u)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          o[u][cb] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(O + (int64_t)sl[u] * d + cc[cb] * 8));
#pragma unroll
      for (int u = 0; u < KG; ++u)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const float lo = fmaf(gk[u], dev::bf16_bits_to_f32(o[u][cb][h] & 0xFFFFu), acc[cb][2 * h]);
            const float hi = fmaf(gk[u], dev::bf16_bits_to_f32(o[u][cb][h] >> 16), acc[cb][2 * h + 1]);
            acc[cb][2 * h] = ok[u] ? lo : acc[cb][2 * h];
            acc[cb][2 * h + 1] = ok[u] ? hi : acc[cb][2 * h + 1];
          }
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = c0 + 64 * cb + lane;
      if (c < nchunk) {
        u32x4 out;
#pragma unroll
        for (int h = 0; h < 4; ++h) out[h] = dev::pack_bf16x2(acc[cb][2 * h], acc[cb][2 * h + 1]);
        __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(Y + t * (int64_t)d + c * 8));
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void combine_f32(const float* __restrict__ O,
                                                       const float* __restrict__ gates,
                                                       const int32_t* __restrict__ inv,
                                                       float* __restrict__ Y, int64_t T, int d,
                                                       int K) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nchunk = d / 4;
  for (int c = lane; c < nchunk; c += 64) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
      const int s = inv[t * K + k];
      if (s < 0) continue;
      const float g = gates[t * K + k];
      const f32x4 o = *reinterpret_cast<const f32x4*>(O + (int64_t)s * d + c * 4);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] = fmaf(g, o[v], acc[v]);
    }
    *reinterpret_cast<f32x4*>(Y + t * (int64_t)d + c * 4) = acc;
  }
}

}  // namespace

hipError_t launch_combine(const Problem& p, const void* O, const float* gates,
                          const int32_t* inv_slot, void* Y, hipStream_t s) {
  const dim3 grid((unsigned)((p.T + kTokPerBlock - 1) / kTokPerBlock));
  if (p.bf16 && p.K <= 2)
    hipLaunchKernelGGL((combine_bf16<4, 2>), grid, dim3(kThreads), 0, s, (const uint16_t*)O, gates,
                       inv_slot, (uint16_t*)Y, p.T, p.d, p.K);
  else if (p.bf16 && p.K <= 4)
    hipLaunchKernelGGL((combine_bf16<4, 4>), grid, dim3(kThreads), 0, s, (const uint16_t*)O, gates,
                       inv_slot, (uint16_t*)Y, p.T, p.d, p.K);
  else if (p.bf16)
    hipLaunchKernelGGL((combine_bf16<4, 8>), grid, dim3(kThreads), 0, s, (const uint16_t*)O, gates,
                       inv_slot, (uint16_t*)Y, p.T, p.d, p.K);
  else
    hipLaunchKernelGGL(combine_f32, grid, dim3(kThreads), 0, s, (const float*)O, gates, inv_slot,
                       (float*)Y, p.T, p.d, p.K);
  return hipGetLastError();
}

}  // namespace moe
