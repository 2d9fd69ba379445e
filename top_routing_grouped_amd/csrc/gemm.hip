// Steps 6-7 of the layer: the two variable-M grouped GEMMs.
//
// up:   H[s,:] = silu(x W_gate[e]) * (x W_up[e]),  x = X[perm_token[s]]
// down: O[s,:] = H[s,:] W_down[e]
// for every expert-major slot s of expert e.  The SonicMoE article lists these
// as steps 3-5 of its GPU pipeline (§3), reads the token rows by index inside
// the GEMM's operand load instead of building a gathered T*K*d copy (§6.2),
// and applies SwiGLU while the products are still in the accumulators (§6.3).
//
// bf16 kernel (gfx950, one 256-thread workgroup per tile, 1 per CU):
// * Tile = 128 expert-major rows x 256 accumulator columns (up: 128 W_gate
//   columns + the same 128 W_up columns, so each lane holds matching gate and
//   up values and SwiGLU is register-local; down: 256 W_down columns).
//   Row tiles come from a device-built table (expert, row range), so experts
//   of any size share one launch; the grid is a host-side upper bound and
//   surplus workgroups exit at once.
// * Loads go global -> LDS with global_load_lds_dwordx4 (no VGPR staging).
//   Each lane supplies its own global address, which is what makes the row
//   gather free: a lane simply points at row perm_token[s] of X.  Three LDS
//   stages of 48 KB keep two k-steps in flight.
// * LDS layouts are XOR-swizzled at 16-byte granularity so both fragment
//   reads are bank-conflict free: token rows (128 B) use slot c^((r>>1)&7);
//   weight rows (512 B, natural [k][n] order) use slot q^(4*(k&3)) and are
//   read with ds_read_b64_tr_b16, which hands each lane 4 consecutive k of
//   one column -- the MFMA operand layout -- so weights are never transposed.
// * The MFMA computes the transposed tile (weights as the A operand, tokens
//   as B), so each lane ends with 4 consecutive output columns of one row and
//   stores 8 bytes at a time.
// * Workgroup ids are remapped so that consecutive tiles (same expert, same
//   token rows) run on the same XCD and share its L2.
#include "moe_internal.hpp"

namespace moe {
namespace {

using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using i16x4 = short __attribute__((ext_vector_type(4)));
using f32x16 = float __attribute__((ext_vector_type(16)));
using u32x2 = uint32_t __attribute__((ext_vector_type(2)));

constexpr int BM = kGemmBM;      // 128 rows (tokens) per tile
constexpr int BN = 256;          // accumulator columns per tile
constexpr int BK = 64;           // k per stage
constexpr int kStages = 3;
constexpr int kThreads = 256;
constexpr int kAStage = BM * BK * 2;        // 16 KB
constexpr int kBStage = BK * BN * 2;        // 32 KB
constexpr int kStageBytes = kAStage + kBStage;
constexpr int kAInstr = kAStage / 1024 / 4; // DMA instructions per wave per stage (4)
constexpr int kBInstr = kBStage / 1024 / 4; // (8)

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16-byte global -> LDS copy per lane; LDS destination = M0 + 16*lane.
// Issued through asm so the compiler does not treat every later LDS read as
// aliasing the copy (it would wait for all copies in flight, which would
// collapse the stage pipeline); completion is awaited explicitly with
// s_waitcnt vmcnt before the barrier that publishes a stage.  The asm has no
// register outputs; the s_nop covers the M0-write -> LDS-DMA hazard.
// M0 is written only here in these kernels (no other instruction reads it),
// so clobbering it is safe; silence the generic reserved-register warning.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_ptr_t)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ float silu_mul(float g, float u) {
  return __fdividef(g, 1.0f + __expf(-g)) * u;
}

template <bool UP>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bf16(
    const uint16_t* __restrict__ A,       // up: X [T][Kd]; down: H [rows][Kd]
    const int32_t* __restrict__ perm,     // up: expert-major slot -> token
    const int32_t* __restrict__ table,    // tile table
    const uint16_t* __restrict__ B0,      // up: W_gate; down: W_down  ([E][Kd][N])
    const uint16_t* __restrict__ B1,      // up: W_up
    uint16_t* __restrict__ C,             // up: H [rows][N]; down: O [rows][N]
    int64_t T, int Kd, int N, int NT) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;

  // ---- tile decode (XCD-aware: consecutive tile ids on one XCD)
  const int total = table[0] * NT;
  const int bid = blockIdx.x;
  if (bid >= total) return;
  const int q8 = total >> 3, r8 = total & 7;
  const int xcd = bid & 7, j = bid >> 3;
  const int L = xcd * q8 + (xcd < r8 ? xcd : r8) + j;
  const int mt = L / NT, nt = L - mt * NT;
  const int32_t* ent = table + 4 * (mt + 1);
  const int e = ent[0], row0 = ent[1];
  const int nrows = ent[2] - row0;
  const int ncol0 = nt * (UP ? BN / 2 : BN);   // first output column of the tile

  // ---- DMA source addresses
  // token tile: instruction i of wave w fills rows (4w+i)*8 + lane/8, slot lane%8
  const uint16_t* asrc[kAInstr];
#pragma unroll
  for (int i = 0; i < kAInstr; ++i) {
    const int r = (w * kAInstr + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int rr = r < nrows ? r : nrows - 1;
    int64_t row;
    if (UP) {
      int64_t tok = perm[row0 + rr];
      tok = tok < 0 ? 0 : (tok > T - 1 ? T - 1 : tok);
      row = tok;
    } else {
      row = row0 + rr;
    }
    asrc[i] = A + row * (int64_t)Kd + c * 8;
  }
  // weight tile: instruction i fills rows 2*(8w+i) + lane/32, slot lane%32;
  // slot -> column chunk depends on the row's k&3 = (2i + lane/32) & 3.
  const uint16_t* bsrc[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int kl = 2 * par + (lane >> 5);
    const int qc = (lane & 31) ^ (4 * (kl & 3));
    const uint16_t* base;
    int col;
    if (UP) {
      base = (qc < 16) ? B0 : B1;
      col = ncol0 + (qc & 15) * 8;
    } else {
      base = B0;
      col = ncol0 + qc * 8;
    }
    if (col >= N) col &= 63;                // in-bounds filler; never stored
    bsrc[par] = base + (int64_t)e * Kd * N + (int64_t)(lane >> 5) * N + col;
  }

  auto issue_stage = [&](int kt, int buf) {
    unsigned char* As = smem + buf * kStageBytes;
    unsigned char* Bs = As + kAStage;
#pragma unroll
    for (int i = 0; i < kAInstr; ++i) dma16(asrc[i] + kt * BK, As + (w * kAInstr + i) * 1024);
#pragma unroll
    for (int i = 0; i < kBInstr; ++i)
      dma16(bsrc[i & 1] + (int64_t)(kt * BK + 2 * (w * kBInstr + i)) * N,
            Bs + (w * kBInstr + i) * 1024);
  };

  // ---- fragment geometry
  // token fragment (MFMA B operand): lane -> token row wm*64 + tb*32 + lane%32, k chunk ks*2 + lane/32
  int a_off[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int r = wm * 64 + tb * 32 + (lane & 31);
      const int c = ks * 2 + (lane >> 5);
      a_off[tb][ks] = r * 128 + ((c ^ ((r >> 1) & 7)) * 16);
    }
  // weight fragment (MFMA A operand) via transpose loads: group g = lane/16,
  // lane s in group -> row ks*16 + 8*(g/2) + s/4 (+4), column n0 + 16*(g%2) + 4*(s%4)
  const int g = lane >> 4, s16 = lane & 15;
  const int tr_row = 8 * (g >> 1) + (s16 >> 2);
  int b_off[4][2];   // [cb][half of k group], byte offset within the stage's weight tile (ks = 0)
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    int colbase;
    if (UP) colbase = (cb < 2) ? (wn * 64 + cb * 32) : (128 + wn * 64 + (cb - 2) * 32);
    else colbase = wn * 128 + cb * 32;
    const int n = colbase + 16 * (g & 1) + 4 * (s16 & 3);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = tr_row + 4 * h;
      const int q = n >> 3;
      b_off[cb][h] = k * 512 + ((q ^ (4 * (k & 3))) * 16) + ((n >> 2) & 1) * 8;
    }
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[cb][tb][v] = 0.f;

  const int KT = Kd / BK;
  issue_stage(0, 0);
  if (KT > 1) issue_stage(1, 1);
  if (KT > 1)
    asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  asm volatile("s_barrier" ::: "memory");

  int buf = 0;
  for (int kt = 0; kt < KT; ++kt) {
    const unsigned char* As = smem + buf * kStageBytes;
    const unsigned char* Bs = As + kAStage;
    bf16x8 af[4][2], bfr[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        af[ks][tb] = *reinterpret_cast<const bf16x8*>(As + a_off[tb][ks]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        // ks advances 16 rows of the weight tile (8 KB); row&3 is unchanged
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(Bs + b_off[cb][0] + ks * 16 * 512));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(Bs + b_off[cb][1] + ks * 16 * 512));
        bfr[ks][cb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
    if (kt + 2 < KT) {
      int nb = buf + 2;
      if (nb >= kStages) nb -= kStages;
      issue_stage(kt + 2, nb);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          acc[cb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ks][cb], af[ks][tb], acc[cb][tb], 0, 0, 0);
    if (kt + 2 < KT)
      asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    buf = (buf + 1 == kStages) ? 0 : buf + 1;
  }

  // ---- epilogue: lane holds, for token column lane%32 of block tb, output
  // columns 8*(v/4) + 4*(lane/32) + v%4 of block cb (v = accumulator index).
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int rloc = wm * 64 + tb * 32 + (lane & 31);
    if (rloc >= nrows) continue;
    uint16_t* crow = C + (int64_t)(row0 + rloc) * N;
    if (UP) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int col = ncol0 + wn * 64 + cb * 32 + 8 * v4 + 4 * (lane >> 5);
          if (col >= N) continue;
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = silu_mul(acc[cb][tb][4 * v4 + r], acc[cb + 2][tb][4 * v4 + r]);
          u32x2 pk = {dev::pack_bf16x2(h[0], h[1]), dev::pack_bf16x2(h[2], h[3])};
          *reinterpret_cast<u32x2*>(crow + col) = pk;
        }
    } else {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int col = ncol0 + wn * 128 + cb * 32 + 8 * v4 + 4 * (lane >> 5);
          if (col >= N) continue;
          u32x2 pk = {dev::pack_bf16x2(acc[cb][tb][4 * v4], acc[cb][tb][4 * v4 + 1]),
                      dev::pack_bf16x2(acc[cb][tb][4 * v4 + 2], acc[cb][tb][4 * v4 + 3])};
          *reinterpret_cast<u32x2*>(crow + col) = pk;
        }
    }
  }
}

// ---------------------------------------------------------------- fp32 (plain FMA)
// 32-row x 64-column tiles, LDS-tiled over k; only for the fp32 element type.
template <bool UP>
__global__ __launch_bounds__(256) void grouped_gemm_f32(
    const float* __restrict__ A, const int32_t* __restrict__ perm, const int32_t* __restrict__ table,
    const float* __restrict__ B0, const float* __restrict__ B1, float* __restrict__ C, int64_t T,
    int Kd, int N, int NT) {
  constexpr int TM = 32, TN = 64, TK = 16;
  __shared__ float As[TM][TK + 1];
  __shared__ float Bg[TK][TN];
  __shared__ float Bu[TK][TN];
  // each 128-row table tile is covered by BM/TM sub-tiles of TM rows
  constexpr int kSub = BM / TM;
  const int total = table[0] * kSub * NT;
  const int bid = blockIdx.x;
  if (bid >= total) return;
  const int mt = bid / (kSub * NT);
  const int rem = bid - mt * (kSub * NT);
  const int sub = rem / NT, nt = rem - (rem / NT) * NT;
  const int32_t* ent = table + 4 * (mt + 1);
  const int e = ent[0], row0 = ent[1] + sub * TM;
  const int nrows = (ent[2] - row0 < TM) ? ent[2] - row0 : TM;
  if (nrows <= 0) return;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float ag[2][4] = {}, au[2][4] = {};
  const float* Wg = B0 + (int64_t)e * Kd * N;
  const float* Wu = UP ? B1 + (int64_t)e * Kd * N : nullptr;
  for (int k0 = 0; k0 < Kd; k0 += TK) {
    for (int idx = tid; idx < TM * TK; idx += 256) {
      const int r = idx / TK, c = idx % TK;
      const int rr = r < nrows ? r : nrows - 1;
      int64_t row;
      if (UP) {
        int64_t tok = perm[row0 + rr];
        row = tok < 0 ? 0 : (tok > T - 1 ? T - 1 : tok);
      } else {
        row = row0 + rr;
      }
      As[r][c] = A[row * Kd + k0 + c];
    }
    for (int idx = tid; idx < TK * TN; idx += 256) {
      const int r = idx / TN, c = idx % TN;
      const int col = nt * TN + c;
      Bg[r][c] = col < N ? Wg[(int64_t)(k0 + r) * N + col] : 0.f;
      if (UP) Bu[r][c] = col < N ? Wu[(int64_t)(k0 + r) * N + col] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float a = As[ty * 2 + i][kk];
#pragma unroll
        for (int jx = 0; jx < 4; ++jx) {
          ag[i][jx] = fmaf(a, Bg[kk][tx * 4 + jx], ag[i][jx]);
          if (UP) au[i][jx] = fmaf(a, Bu[kk][tx * 4 + jx], au[i][jx]);
        }
      }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = ty * 2 + i;
    if (r >= nrows) continue;
#pragma unroll
    for (int jx = 0; jx < 4; ++jx) {
      const int col = nt * TN + tx * 4 + jx;
      if (col >= N) continue;
      float v = ag[i][jx];
      if (UP) v = v / (1.0f + expf(-v)) * au[i][jx];
      C[(int64_t)(row0 + r) * N + col] = v;
    }
  }
}

}  // namespace

hipError_t launch_gemm_up(const Problem& p, const void* X, const int32_t* perm,
                          const int32_t* table, const void* W_gate, const void* W_up, void* H,
                          hipStream_t s) {
  const int64_t mtiles = max_row_tiles(p, BM);
  if (p.bf16) {
    const int NT = (p.n + BN / 2 - 1) / (BN / 2);
    const size_t smem = (size_t)kStages * kStageBytes;
    hipError_t err = hipFuncSetAttribute((const void*)grouped_gemm_bf16<true>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(grouped_gemm_bf16<true>, dim3((unsigned)(mtiles * NT)), dim3(kThreads), smem,
                       s, (const uint16_t*)X, perm, table, (const uint16_t*)W_gate,
                       (const uint16_t*)W_up, (uint16_t*)H, p.T, p.d, p.n, NT);
  } else {
    const int NT = (p.n + 63) / 64;
    hipLaunchKernelGGL(grouped_gemm_f32<true>, dim3((unsigned)(mtiles * 4 * NT)), dim3(256), 0, s,
                       (const float*)X, perm, table, (const float*)W_gate, (const float*)W_up,
                       (float*)H, p.T, p.d, p.n, NT);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_down(const Problem& p, const void* H, const int32_t* table,
                            const void* W_down, void* O, hipStream_t s) {
  const int64_t mtiles = max_row_tiles(p, BM);
  if (p.bf16) {
    const int NT = (p.d + BN - 1) / BN;
    const size_t smem = (size_t)kStages * kStageBytes;
    hipError_t err = hipFuncSetAttribute((const void*)grouped_gemm_bf16<false>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(grouped_gemm_bf16<false>, dim3((unsigned)(mtiles * NT)), dim3(kThreads),
                       smem, s, (const uint16_t*)H, nullptr, table, (const uint16_t*)W_down,
                       nullptr, (uint16_t*)O, p.T, p.n, p.d, NT);
  } else {
    const int NT = (p.d + 63) / 64;
    hipLaunchKernelGGL(grouped_gemm_f32<false>, dim3((unsigned)(mtiles * 4 * NT)), dim3(256), 0, s,
                       (const float*)H, nullptr, table, (const float*)W_down, nullptr, (float*)O,
                       p.T, p.n, p.d, NT);
  }
  return hipGetLastError();
}

}  // namespace moe
