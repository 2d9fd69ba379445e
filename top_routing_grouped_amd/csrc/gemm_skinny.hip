// Steps 6-7 of the layer for batches with few rows per expert (decode-sized
// batches): the grouped GEMMs become weight streams.
//
// Same arithmetic as the tiled kernels in gemm.hip (the SonicMoE article's
// gathered up-projection with a SwiGLU epilogue, §3, §6.2, §6.3, and the
// down-projection), but with a handful of rows per expert almost every byte
// moved is weight: the work is bound by reading each active expert's
// weights once from HBM, so the kernel is organised around that stream.
//
// * One workgroup (4 waves) owns one expert and one block of 256 weight
//   columns (up: 128 W_gate columns + the same 128 W_up columns, so SwiGLU is
//   register-local; down: 256 W_down columns).  Experts without rows exit
//   at once; only active experts' weights are read.  Measured at the decode
//   size (T=64, d=4096, E=256, n=512) with cached copies: the weight stream
//   ran at 4.7-4.9 TB/s whether or not the MFMAs ran and for 3 to 8 stages,
//   i.e. bound by the memory system for these strided 512-byte row pieces
//   (128-column blocks: 4.5-4.75 TB/s).  The weight copies carry the
//   non-temporal hint (each weight is read once per launch): that lifted the
//   up projection from 374 to 305 us at this size.
// * The expert's rows are taken in passes of up to 64 (four 16-row MFMA
//   blocks; 32 when the batch averages at most 16 rows per expert); a pass
//   streams the column block over the whole k range through four LDS
//   stages (64 k each), filled with global_load_lds_dwordx4 and counted with
//   explicit vmcnt waits, three stages in flight.  Row blocks past the pass's
//   last row skip their MFMAs.
// * 16x16x32 bf16 MFMA.  Token rows (gathered through perm_token for up)
//   sit in LDS with the 128-byte-row XOR swizzle and are read with
//   ds_read_b128; weight rows keep the natural [k][n] order (256-byte rows,
//   XOR-swizzled) and are read with ds_read_b64_tr_b16.  Both reads are
//   bank-conflict free.
#include "moe_internal.hpp"

namespace moe {
namespace {

using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using i16x4 = short __attribute__((ext_vector_type(4)));
using f32x4 = float __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;             // 4 waves
constexpr int kBK = 64;                   // k per stage
constexpr int kNST = 4;                   // LDS stages (3 to 8 measured alike)
constexpr int kSkinnyCols = 256;          // weight columns per workgroup (128-column blocks were slower)

// ROWS rows per pass (ROWS/16 MFMA row blocks): 64, or 32 for batches with at
// most 16 rows per expert on average (a smaller token tile leaves more LDS to
// weights).  COLS weight columns per workgroup (up: COLS/2 of W_gate + the same
// of W_up), CB = COLS/64 16-column MFMA blocks per wave.
template <int ROWS, int COLS>
struct SkinnyGeo {
  static constexpr int kRB = ROWS / 16;
  static constexpr int CB = COLS / 64;
  static constexpr int CPR = COLS / 8;              // 16-byte chunks per weight tile row
  static constexpr int kRPC = 64 / CPR;             // weight rows per copy instruction
  static constexpr int kA = ROWS * kBK * 2;
  static constexpr int kB = kBK * COLS * 2;
  static constexpr int kStage = kA + kB;
  static constexpr int kLds = kNST * kStage;
  static constexpr int kAI = kA / 1024 / 4;
  static constexpr int kBI = kB / 1024 / 4;
  static constexpr int kInstr = kAI + kBI;
  static constexpr int kOcc = (kLds <= 80 * 1024) ? 2 : 1;   // workgroups per CU
  static_assert(kLds <= 160 * 1024, "LDS");
};

// XOR of the 16-byte chunk index of weight tile row r (16 or 32 chunks per
// row) that makes a 16x16x32 transpose read hit every bank equally.
__device__ __forceinline__ int wswz(int r) { return 2 * ((r & 3) + 4 * ((r >> 3) & 1)); }

// Wait until at most `pending` stages (INSTR copies each) of this wave are in
// flight (pending <= kNST - 2).
template <int INSTR>
__device__ __forceinline__ void wait_stages(int pending) {
  static_assert(kNST - 2 <= 6 && 6 * INSTR <= 63, "vmcnt range");
  if (pending >= 6) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(6 * INSTR) : "memory");
  else if (pending == 5) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(5 * INSTR) : "memory");
  else if (pending == 4) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * INSTR) : "memory");
  else if (pending == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * INSTR) : "memory");
  else if (pending == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * INSTR) : "memory");
  else if (pending == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(INSTR) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * dev::sigmoid(g) * u;
}

template <bool UP, int ROWS, int COLS>
__global__ __launch_bounds__(kThreads, (SkinnyGeo<ROWS, COLS>::kOcc)) void skinny_gemm_bf16(
    const uint16_t* __restrict__ A,        // up: X [T][Kd]; down: H [rows][Kd]
    const int32_t* __restrict__ perm,      // up: expert-major slot -> token
    const int32_t* __restrict__ offsets,   // [E+1] expert row ranges
    const uint16_t* __restrict__ B0,       // up: W_gate; down: W_down ([E][Kd][N])
    const uint16_t* __restrict__ B1,       // up: W_up
    uint16_t* __restrict__ C,              // up: H [rows][N]; down: O [rows][N]
    int64_t T, int Kd, int N, int64_t rows_max) {
  using G = SkinnyGeo<ROWS, COLS>;
  constexpr int kRows = ROWS, kRB = G::kRB, kA = G::kA, kStage = G::kStage, kAI = G::kAI;
  constexpr int kBI = G::kBI, kInstr = G::kInstr, CB = G::CB, CPR = G::CPR;
  const int e = blockIdx.y;
  int off = offsets[e], end = offsets[e + 1];
  if (off < 0) off = 0;
  if ((int64_t)end > rows_max) end = (int)rows_max;
  const int m = end - off;
  if (m <= 0) return;
  const int ncol0 = blockIdx.x * (UP ? COLS / 2 : COLS);

  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds_base = (uint32_t)(size_t)(__attribute__((address_space(3))) void*)smem;
  const int KT = Kd / kBK;

  // weight copies: instruction j = kBI*w + i fills tile rows kRPC*j +
  // lane/CPR, slot lane%CPR holding column chunk q = slot ^ wswz(row); up:
  // the first CPR/2 chunks are W_gate columns, the rest the same W_up
  // columns.  Columns past N (partial last block) read column 0: in bounds,
  // never stored.
  const uint16_t* bsrc[kBI];
#pragma unroll
  for (int i = 0; i < kBI; ++i) {
    const int r = (w * kBI + i) * G::kRPC + lane / CPR;
    const int q = (lane % CPR) ^ wswz(r);
    const uint16_t* base = (UP && q >= CPR / 2) ? B1 : B0;
    int col = UP ? ncol0 + 8 * (q % (CPR / 2)) : ncol0 + 8 * q;
    if (col >= N) col = 0;
    bsrc[i] = base + (int64_t)e * Kd * N + (int64_t)r * N + col;
  }
  // fragment offsets.  Tokens (A operand): lane -> row 16*rb + lane%16, k
  // chunk 4*ks + lane/16.  Weights (B operand, transpose read): lane group
  // g = lane/16, s = lane%16 -> tile row 32*ks + 8g + s/4 (+4 for the upper
  // half), column 16*block + 4*(s%4).  Wave w's CB column blocks: up -> CB/2
  // blocks of W_gate columns and the matching W_up blocks; down -> CB
  // consecutive blocks.
  int ao[kRB][2];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r = rb * 16 + (lane & 15);
      const int c = 4 * ks + (lane >> 4);
      ao[rb][ks] = r * 128 + ((c ^ ((r >> 1) & 7)) * 16);
    }
  const int g = lane >> 4, s4 = lane & 15;
  int bo[CB][2][2];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 32 * ks + 8 * g + (s4 >> 2) + 4 * h;
        const int colbase = UP ? ((cb < CB / 2) ? 16 * (w * (CB / 2) + cb)
                                                : COLS / 2 + 16 * (w * (CB / 2) + cb - CB / 2))
                               : 16 * (w * CB + cb);
        const int col = colbase + 4 * (s4 & 3);
        bo[cb][ks][h] = kA + r * (COLS * 2) + (((col >> 3) ^ wswz(r)) * 16) + (col & 7) * 2;
      }

  for (int p0 = 0; p0 < m; p0 += kRows) {
    const int pm = (m - p0 < kRows) ? m - p0 : kRows;   // rows in this pass
    const int nrb = (pm + 15) >> 4;
    // token copies: instruction j = kAI*w + i fills tile rows 8j + lane/8,
    // slot lane%8 holding k chunk slot ^ ((row >> 1) & 7).  Rows past the
    // pass repeat its last row.
    const uint16_t* asrc[kAI];
#pragma unroll
    for (int i = 0; i < kAI; ++i) {
      const int r = (w * kAI + i) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int rr = off + p0 + (r < pm ? r : pm - 1);
      int64_t row;
      if (UP) {
        int64_t tok = perm[rr];
        tok = tok < 0 ? 0 : (tok > T - 1 ? T - 1 : tok);
        row = tok;
      } else {
        row = rr;
      }
      asrc[i] = A + row * (int64_t)Kd + c * 8;
    }
    auto issue = [&](int kt) {
      const uint32_t base = lds_base + (uint32_t)((kt % kNST) * kStage);
#pragma unroll
      for (int i = 0; i < kAI; ++i) dev::lds_copy16(asrc[i] + kt * kBK, base + (w * kAI + i) * 1024);
#pragma unroll
      for (int i = 0; i < kBI; ++i)
        dev::lds_copy16_stream(bsrc[i] + (int64_t)kt * kBK * N, base + kA + (w * kBI + i) * 1024);
    };

    f32x4 acc[kRB][CB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int st = 0; st < kNST - 1; ++st)
      if (st < KT) issue(st);
    for (int kt = 0; kt < KT; ++kt) {
      // stage kt landed (own copies), published to all waves; the barrier
      // also tells every wave that stage kt-1 (refilled below) is free
      const int issued = (kt + kNST - 2 < KT - 1) ? kt + kNST - 2 : KT - 1;
      wait_stages<kInstr>(issued - kt);
      asm volatile("s_barrier" ::: "memory");
      if (kt + kNST - 1 < KT) issue(kt + kNST - 1);
      const unsigned char* S = smem + (kt % kNST) * kStage;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 b[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(S + bo[cb][ks][0]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(S + bo[cb][ks][1]));
          b[cb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          if (rb < nrb) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(S + ao[rb][ks]);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
              acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[cb], acc[rb][cb], 0, 0, 0);
          }
        }
      }
    }

    // epilogue: lane holds output column lane%16 of its column block, rows
    // 4*(lane/16)..+3 of each row block
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      if (rb < nrb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rb * 16 + 4 * (lane >> 4) + i;
          if (r < pm) {
            uint16_t* crow = C + (int64_t)(off + p0 + r) * N;
            if (UP) {
#pragma unroll
              for (int cb = 0; cb < CB / 2; ++cb) {
                const int col = ncol0 + 16 * (w * (CB / 2) + cb) + (lane & 15);
                if (col < N)
                  crow[col] = dev::f32_to_bf16_bits(silu_mul(acc[rb][cb][i], acc[rb][cb + CB / 2][i]));
              }
            } else {
#pragma unroll
              for (int cb = 0; cb < CB; ++cb) {
                const int col = ncol0 + 16 * (w * CB + cb) + (lane & 15);
                if (col < N) crow[col] = dev::f32_to_bf16_bits(acc[rb][cb][i]);
              }
            }
          }
        }
      }
    }
    __syncthreads();   // every wave is done with the stage buffers before the next pass
  }
}

template <bool UP, int ROWS>
hipError_t launch_rows(const Problem& p, const uint16_t* A, const int32_t* perm,
                       const int32_t* offsets, const uint16_t* B0, const uint16_t* B1,
                       uint16_t* C, hipStream_t s) {
  constexpr int kCols = kSkinnyCols;
  auto* kern = skinny_gemm_bf16<UP, ROWS, kCols>;
  constexpr int kLds = SkinnyGeo<ROWS, kCols>::kLds;
  const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (err != hipSuccess) return err;
  const int N = UP ? p.n : p.d;
  const int Kd = UP ? p.d : p.n;
  const int cols = UP ? kCols / 2 : kCols;
  const dim3 grid((unsigned)((N + cols - 1) / cols), (unsigned)p.E);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), (size_t)kLds, s, A, perm, offsets, B0, B1, C,
                     p.T, Kd, N, p.rows_max);
  return hipGetLastError();
}

template <bool UP>
hipError_t launch_skinny(const Problem& p, const uint16_t* A, const int32_t* perm,
                         const int32_t* offsets, const uint16_t* B0, const uint16_t* B1,
                         uint16_t* C, hipStream_t s) {
  if (p.T * (int64_t)p.K <= 16 * (int64_t)p.E)
    return launch_rows<UP, 32>(p, A, perm, offsets, B0, B1, C, s);
  return launch_rows<UP, 64>(p, A, perm, offsets, B0, B1, C, s);
}

}  // namespace

hipError_t launch_gemm_up_skinny(const Problem& p, const void* X, const int32_t* perm,
                                 const int32_t* offsets, const void* W_gate, const void* W_up,
                                 void* H, hipStream_t s) {
  return launch_skinny<true>(p, (const uint16_t*)X, perm, offsets, (const uint16_t*)W_gate,
                             (const uint16_t*)W_up, (uint16_t*)H, s);
}

hipError_t launch_gemm_down_skinny(const Problem& p, const void* H, const int32_t* offsets,
                                   const void* W_down, void* O, hipStream_t s) {
  return launch_skinny<false>(p, (const uint16_t*)H, nullptr, offsets, (const uint16_t*)W_down,
                              nullptr, (uint16_t*)O, s);
}

}  // namespace moe
