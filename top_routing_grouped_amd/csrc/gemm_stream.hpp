// Weight-streaming body of the grouped GEMMs (steps 6-7 of the layer) for
// experts with few rows: one workgroup owns one expert and one block of COLS
// weight columns and streams that block over the whole k range once per pass
// of up to ROWS rows.  The SonicMoE article's arithmetic (§3 steps 3-5: the
// gathered up-projection with SwiGLU in the epilogue, §6.2-6.3, and the
// down-projection); with a handful of rows per expert almost every byte
// moved is weight, so the work is bound by reading the expert's weights.
//
// Two users: the stand-alone weight-streaming kernels (4 waves, decode-sized
// batches) and the 256x256-tiled kernels, whose launch appends one such
// workgroup (8 waves) per expert and column block for the experts with at
// most a few dozen rows (a skewed router leaves many of those next to a few
// full ones).
//
// * Up: COLS/2 W_gate columns + the same COLS/2 W_up columns, so SwiGLU is
//   register-local; down: COLS W_down columns.  Experts with no rows, or with
//   more than max_rows, return at once.
// * A pass streams the column block over k through kNST LDS stages (64 k
//   each) filled with global_load_lds_dwordx4 (weights with the non-temporal
//   hint: each is read once per pass) and counted with explicit vmcnt waits,
//   kNST-1 stages in flight.  Row blocks past the pass's last row skip their
//   MFMAs.
// * 16x16x32 bf16 MFMA.  Token rows (gathered through perm_token for up) sit
//   in LDS with the 128-byte-row XOR swizzle and are read with ds_read_b128;
//   weight rows keep the natural [k][n] order (XOR-swizzled) and are read
//   with ds_read_b64_tr_b16.  Both reads are bank-conflict free.
#pragma once
#include "moe_internal.hpp"

namespace moe {
namespace wstream {

using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using i16x4 = short __attribute__((ext_vector_type(4)));
using f32x4 = float __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;     // k per stage
constexpr int kNST = 4;     // LDS stages (3 to 8 measured alike)

// ROWS rows per pass (ROWS/16 MFMA row blocks), COLS weight columns per
// workgroup, NW waves; CB = 16-column MFMA blocks per wave.
template <int ROWS, int COLS, int NW>
struct Geo {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kRB = ROWS / 16;
  static constexpr int CB = COLS / (16 * NW);
  static constexpr int CPR = COLS / 8;              // 16-byte chunks per weight tile row
  static constexpr int kRPC = 64 / CPR;             // weight rows per copy instruction
  static constexpr int kA = ROWS * kBK * 2;
  static constexpr int kB = kBK * COLS * 2;
  static constexpr int kStage = kA + kB;
  static constexpr int kLds = kNST * kStage;
  static constexpr int kAI = kA / 1024 / NW;        // copy instructions per wave per stage
  static constexpr int kBI = kB / 1024 / NW;
  static constexpr int kInstr = kAI + kBI;
  static_assert(kAI * 1024 * NW == kA && kBI * 1024 * NW == kB, "copy split");
  static_assert(CB * 16 * NW == COLS && CB % 2 == 0, "column blocks");
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

// One workgroup of Geo<ROWS, COLS, NW>::kThreads threads: expert e, column
// block bx (up: output columns bx*COLS/2 ..; down: bx*COLS ..).  smem holds
// Geo::kLds bytes.  Every thread of the workgroup must call it.
template <bool UP, int ROWS, int COLS, int NW>
__device__ __forceinline__ void stream_block(
    const uint16_t* __restrict__ A,        // up: X [T][Kd]; down: H [rows][Kd]
    const int32_t* __restrict__ perm,      // up: expert-major slot -> token
    const int32_t* __restrict__ offsets,   // [E+1] expert row ranges
    const uint16_t* __restrict__ B0,       // up: W_gate; down: W_down ([E][Kd][N])
    const uint16_t* __restrict__ B1,       // up: W_up
    uint16_t* __restrict__ C,              // up: H [rows][N]; down: O [rows][N]
    int64_t T, int Kd, int N, int64_t rows_max, int max_rows, int e, int bx,
    unsigned char* smem) {
  using G = Geo<ROWS, COLS, NW>;
  constexpr int kRows = ROWS, kRB = G::kRB, kA = G::kA, kStage = G::kStage, kAI = G::kAI;
  constexpr int kBI = G::kBI, kInstr = G::kInstr, CB = G::CB, CPR = G::CPR;
  int off = offsets[e], end = offsets[e + 1];
  if (off < 0) off = 0;
  if ((int64_t)end > rows_max) end = (int)rows_max;
  const int m = end - off;
  if (m <= 0 || m > max_rows) return;
  const int ncol0 = bx * (UP ? COLS / 2 : COLS);

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

}  // namespace wstream
}  // namespace moe
