// Backward of the layer (training), following the SonicMoE article's
// reordering (§6.4): the forward keeps only X and the pre-SwiGLU activations
// (x W_gate | x W_up) per kept slot; the backward never forms the expert
// outputs O or Y.  Per slot s of expert e (token t, gate g):
//
//   dA'[s] = dY[t] W_down[e]^T                        (alpha GEMM, rows gathered)
//   dS[s]  = <dA'[s], A[s]>,  A = silu(Hg) * Hu        (its epilogue, A recomputed)
//   dHg    = g dA' * Hu * silu'(Hg),  dHu = g dA' * silu(Hg)   (§6.3: in the epilogue)
//   dXs[s] = dHg W_gate[e]^T + dHu W_up[e]^T           (alpha GEMM, k over 2n)
//   dW_down[e] = sum_s (g A[s])^T dY[t]                 (beta GEMM, rows gathered)
//   dW_gate[e] | dW_up[e] = sum_s X[t]^T (dHg | dHu)    (beta GEMM, rows gathered)
//   router: dg = dS, softmax-over-top-K Jacobian -> dl; dW_r = X^T dl;
//   dX[t] = sum over kept k of dXs[slot] + sum_k dl[t, id_k] W_r[:, id_k]
//
// Both GEMM kernels use the forward's tiling (256x256 tiles, 8 waves of
// 128x64, 32x32x16 bf16 MFMA, fp32 accumulators, two 64-deep LDS stages
// filled with global_load_lds_dwordx4 and counted vmcnt waits):
// * alpha: C[s][j] = sum_k A[row(s)][k] B[e][j][k] -- both operands have k
//   contiguous in memory, so both tiles are [256 rows][64 k] with the
//   forward's token-tile swizzle and both fragment reads are ds_read_b128.
// * beta:  C[g][i][j] = sum over the group's rows s of P[row(s)][i] Q[row(s)][j]
//   -- the reduction runs over rows, so both tiles are [64 rows][256 cols] in
//   natural order (the forward's weight-tile swizzle) and both fragment reads
//   are ds_read_b64_tr_b16.  Rows past a group's end copy zeros.
#include "moe_internal.hpp"

namespace moe {
namespace {

using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using i16x4 = short __attribute__((ext_vector_type(4)));
using f32x16 = float __attribute__((ext_vector_type(16)));
using f32x4 = float __attribute__((ext_vector_type(4)));
using u32x2 = uint32_t __attribute__((ext_vector_type(2)));
using u32x4 = uint32_t __attribute__((ext_vector_type(4)));

constexpr int kWGN = 4, kWTB = 4, kWCB = 2;   // 2 x 4 waves, each 128 rows x 64 columns
constexpr int kThreads = 512;
constexpr int kTile = 256;                   // rows and columns per tile
constexpr int kBK = 64;                      // k per stage
constexpr int kHalf = 32768;                 // bytes of one operand tile per stage
constexpr int kStage = 2 * kHalf;
constexpr int kLds = 2 * kStage;             // two stages: 128 KB
constexpr int kCopies = kHalf / 1024 / 8;    // copy instructions per wave per operand tile
constexpr int kInstr = 2 * kCopies;
constexpr int kWaitLds = 0xC07F;             // s_waitcnt lgkmcnt(0)

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void wait_copies(bool one_pending) {
  if (one_pending) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kInstr) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// [256 rows][64 k] tile with k contiguous: 128-byte rows, 16-byte chunk c of
// row r stored at slot c ^ ((r >> 1) & 7).
__device__ __forceinline__ int kmaj_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) * 16); }
// [64 k][256 columns] tile in natural order: 512-byte rows, chunk q of row k
// at slot q ^ (4 * (k & 3)); byte offset of 4 columns starting at `col`.
__device__ __forceinline__ int nat_off(int k, int col) {
  return k * 512 + ((((col >> 3) ^ (4 * (k & 3)))) * 16) + ((col >> 2) & 1) * 8;
}

template <int WTB, int WCB>
struct Frags {
  bf16x8 a[WTB];   // row operand (MFMA B), one per 32-row block
  bf16x8 b[WCB];   // column operand (MFMA A), one per 32-column block
};

// Tile decode shared with the forward: the tile table lists (expert, row
// range) per 256-row tile; ids are remapped so each XCD takes a contiguous
// range (same expert, same rows close together).
struct TileInfo {
  int e, row0, nrows, nt, L;
  bool valid;
};
__device__ __forceinline__ TileInfo decode_tile(const int32_t* table, int NT) {
  TileInfo ti{0, 0, 0, 0, 0, false};
  const int total = table[0] * NT;
  const int bid = blockIdx.x;
  if (bid >= total) return ti;
  const int q8 = total >> 3, r8 = total & 7;
  const int xcd = bid & 7, j = bid >> 3;
  const int L = xcd * q8 + (xcd < r8 ? xcd : r8) + j;
  const int mt = L / NT;
  const int32_t* ent = table + 4 * (mt + 1);
  ti.e = tile_expert((uint32_t)ent[0]);
  ti.row0 = ent[1];
  ti.nrows = ent[2] - ent[1];
  ti.nt = L - mt * NT;
  ti.L = L;
  ti.valid = true;
  return ti;
}

// ---------------------------------------------------------------- alpha GEMM
enum { kEpiStore = 0, kEpiDSwiGLU = 1 };

// Column order of the dSwiGLU alpha GEMM's 32-column MFMA blocks (the
// store-epilogue instance keeps the natural order, col(i) = i): lane l feeds
// the MFMA the column-operand row sig(l % 32), sig swapping bits 2 and 3.  The
// accumulator a lane holds for block column i (i = 8*(v/4) + 4*(lane/32) +
// v%4) is then output column sig(i), so each lane ends with two runs of 8
// adjacent columns (16p + 8*(lane/32) + 0..7, p = 0, 1) instead of four
// runs of 4, and the dSwiGLU epilogue reads the matching pre-activations
// with 16-byte loads (half as many requests as 8-byte ones).
__device__ __forceinline__ int sig(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
template <int EPI>
__device__ __forceinline__ int block_col(int i) { return EPI == kEpiDSwiGLU ? sig(i) : i; }

// C[s][j] = sum_k A[row(s)][k] * B[e][j][k] for the slots s of each tile.
//   A: [.][Kd] (rows gathered through perm when GATHER, else the slot rows)
//   B: B0[e][N][Kb] for k < Kb and B1[e][N][Kb] for k >= Kb (Kd = Kb or 2 Kb)
// kEpiStore:   C[s][j] (bf16, [rows][N]).
// kEpiDSwiGLU: with Hpre[s] = (Hg | Hu) and gs[s] the slot gate: writes
//   dH[s] = (g dA' Hu silu'(Hg) | g dA' silu(Hg)), gA[s] = g silu(Hg) Hu and
//   the tile's share of dS[s] = <dA', A> to dS_part[s][nt].
template <int EPI, bool GATHER>
__global__ __launch_bounds__(kThreads, 1) void alpha_gemm(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ table, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, int64_t T, int Kd, int Kb, int N, int NT,
    uint16_t* __restrict__ C, const uint16_t* __restrict__ Hpre, const float* __restrict__ gs,
    uint16_t* __restrict__ dH, uint16_t* __restrict__ gA, float* __restrict__ dS_part) {
  constexpr int KS = kBK / 16;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / kWGN, wn = w - (w / kWGN) * kWGN;
  const uint32_t lds_base = (uint32_t)(size_t)(lds_ptr_t)smem;

  const TileInfo ti = decode_tile(table, NT);
  if (!ti.valid) return;
  const int e = ti.e, row0 = ti.row0, nrows = ti.nrows;
  const int ncol0 = ti.nt * kTile;
  int ntb = (nrows - wm * (kWTB * 32) + 31) / 32;
  ntb = ntb < 0 ? 0 : (ntb > kWTB ? kWTB : ntb);

  // copies: instruction j = kCopies*w + i fills tile rows 8j + lane/8 of each
  // operand, slot lane%8 holding k chunk slot ^ ((row >> 1) & 7)
  const uint16_t* asrc[kCopies];
  const uint16_t* bsrc0[kCopies];
  const uint16_t* bsrc1[kCopies];
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int r = (w * kCopies + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int rr = r < nrows ? r : nrows - 1;
    int64_t row;
    if (GATHER) {
      int64_t tok = perm[row0 + rr];
      row = tok < 0 ? 0 : (tok > T - 1 ? T - 1 : tok);
    } else {
      row = row0 + rr;
    }
    asrc[i] = A + row * (int64_t)Kd + c * 8;
    int col = ncol0 + r;
    if (col >= N) col = 0;                   // in-bounds filler; never stored
    const int64_t boff = ((int64_t)e * N + col) * Kb + c * 8;
    bsrc0[i] = B0 + boff;
    bsrc1[i] = (B1 ? B1 : B0) + boff;
  }
  // Tile L starts its k loop at k-step L mod KT and wraps, so the tiles an
  // XCD runs together work on the same k slice and share it in L2 (as in
  // the forward's down projection): dXs 902 -> 837 us, dA' 664 -> 656 us at
  // the Qwen3 shape.  Each tile's summation order depends only on L.
  const int KTall = Kd / kBK;
  const int arot = ti.L % KTall;
  auto issue_stage = [&](int kt) {
    const uint32_t As = lds_base + (uint32_t)((kt & 1) * kStage);
    const uint32_t Bs = As + kHalf;
    int kr = kt + arot;
    if (kr >= KTall) kr -= KTall;
    const int kk = kr * kBK;
#pragma unroll
    for (int i = 0; i < kCopies; ++i) dev::lds_copy16(asrc[i] + kk, As + (w * kCopies + i) * 1024);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const uint16_t* src = (kk < Kb) ? bsrc0[i] + kk : bsrc1[i] + (kk - Kb);
      dev::lds_copy16(src, Bs + (w * kCopies + i) * 1024);
    }
  };

  int a_off[kWTB][KS], b_off[kWCB][KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c = ks * 2 + (lane >> 5);
#pragma unroll
    for (int tb = 0; tb < kWTB; ++tb) a_off[tb][ks] = kmaj_off(wm * 128 + tb * 32 + (lane & 31), c);
#pragma unroll
    for (int cb = 0; cb < kWCB; ++cb) b_off[cb][ks] = kHalf + kmaj_off(wn * 64 + cb * 32 + block_col<EPI>(lane & 31), c);
  }
  auto read_frags = [&](Frags<kWTB, kWCB>& f, int kt, int ks) {
    const unsigned char* S = smem + (kt & 1) * kStage;
#pragma unroll
    for (int tb = 0; tb < kWTB; ++tb) f.a[tb] = *reinterpret_cast<const bf16x8*>(S + a_off[tb][ks]);
#pragma unroll
    for (int cb = 0; cb < kWCB; ++cb) f.b[cb] = *reinterpret_cast<const bf16x8*>(S + b_off[cb][ks]);
  };
  f32x16 acc[kWCB][kWTB];
#pragma unroll
  for (int cb = 0; cb < kWCB; ++cb)
#pragma unroll
    for (int tb = 0; tb < kWTB; ++tb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[cb][tb][v] = 0.f;
  auto mma = [&](const Frags<kWTB, kWCB>& f) {
#pragma unroll
    for (int tb = 0; tb < kWTB; ++tb)
      if (tb < ntb) {
#pragma unroll
        for (int cb = 0; cb < kWCB; ++cb)
          acc[cb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[cb], f.a[tb], acc[cb][tb], 0, 0, 0);
      }
  };

  // main loop (the forward's schedule): stage kt+1 loads while stage kt is
  // multiplied; fragments are read one 16-deep sub-step ahead.
  const int KT = Kd / kBK;
  issue_stage(0);
  wait_copies(false);
  asm volatile("s_barrier" ::: "memory");
  Frags<kWTB, kWCB> cur, nxt;
  read_frags(cur, 0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) issue_stage(kt + 1);
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      __builtin_amdgcn_s_waitcnt(kWaitLds);
      __builtin_amdgcn_sched_barrier(0);
      read_frags(nxt, kt, ks + 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(cur);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitLds);
      if (ks + 2 < KS) {
        read_frags(cur, kt, ks + 2);
      } else if (kt + 1 < KT) {
        wait_copies(false);
        asm volatile("s_barrier" ::: "memory");
        read_frags(cur, kt + 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mma(nxt);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue.  A lane holds, for row lane%32 of block tb, columns
  // block_col(8*(v/4) + 4*(lane/32)) + v%4 of block cb.  Output tiles go through the
  // stage buffers (row-major bf16, 16-byte chunks XOR-swizzled by row) and
  // leave as whole rows.
  constexpr int kRowBytes = kTile * 2, kChunks = kRowBytes / 16;
  // The lane index is passed through an empty asm per pass so that the
  // compiler recomputes these addresses in each pass instead of keeping one
  // copy of every address live across all passes (that alone spilled).
  auto fresh = [](int v) {
    asm volatile("" : "+v"(v));
    return v;
  };
  auto stage_value = [&](int ln, int tb, int cb, int v4, const float* v) {
    const int rloc = wm * 128 + tb * 32 + (ln & 31);
    const int col = wn * 64 + cb * 32 + block_col<EPI>(8 * v4 + 4 * (ln >> 5));
    const u32x2 pk = {dev::pack_bf16x2(v[0], v[1]), dev::pack_bf16x2(v[2], v[3])};
    const int chunk = (col >> 3) ^ (rloc & (kChunks - 1));
    *reinterpret_cast<u32x2*>(smem + rloc * kRowBytes + chunk * 16 + ((col >> 2) & 1) * 8) = pk;
  };
  // thread t stores chunk t%32 of rows t/32 + 16 i
  auto store_tile = [&](uint16_t* out, int64_t pitch, int col_off) {
    __syncthreads();
    const int t0 = fresh(tid);
    const int r0 = t0 >> 5, c = t0 & (kChunks - 1);
    const int col = ncol0 + c * 8;
    uint16_t* dst = out + (int64_t)(row0 + r0) * pitch + col_off + col;
    const unsigned char* src = smem + r0 * kRowBytes;
    constexpr int kIters = kTile * kChunks / kThreads;
    constexpr int kStep = kThreads / kChunks;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int rloc = r0 + kStep * i;
      if (rloc < nrows && col < N) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(
            src + kStep * i * kRowBytes + ((c ^ (rloc & (kChunks - 1))) * 16));
        *reinterpret_cast<bf16x8*>(dst + (int64_t)kStep * i * pitch) = v;
      }
    }
    __syncthreads();
  };
  asm volatile("s_barrier" ::: "memory");    // every wave is done reading the last stage

  if constexpr (EPI == kEpiStore) {
    const int ln = fresh(lane);
#pragma unroll
    for (int tb = 0; tb < kWTB; ++tb)
#pragma unroll
      for (int cb = 0; cb < kWCB; ++cb)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[cb][tb][4 * v4 + r];
          stage_value(ln, tb, cb, v4, v);
        }
    store_tile(C, N, 0);
  } else {

  // kEpiDSwiGLU: three passes (dHg, dHu, gA) through the staging tile; the
  // pre-activations are re-read per pass (L2-resident after the first).
  float gsl[kWTB];
#pragma unroll
  for (int tb = 0; tb < kWTB; ++tb) {
    const int rloc = wm * 128 + tb * 32 + (lane & 31);
    gsl[tb] = (rloc < nrows) ? gs[row0 + rloc] : 0.f;
  }
  // Pre-activations of the lane's values: row rloc, columns
  // ncol0 + wn*64 + cb*32 + 16*p + 8*(lane/32) + 0..7 (the values of
  // v4 = 2p and 2p+1) -- one row pointer per 32-row block and constant
  // offsets, 16 bytes per load.  N is a multiple of 64, so a wave's
  // 64 columns are all inside or all outside the layer (a uniform branch);
  // rows past the tile's end read its first row and are zeroed.
  const bool colok = ncol0 + wn * 64 < N;
  // pass 1: dHg is staged and stored; dHu and g*A are rounded to bf16 and
  // kept, packed in pairs, in the accumulator registers they replace (dA' is
  // not needed again), so the pre-activations are read once.
  float dsum[kWTB];
  const int ln1 = fresh(lane);
#pragma unroll
  for (int tb = 0; tb < kWTB; ++tb) {
    dsum[tb] = 0.f;
    const int rloc = wm * 128 + tb * 32 + (lane & 31);
    const bool rok = rloc < nrows;
    const uint16_t* hrow =
        Hpre + (int64_t)(row0 + (rok ? rloc : 0)) * (2 * N) + ncol0 + wn * 64 + 8 * (lane >> 5);
    u32x2 ga[kWCB][4], ua[kWCB][4];
#pragma unroll
    for (int cb = 0; cb < kWCB; ++cb)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if (colok) {
          const u32x4 g4 = *reinterpret_cast<const u32x4*>(hrow + cb * 32 + 16 * p);
          const u32x4 u4 = *reinterpret_cast<const u32x4*>(hrow + N + cb * 32 + 16 * p);
          ga[cb][2 * p] = u32x2{g4[0], g4[1]};
          ga[cb][2 * p + 1] = u32x2{g4[2], g4[3]};
          ua[cb][2 * p] = u32x2{u4[0], u4[1]};
          ua[cb][2 * p + 1] = u32x2{u4[2], u4[3]};
        } else {
          ga[cb][2 * p] = ga[cb][2 * p + 1] = u32x2{0u, 0u};
          ua[cb][2 * p] = ua[cb][2 * p + 1] = u32x2{0u, 0u};
        }
      }
#pragma unroll
    for (int cb = 0; cb < kWCB; ++cb)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        float out[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t gw = ga[cb][v4][r >> 1], uw = ua[cb][v4][r >> 1];
          const float hg = rok ? dev::bf16_bits_to_f32((r & 1) ? (gw >> 16) : (gw & 0xFFFFu)) : 0.f;
          const float hu = rok ? dev::bf16_bits_to_f32((r & 1) ? (uw >> 16) : (uw & 0xFFFFu)) : 0.f;
          const float dap = acc[cb][tb][4 * v4 + r];
          const float sg = dev::sigmoid(hg);
          const float sl = hg * sg;                          // silu(Hg)
          const float da = gsl[tb] * dap;                    // dA = g dA'
          dsum[tb] = fmaf(dap, sl * hu, dsum[tb]);
          out[r] = da * hu * sg * (1.0f + hg * (1.0f - sg));
          uint32_t kept = dev::pack_bf16x2(da * sl, gsl[tb] * sl * hu);
          asm volatile("" : "+v"(kept));            // computed here, not at its use
          acc[cb][tb][4 * v4 + r] = __uint_as_float(kept);
        }
        stage_value(ln1, tb, cb, v4, out);
      }
    // finish the block's dS share here: left to the compiler, the sum (like
    // the kept values above) was sunk to its use after the store, keeping
    // every loaded value live
    asm volatile("" : "+v"(dsum[tb]));
    __builtin_amdgcn_sched_barrier(0);
  }
  store_tile(dH, 2 * (int64_t)N, 0);
  // dS share: lanes l and l+32 hold the same row; then the 4 column waves
  float* red = reinterpret_cast<float*>(smem);          // [4 waves][256 rows]
#pragma unroll
  for (int tb = 0; tb < kWTB; ++tb) {
    const float other = __shfl_xor(dsum[tb], 32);
    if (lane < 32) red[wn * kTile + wm * 128 + tb * 32 + lane] = dsum[tb] + other;
  }
  __syncthreads();
  if (tid < kTile && tid < nrows) {
    const float v = ((red[tid] + red[kTile + tid]) + red[2 * kTile + tid]) + red[3 * kTile + tid];
    dS_part[(int64_t)(row0 + tid) * NT + ti.nt] = v;
  }
  __syncthreads();
  // passes 2 and 3: the kept bf16 halves (dHu, then g*A)
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int ln = fresh(lane);
#pragma unroll
    for (int tb = 0; tb < kWTB; ++tb)
#pragma unroll
      for (int cb = 0; cb < kWCB; ++cb)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          float out[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t pk = __float_as_uint(acc[cb][tb][4 * v4 + r]);
            out[r] = dev::bf16_bits_to_f32(half ? (pk >> 16) : (pk & 0xFFFFu));
          }
          stage_value(ln, tb, cb, v4, out);
        }
    if (half == 0) store_tile(dH, 2 * (int64_t)N, N);
    else store_tile(gA, N, 0);
  }
  }
}

// ---------------------------------------------------------------- beta GEMM
// C[g][i][j] = sum over rows s of group g (k split z of ksplit) of
// P[prow(s)][i] * Q[qrow(s)][j], fp32.  Groups are the experts' slot ranges
// (offsets), or one group of `rows_total` rows when offsets is NULL.  prow /
// qrow go through perm when PG / QG.  Columns j < Jsplit go to C0[g][i][j]
// (pitch Jsplit), the rest to C1[g][i][j - Jsplit] (pitch Jq - Jsplit); with
// ksplit > 1, C0 is a partial buffer and split z writes at z * zstride.
//
// The reduction runs over an expert's rows, a few hundred to a few thousand,
// so a tile has few k-steps.  NST stages of BK rows: on the Qwen3-shaped
// layer two 64-row stages ran fastest (dW_gate|dW_up 1.31 ms); four or five
// 32-row stages (more bytes in flight, twice the barriers) were 5-11% slower.
template <int NST, int BK>
struct BetaGeo {
  static constexpr int kOpBytes = BK * kTile * 2;        // one operand tile of a stage
  static constexpr int kStage = 2 * kOpBytes;
  static constexpr int kLds = NST * kStage;
  static constexpr int kCopies = kOpBytes / 1024 / 8;    // copy instructions per wave per operand
  static constexpr int kInstr = 2 * kCopies;
  static constexpr int KS = BK / 16;
  static_assert(kCopies * 1024 * 8 == kOpBytes, "copy split");
  static_assert(kLds <= 160 * 1024, "LDS per workgroup");
  static_assert(NST >= 2 && NST <= 5, "stage count");
};

// Wait until at most `pending` stages (INSTR copy instructions each) of this
// wave are in flight.
template <int INSTR>
__device__ __forceinline__ void wait_stages(int pending) {
  if (pending >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * INSTR) : "memory");
  else if (pending == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * INSTR) : "memory");
  else if (pending == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(INSTR) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <bool PG, bool QG, int NST, int BK>
__global__ __launch_bounds__(kThreads, 1) void beta_gemm(
    const uint16_t* __restrict__ P, const uint16_t* __restrict__ Q,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets, int64_t rows_total,
    int64_t T, int Ip, int Jq, int IT, int JT, int ksplit, const uint16_t* __restrict__ zero,
    float* __restrict__ C0, float* __restrict__ C1, int Jsplit, int64_t zstride) {
  using G = BetaGeo<NST, BK>;
  constexpr int KS = G::KS, kCp = G::kCopies, kInstrS = G::kInstr;
  constexpr int kOp = G::kOpBytes, kSt = G::kStage;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / kWGN, wn = w - (w / kWGN) * kWGN;
  const uint32_t lds_base = (uint32_t)(size_t)(lds_ptr_t)smem;

  // tile decode: logical id L = group * IT * JT + it * JT + jt; y = k split.
  // Workgroups go to the 8 XCDs round robin; the remap gives each XCD a
  // contiguous range of L, so the tiles running together on an XCD belong to
  // one or two groups, advance over the same rows together and share the
  // row slabs in its L2 (round robin spread every group over all 8 XCDs).
  const int total = gridDim.x;
  const int q8 = total >> 3, r8 = total & 7;
  const int xcd = blockIdx.x & 7;
  const int L = xcd * q8 + (xcd < r8 ? xcd : r8) + (blockIdx.x >> 3);
  const int per_group = IT * JT;
  const int g = L / per_group;
  const int rem = L - g * per_group;
  const int it = rem / JT, jt = rem - (rem / JT) * JT;
  const int z = blockIdx.y;
  int64_t s0, s1;
  if (offsets) {
    s0 = offsets[g];
    s1 = offsets[g + 1];
  } else {
    s0 = 0;
    s1 = rows_total;
  }
  const int64_t m = s1 - s0;
  const int64_t lo = s0 + (m * z) / ksplit, hi = s0 + (m * (z + 1)) / ksplit;
  const int i0 = it * kTile, j0 = jt * kTile;
  const int64_t zoff = (int64_t)z * zstride;
  if (hi <= lo) {
    // an empty group (or split) still owns its output block: write zeros
    for (int idx = tid; idx < kTile * kTile / 4; idx += kThreads) {
      const int i = idx / (kTile / 4), j = (idx - (idx / (kTile / 4)) * (kTile / 4)) * 4;
      if (i0 + i >= Ip || j0 + j >= Jq) continue;
      const int jj = j0 + j;
      float* dst = (jj < Jsplit) ? C0 + zoff + ((int64_t)g * Ip + i0 + i) * Jsplit + jj
                                 : C1 + ((int64_t)g * Ip + i0 + i) * (Jq - Jsplit) + (jj - Jsplit);
      *reinterpret_cast<f32x4*>(dst) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }

  // copies: instruction c = kCp*w + i fills tile rows 2c + lane/32 of each
  // operand (so wave w owns rows 2*kCp*w .. 2*kCp*w + 2*kCp - 1), slot
  // lane%32 holding column chunk slot ^ (4 * (row & 3)).  Columns past the
  // operand's width read column 0 (in bounds; they only feed output columns
  // that are never stored); rows past the range copy zeros.
  int pcol[kCp], qcol[kCp];
#pragma unroll
  for (int i = 0; i < kCp; ++i) {
    const int k = 2 * (w * kCp + i) + (lane >> 5);
    const int q = (lane & 31) ^ (4 * (k & 3));
    const int pc = i0 + q * 8, qc = j0 + q * 8;
    pcol[i] = pc < Ip ? pc : 0;
    qcol[i] = qc < Jq ? qc : 0;
  }
  // Source rows of the next stage to issue (-1: past the range).  The row
  // numbers are wave-uniform per half wave, so gathered ones come from perm
  // with scalar loads: they do not count against the vector-memory counter
  // that the stage waits use, and are fetched one stage ahead of their use.
  int prow[kCp], qrow[kCp];
  int rot = 0, KTr = 1;
  auto fetch_rows = [&](int kt) {
    int kk = kt + rot;
    if (kk >= KTr) kk -= KTr;
    const int64_t sb = lo + (int64_t)kk * BK + 2 * kCp * w;
#pragma unroll
    for (int i = 0; i < kCp; ++i) {
      int r[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t sr = sb + 2 * i + h;
        int v = -1;
        if (sr < hi) {
          if (PG || QG) {
            const int64_t t = perm[sr];
            v = (int)(t < 0 ? 0 : (t > T - 1 ? T - 1 : t));
          } else {
            v = (int)sr;
          }
        }
        r[h] = v;
      }
      const int rg = (lane >> 5) ? r[1] : r[0];                  // gathered (or own) row
      const int rs = rg < 0 ? -1 : (int)(sb + 2 * i + (lane >> 5));  // slot row
      prow[i] = PG ? rg : rs;
      qrow[i] = QG ? rg : rs;
    }
  };
  auto issue_stage = [&](int kt) {
    const uint32_t Ps = lds_base + (uint32_t)((kt % NST) * kSt);
    const uint32_t Qs = Ps + kOp;
#pragma unroll
    for (int i = 0; i < kCp; ++i) {
      const uint16_t* ps = prow[i] >= 0 ? P + (int64_t)prow[i] * Ip + pcol[i] : zero;
      const uint16_t* qs = qrow[i] >= 0 ? Q + (int64_t)qrow[i] * Jq + qcol[i] : zero;
      dev::lds_copy16(ps, Ps + (w * kCp + i) * 1024);
      dev::lds_copy16(qs, Qs + (w * kCp + i) * 1024);
    }
  };

  // fragments by transpose read (the forward's weight-fragment geometry):
  // group gq = lane/16, lane s in the group -> tile row 16*ks + 8*(gq/2) + s/4
  // (+4 for the upper half), column 16*(gq%2) + 4*(s%4) of the 32-column block
  const int gq = lane >> 4, s16 = lane & 15;
  const int tr_row = 8 * (gq >> 1) + (s16 >> 2);
  int p_off[kWTB][2], q_off[kWCB][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = tr_row + 4 * h;
#pragma unroll
    for (int tb = 0; tb < kWTB; ++tb)
      p_off[tb][h] = nat_off(k, wm * 128 + tb * 32 + 16 * (gq & 1) + 4 * (s16 & 3));
#pragma unroll
    for (int cb = 0; cb < kWCB; ++cb)
      q_off[cb][h] = kOp + nat_off(k, wn * 64 + cb * 32 + 16 * (gq & 1) + 4 * (s16 & 3));
  }
  auto tr8 = [&](const unsigned char* S, int o0, int o1) {
    const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(S + o0));
    const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(S + o1));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto read_frags = [&](Frags<kWTB, kWCB>& f, int kt, int ks) {
    const unsigned char* S = smem + (kt % NST) * kSt + ks * 16 * 512;
#pragma unroll
    for (int tb = 0; tb < kWTB; ++tb) f.a[tb] = tr8(S, p_off[tb][0], p_off[tb][1]);
#pragma unroll
    for (int cb = 0; cb < kWCB; ++cb) f.b[cb] = tr8(S, q_off[cb][0], q_off[cb][1]);
  };
  f32x16 acc[kWCB][kWTB];
#pragma unroll
  for (int cb = 0; cb < kWCB; ++cb)
#pragma unroll
    for (int tb = 0; tb < kWTB; ++tb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[cb][tb][v] = 0.f;
  auto mma = [&](const Frags<kWTB, kWCB>& f) {
#pragma unroll
    for (int tb = 0; tb < kWTB; ++tb)
#pragma unroll
      for (int cb = 0; cb < kWCB; ++cb)
        acc[cb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[cb], f.a[tb], acc[cb][tb], 0, 0, 0);
  };

  // main loop: stages kt+1 .. kt+NST-1 in flight while stage kt is multiplied
  const int KT = (int)((hi - lo + BK - 1) / BK);
  // the k (row) loop starts at row block L mod KT and wraps, as in the
  // alpha GEMMs: dW_down 623 -> 593 us, dW_gate|dW_up unchanged
  KTr = KT;
  rot = L % KT;
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < KT) {
      fetch_rows(st);
      issue_stage(st);
    }
  if (NST - 1 < KT) fetch_rows(NST - 1);
  wait_stages<kInstrS>((KT - 1 < NST - 2) ? KT - 1 : NST - 2);
  asm volatile("s_barrier" ::: "memory");
  Frags<kWTB, kWCB> cur, nxt;
  read_frags(cur, 0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + NST - 1 < KT) issue_stage(kt + NST - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      __builtin_amdgcn_s_waitcnt(kWaitLds);
      __builtin_amdgcn_sched_barrier(0);
      read_frags(nxt, kt, ks + 1);
      // the next stage's rows: every LDS wait also waits for scalar loads,
      // so they are issued where the MFMAs below cover their latency
      if (ks == 0 && kt + NST < KT) fetch_rows(kt + NST);
      __builtin_amdgcn_sched_barrier(0);
      mma(cur);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitLds);
      if (ks + 2 < KS) {
        read_frags(cur, kt, ks + 2);
      } else if (kt + 1 < KT) {
        // stage kt+1 landed (own copies), then publish it to all waves; the
        // barrier also tells every wave that stage kt's buffer is free
        const int last = (kt + NST - 1 < KT) ? kt + NST - 1 : KT - 1;
        wait_stages<kInstrS>(last - (kt + 1));
        asm volatile("s_barrier" ::: "memory");
        read_frags(cur, kt + 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mma(nxt);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // output: the fp32 tile is staged through the (idle) stage buffers in two
  // halves of 128 rows (1 KB rows, 16-byte chunks XOR-swizzled by row) and
  // stored as whole rows with the non-temporal hint.  A lane holds row
  // lane%32 of block tb and 4 consecutive columns 8*(v/4) + 4*(lane/32) of
  // block cb; stored from the accumulators, every instruction wrote 16-byte
  // pieces of 32 rows.  Staged and non-temporal, the backward takes 3.49
  // instead of 3.66 ms at the Qwen3 shape (non-temporal pieces of rows were
  // slower than cached ones: 4.15 ms).
  constexpr int kCh = kTile / 4;             // 16-byte chunks per fp32 row
  static_assert(128 * kCh * 16 <= G::kLds, "half tile must fit the stage buffers");
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __syncthreads();                         // MFMA reads / previous half done
    if (wm == h) {
#pragma unroll
      for (int tb = 0; tb < kWTB; ++tb) {
        const int rl = tb * 32 + (lane & 31);
#pragma unroll
        for (int cb = 0; cb < kWCB; ++cb)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int c = (wn * 64 + cb * 32 + 8 * v4 + 4 * (lane >> 5)) >> 2;
            const f32x4 v = {acc[cb][tb][4 * v4], acc[cb][tb][4 * v4 + 1], acc[cb][tb][4 * v4 + 2],
                             acc[cb][tb][4 * v4 + 3]};
            *reinterpret_cast<f32x4*>(smem + rl * (kCh * 16) + ((c ^ (rl & (kCh - 1))) * 16)) = v;
          }
      }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 128 * kCh / kThreads; ++it) {
      const int idx = tid + kThreads * it;
      const int rl = idx / kCh, c = idx - (idx / kCh) * kCh;
      const int i = i0 + h * 128 + rl, j = j0 + 4 * c;
      if (i < Ip && j < Jq) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(smem + rl * (kCh * 16) + ((c ^ (rl & (kCh - 1))) * 16));
        float* dst = (j < Jsplit) ? C0 + zoff + ((int64_t)g * Ip + i) * Jsplit + j
                                  : C1 + ((int64_t)g * Ip + i) * (Jq - Jsplit) + (j - Jsplit);
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
      }
    }
  }
}

// ---------------------------------------------------------------- small kernels
// gs[inv[t,k]] = gates[t,k] for kept assignments; clears the zero rows that
// the weight-gradient GEMMs copy past a group's end.
__global__ __launch_bounds__(256) void slot_gate_kernel(const float* __restrict__ gates,
                                                        const int32_t* __restrict__ inv,
                                                        float* __restrict__ gs, int64_t TK,
                                                        uint32_t* __restrict__ zero) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.x == 0 && threadIdx.x < kZeroBytes / 4) zero[threadIdx.x] = 0u;
  if (i >= TK) return;
  const int s = inv[i];
  if (s >= 0) gs[s] = gates[i];
}

// W_rT[e][i] = W_r[i][e], so that the router's share of dX is a row gather.
__global__ __launch_bounds__(256) void transpose_router_kernel(const uint16_t* __restrict__ W_r,
                                                               uint16_t* __restrict__ W_rT, int d,
                                                               int E) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)d * E) return;
  const int e = (int)(i / d), k = (int)(i - (i / d) * d);
  W_rT[i] = W_r[(int64_t)k * E + e];
}

// Per token (one wave each):
//   dg[k]   = dS[slot(t,k)] = sum of its tile shares in tile order (0 if dropped)
//   dsel[k] = g_k (dg_k - sum_j g_j dg_j)       (softmax over the K selected)
//   dl[t]   = dsel scattered to the selected experts, zeros elsewhere (bf16, Epad wide)
//   dX[t]   = sum over kept k of dXs[slot(t,k)] + sum_k dsel[k] W_rT[id_k]   (fp32, k order)
constexpr int kTokWaves = 4;
constexpr int kMaxK = 256;
__global__ __launch_bounds__(64 * kTokWaves) void token_backward_kernel(
    const float* __restrict__ dS_part, int NT, const int32_t* __restrict__ ids,
    const float* __restrict__ gates, const int32_t* __restrict__ inv,
    const uint16_t* __restrict__ dXs, const uint16_t* __restrict__ W_rT,
    uint16_t* __restrict__ dl, uint16_t* __restrict__ dX, int64_t T, int d, int K, int Epad) {
  __shared__ float s_dsel[kTokWaves][kMaxK];
  __shared__ int s_id[kTokWaves][kMaxK];
  __shared__ int s_slot[kTokWaves][kMaxK];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kTokWaves + wv;
  const bool live = t < T;
  float part = 0.f;
  if (live) {
    for (int k = lane; k < K; k += 64) {
      const int s = inv[t * K + k];
      float dg = 0.f;
      if (s >= 0)
        for (int q = 0; q < NT; ++q) dg += dS_part[(int64_t)s * NT + q];
      s_dsel[wv][k] = dg;
      s_id[wv][k] = ids[t * K + k];
      s_slot[wv][k] = s;
      part = fmaf(gates[t * K + k], dg, part);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
  if (live)
    for (int k = lane; k < K; k += 64) s_dsel[wv][k] = gates[t * K + k] * (s_dsel[wv][k] - part);
  __syncthreads();
  if (!live) return;
  for (int e = lane; e < Epad; e += 64) {
    float v = 0.f;
    for (int k = 0; k < K; ++k) v = (s_id[wv][k] == e) ? s_dsel[wv][k] : v;
    dl[t * Epad + e] = dev::f32_to_bf16_bits(v);
  }
  constexpr int KG = 8;
  const int nchunk = d / 8;
  for (int c = lane; c < nchunk; c += 64) {
    float acc[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[v] = 0.f;
    for (int k0 = 0; k0 < K; k0 += KG) {
      // Entries that are dropped, or past K, load a kept row of the token
      // (one already being read) and are left out of the sum; a group with
      // no kept row loads nothing.  Sending them all to row 0 made that row
      // a hot spot in L2 for every token that lost its assignments.
      int sl[KG];
      bool ok[KG];
      int fb = -1;
#pragma unroll
      for (int u = 0; u < KG; ++u) {
        const int k = k0 + u < K ? k0 + u : K - 1;
        sl[u] = s_slot[wv][k];
        ok[u] = (k0 + u < K) && sl[u] >= 0;
      }
#pragma unroll
      for (int u = KG - 1; u >= 0; --u) fb = ok[u] ? sl[u] : fb;
      if (fb < 0) continue;
      u32x4 o[KG];
#pragma unroll
      for (int u = 0; u < KG; ++u)
        o[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(dXs + (int64_t)(ok[u] ? sl[u] : fb) * d + c * 8));
#pragma unroll
      for (int u = 0; u < KG; ++u)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float lo = acc[2 * h] + dev::bf16_bits_to_f32(o[u][h] & 0xFFFFu);
          const float hi = acc[2 * h + 1] + dev::bf16_bits_to_f32(o[u][h] >> 16);
          acc[2 * h] = ok[u] ? lo : acc[2 * h];
          acc[2 * h + 1] = ok[u] ? hi : acc[2 * h + 1];
        }
    }
    for (int k0 = 0; k0 < K; k0 += KG) {
      u32x4 o[KG];
      float gk[KG];
#pragma unroll
      for (int u = 0; u < KG; ++u) {
        const int k = k0 + u < K ? k0 + u : K - 1;
        gk[u] = (k0 + u < K) ? s_dsel[wv][k] : 0.f;
        o[u] = *reinterpret_cast<const u32x4*>(W_rT + (int64_t)s_id[wv][k] * d + c * 8);
      }
#pragma unroll
      for (int u = 0; u < KG; ++u)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc[2 * h] = fmaf(gk[u], dev::bf16_bits_to_f32(o[u][h] & 0xFFFFu), acc[2 * h]);
          acc[2 * h + 1] = fmaf(gk[u], dev::bf16_bits_to_f32(o[u][h] >> 16), acc[2 * h + 1]);
        }
    }
    u32x4 out;
#pragma unroll
    for (int h = 0; h < 4; ++h) out[h] = dev::pack_bf16x2(acc[2 * h], acc[2 * h + 1]);
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(dX + t * (int64_t)d + c * 8));
  }
}

// dW_r[i][e] = sum over splits z of part[z][i][e] (pitch Epad), in z order.
__global__ __launch_bounds__(256) void router_grad_sum_kernel(const float* __restrict__ part,
                                                              float* __restrict__ dW_r, int d,
                                                              int E, int Epad, int parts) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)d * E) return;
  const int64_t i = idx / E;
  const int e = (int)(idx - i * E);
  const int64_t stride = (int64_t)d * Epad;
  float v = 0.f;
  for (int z = 0; z < parts; ++z) v += part[z * stride + i * Epad + e];
  dW_r[idx] = v;
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

template <typename Kern>
hipError_t allow_lds(Kern* k, int bytes = kLds) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

int pad64(int E) { return (E + 63) / 64 * 64; }

// two 64-row stages (the measured best; see the stage note at BetaGeo)
constexpr int kBNst = 2, kBBk = 64;
constexpr int kBLds = BetaGeo<kBNst, kBBk>::kLds;

}  // namespace

int bwd_router_ksplit(const Problem& p) {
  const int64_t tiles = (int64_t)((p.d + kTile - 1) / kTile) * ((pad64(p.E) + kTile - 1) / kTile);
  int64_t z = 256 / tiles;
  if (z > 32) z = 32;
  if (z > p.T / 256) z = p.T / 256;      // at least four 64-deep k-steps per split
  return z > 1 ? (int)z : 1;
}

size_t backward_ws_bytes(const Problem& p, BackwardWs* w, unsigned char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* ptr = base ? base + off : nullptr;
    off += (bytes + 255) / 256 * 256;
    return ptr;
  };
  const int64_t rows = p.rows_max;
  const int NT = (p.n + kTile - 1) / kTile;
  const int Epad = pad64(p.E);
  BackwardWs ws{};
  ws.gs = reinterpret_cast<float*>(take((size_t)rows * 4));
  ws.dS_part = reinterpret_cast<float*>(take((size_t)rows * NT * 4));
  ws.dH = reinterpret_cast<uint16_t*>(take((size_t)rows * 2 * p.n * 2));
  ws.gA = reinterpret_cast<uint16_t*>(take((size_t)rows * p.n * 2));
  ws.dXs = reinterpret_cast<uint16_t*>(take((size_t)rows * p.d * 2));
  ws.dl = reinterpret_cast<uint16_t*>(take((size_t)p.T * Epad * 2));
  ws.W_rT = reinterpret_cast<uint16_t*>(take((size_t)p.E * p.d * 2));
  ws.zero = reinterpret_cast<uint32_t*>(take(kZeroBytes));
  ws.dWr_part = reinterpret_cast<float*>(take((size_t)bwd_router_ksplit(p) * p.d * Epad * 4));
  if (w) *w = ws;
  return off;
}

hipError_t launch_zero_grads(const Problem& p, float* dW_r, float* dW_gate, float* dW_up,
                             float* dW_down, hipStream_t s) {
  const int64_t nr = (int64_t)p.d * p.E, nw = (int64_t)p.E * p.d * p.n;
  float* outs[4] = {dW_r, dW_gate, dW_up, dW_down};
  const int64_t ns[4] = {nr, nw, nw, nw};
  for (int i = 0; i < 4; ++i) {
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((ns[i] + 255) / 256)), dim3(256), 0, s,
                       outs[i], ns[i]);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_backward(const Problem& p, const void* X, const void* W_r, const void* W_gate,
                           const void* W_up, const void* W_down, const void* dY,
                           const int32_t* ids, const float* gates, const int32_t* inv,
                           const int32_t* perm, const int32_t* offsets, const int32_t* table,
                           const void* Hpre, void* dX, float* dW_r, float* dW_gate, float* dW_up,
                           float* dW_down, const BackwardWs& w, hipStream_t s) {
  if (!p.bf16) return hipErrorNotSupported;
  if (p.K > kMaxK) return hipErrorInvalidValue;
  hipError_t err;
  const int64_t TK = p.T * (int64_t)p.K;
  const int64_t mtiles = max_row_tiles(p, kTile);
  const int NTn = (p.n + kTile - 1) / kTile, NTd = (p.d + kTile - 1) / kTile;
  const int Epad = pad64(p.E);
  const uint16_t* zero = reinterpret_cast<const uint16_t*>(w.zero);
#define MOE_BWD_TRY(x) do { err = (x); if (err != hipSuccess) return err; } while (0)
  hipLaunchKernelGGL(slot_gate_kernel, dim3((unsigned)((TK + 255) / 256)), dim3(256), 0, s, gates,
                     inv, w.gs, TK, w.zero);
  MOE_BWD_TRY(hipGetLastError());
  hipLaunchKernelGGL(transpose_router_kernel, dim3((unsigned)(((int64_t)p.d * p.E + 255) / 256)),
                     dim3(256), 0, s, (const uint16_t*)W_r, w.W_rT, p.d, p.E);
  MOE_BWD_TRY(hipGetLastError());
  // dA' = dY[perm] W_down^T, consumed by the dSwiGLU epilogue: dH, g A, dS shares
  {
    auto* k = alpha_gemm<kEpiDSwiGLU, true>;
    MOE_BWD_TRY(allow_lds(k));
    hipLaunchKernelGGL(k, dim3((unsigned)(mtiles * NTn)), dim3(kThreads), (size_t)kLds, s,
                       (const uint16_t*)dY, perm, table, (const uint16_t*)W_down, nullptr, p.T,
                       p.d, p.d, p.n, NTn, nullptr, (const uint16_t*)Hpre, w.gs, w.dH, w.gA,
                       w.dS_part);
    MOE_BWD_TRY(hipGetLastError());
  }
  // dXs = dHg W_gate^T + dHu W_up^T per slot (k runs over the 2n columns of dH)
  {
    auto* k = alpha_gemm<kEpiStore, false>;
    MOE_BWD_TRY(allow_lds(k));
    hipLaunchKernelGGL(k, dim3((unsigned)(mtiles * NTd)), dim3(kThreads), (size_t)kLds, s, w.dH,
                       nullptr, table, (const uint16_t*)W_gate, (const uint16_t*)W_up, p.T,
                       2 * p.n, p.n, p.d, NTd, w.dXs, nullptr, nullptr, nullptr, nullptr, nullptr);
    MOE_BWD_TRY(hipGetLastError());
  }
  hipLaunchKernelGGL(token_backward_kernel, dim3((unsigned)((p.T + kTokWaves - 1) / kTokWaves)),
                     dim3(64 * kTokWaves), 0, s, w.dS_part, NTn, ids, gates, inv, w.dXs, w.W_rT,
                     w.dl, (uint16_t*)dX, p.T, p.d, p.K, Epad);
  MOE_BWD_TRY(hipGetLastError());
  // dW_down[e] = (g A)^T dY[perm]
  {
    auto* k = beta_gemm<false, true, kBNst, kBBk>;
    MOE_BWD_TRY(allow_lds(k, kBLds));
    const int IT = NTn, JT = NTd;
    hipLaunchKernelGGL(k, dim3((unsigned)(p.E * IT * JT), 1), dim3(kThreads), (size_t)kBLds, s,
                       w.gA, (const uint16_t*)dY, perm, offsets, (int64_t)0, p.T, p.n, p.d, IT, JT,
                       1, zero, dW_down, nullptr, p.d, (int64_t)0);
    MOE_BWD_TRY(hipGetLastError());
  }
  // dW_gate[e] | dW_up[e] = X[perm]^T (dHg | dHu)
  {
    auto* k = beta_gemm<true, false, kBNst, kBBk>;
    MOE_BWD_TRY(allow_lds(k, kBLds));
    const int IT = NTd, JT = (2 * p.n + kTile - 1) / kTile;
    hipLaunchKernelGGL(k, dim3((unsigned)(p.E * IT * JT), 1), dim3(kThreads), (size_t)kBLds, s,
                       (const uint16_t*)X, w.dH, perm, offsets, (int64_t)0, p.T, p.d, 2 * p.n, IT,
                       JT, 1, zero, dW_gate, dW_up, p.n, (int64_t)0);
    MOE_BWD_TRY(hipGetLastError());
  }
  // dW_r = X^T dl: one group of T rows split over k, partials of pitch Epad,
  // then the sum over the splits
  {
    const int zsplit = bwd_router_ksplit(p);
    auto* k = beta_gemm<false, false, kBNst, kBBk>;
    MOE_BWD_TRY(allow_lds(k, kBLds));
    const int IT = NTd, JT = (Epad + kTile - 1) / kTile;
    hipLaunchKernelGGL(k, dim3((unsigned)(IT * JT), (unsigned)zsplit), dim3(kThreads),
                       (size_t)kBLds, s, (const uint16_t*)X, w.dl, perm, nullptr, p.T, p.T, p.d,
                       Epad, IT, JT, zsplit, zero, w.dWr_part, nullptr, Epad,
                       (int64_t)p.d * Epad);
    MOE_BWD_TRY(hipGetLastError());
    const int64_t n = (int64_t)p.d * p.E;
    hipLaunchKernelGGL(router_grad_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       w.dWr_part, dW_r, p.d, p.E, Epad, zsplit);
    MOE_BWD_TRY(hipGetLastError());
  }
#undef MOE_BWD_TRY
  return hipSuccess;
}

}  // namespace moe
