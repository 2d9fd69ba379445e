// Steps 6-7 of the layer: the two variable-M grouped GEMMs.
//
// up:   H[s,:] = silu(x W_gate[e]) * (x W_up[e]),  x = X[perm_token[s]]
// down: O[s,:] = H[s,:] W_down[e]
// for every expert-major slot s of expert e.  The SonicMoE article lists these
// as steps 3-5 of its GPU pipeline (§3), reads the token rows by index inside
// the GEMM's operand load instead of building a gathered T*K*d copy (§6.2),
// and applies SwiGLU while the products are still in the accumulators (§6.3).
//
// bf16 kernel (gfx950, one 512-thread workgroup per tile, 1 per CU):
// * Tile = 256 expert-major rows x 256 accumulator columns (up: 128 W_gate
//   columns + the same 128 W_up columns, so each lane holds matching gate and
//   up values and SwiGLU is register-local; down: 256 W_down columns).
//   Row tiles come from a device-built table (expert, row range), so experts
//   of any size share one launch; the grid is a host-side upper bound and
//   surplus workgroups exit at once.
// * Loads go global -> LDS with global_load_lds_dwordx4 (no VGPR staging).
//   Each lane supplies its own global address, which is what makes the row
//   gather free: a lane simply points at row perm_token[s] of X.  Two LDS
//   stages of 64 KB (k depth 64, so every gathered row chunk is a whole
//   128-byte line) keep the next k-step loading while this one multiplies.
// * 8 waves (2 per SIMD) in a 2 x 4 grid; each wave owns 128 token rows x 64
//   accumulator columns (128 fp32 accumulators per lane).  Fragments are read
//   one 16-deep sub-step ahead of the MFMAs that use them, and 32-row blocks
//   past an expert's last row skip their MFMAs.
// * LDS layouts are XOR-swizzled at 16-byte granularity so both fragment
//   reads are bank-conflict free: token rows (128 B) use slot c^((r>>1)&7);
//   weight rows (512 B, natural [k][n] order) use slot q^(4*(k&3)) and are
//   read with ds_read_b64_tr_b16, which hands each lane 4 consecutive k of
//   one column -- the MFMA operand layout -- so weights are never transposed.
// * The MFMA computes the transposed tile (weights as the A operand, tokens
//   as B), so each lane ends with 4 consecutive output columns of one row.
// * Epilogue: the finished tile is written into the (now idle) stage buffers
//   as a row-major bf16 tile and stored as whole rows with 16-byte lanes;
//   storing straight from the accumulators would write 16-byte pieces of 32
//   different rows per instruction, which made the store phase cost about a
//   third of the down-projection's time.  The stores are non-temporal: the
//   output is not read again by this kernel, and keeping it out of L2 leaves
//   the space to the operand tiles (down projection and the combine after
//   it about 2% and 6% faster).
// * Workgroup ids are remapped so that consecutive tiles (same expert, same
//   token rows) run on the same XCD and share its L2.
// * Optionally (stream_rows > 0) the grid also holds one weight-streaming
//   block (gemm_stream.hpp) per expert and column block, after every tile:
//   experts with at most stream_rows rows are computed there instead of by
//   their single, mostly empty tile.
//
// fp32 kernel (correctness-sized layers): fp32 MFMA on 64 x 64 tiles.
#include "gemm_stream.hpp"

namespace moe {
namespace {

using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using i16x4 = short __attribute__((ext_vector_type(4)));
using f32x16 = float __attribute__((ext_vector_type(16)));
using u32x2 = uint32_t __attribute__((ext_vector_type(2)));

constexpr int BN = 256;          // accumulator columns per tile
// Column tiles per block of an expert's tile order (up / down), measured on
// the Qwen3-shaped layer: the up projection runs best with whole-expert
// blocks, the down projection with narrow ones (-4%).
constexpr int kColBlockUp = 8, kColBlockDown = 3;

// Tile geometry: a WGM x WGN grid of waves, each owning WTB 32-row token
// blocks x WCB 32-column blocks; NST LDS stages of depth BK (32 or 64).
template <int WGM, int WGN, int WTB, int WCB, int NST, int BK>
struct Geo {
  static constexpr int kWaves = WGM * WGN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = WGM * WTB * 32;
  static_assert(WGN * WCB * 32 == BN, "waves must cover the 256 accumulator columns");
  static constexpr int kAStage = BM * BK * 2;
  static constexpr int kBStage = BK * BN * 2;
  static constexpr int kStageBytes = kAStage + kBStage;
  static constexpr int kAInstr = kAStage / 1024 / kWaves;   // copy instructions per wave per stage
  static constexpr int kBInstr = kBStage / 1024 / kWaves;
  static_assert(kAInstr * 1024 * kWaves == kAStage && kBInstr * 1024 * kWaves == kBStage, "copy split");
  static constexpr int kInstr = kAInstr + kBInstr;
  static constexpr int kLds = NST * kStageBytes;
  // token tile rows hold BK/8 16-byte chunks; XOR swizzle slot = c ^ ((r >> kSh) & (kCpr-1))
  static constexpr int kCpr = BK / 8;
  static constexpr int kSh = (BK == 32) ? 2 : 1;
  static_assert(BK == 32 || BK == 64, "stage depth");
};
// Production geometry: 256 x 256 tiles, 8 waves (2 per SIMD) in a 2 x 4 grid,
// each wave 128 tokens x 64 columns (128 fp32 accumulators per lane).  The
// wave tile is tall (more token rows than weight columns) because weight
// fragments come through the transpose reads, whose LDS throughput is well
// below that of the 16-byte token-fragment reads.
constexpr int kWGM = 2, kWGN = 4, kWTB = 4, kWCB = 2;
// Two 64-deep stages of 64 KB: 64-deep stages make every gathered token-row
// chunk a whole 128-byte line.  The copy rate is bounded by the requests an
// L1 keeps in flight, so full-line requests move more bytes per request.
constexpr int kNST = 2, kBK = 64;
using ProdGeo = Geo<kWGM, kWGN, kWTB, kWCB, kNST, kBK>;
static_assert(ProdGeo::BM == kGemmBM, "tile table rows must match the kernel tile");
// Weight-streaming blocks appended to a launch: passes of kStreamRows rows,
// kStreamCols weight columns per block, the tile kernel's 8 waves.
constexpr int kStreamRows = 64, kStreamCols = 256;
using StreamGeo = wstream::Geo<kStreamRows, kStreamCols, kWGM * kWGN>;
static_assert(StreamGeo::kThreads == ProdGeo::kThreads, "one workgroup size for both kinds");
static_assert(kMaxStreamRows <= kGemmBM, "a streamed expert must be a single tile");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt lgkmcnt(0) as a builtin (gfx9 encoding: vmcnt and expcnt left at
// their maxima), so the compiler's own wait tracking sees it.
constexpr int kWaitLds = 0xC07F;

// Wait until at most `pending` stages (INSTR copy instructions each) of this
// wave are still in flight.
template <int INSTR>
__device__ __forceinline__ void wait_copies(int pending) {
  if (pending >= 4) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * INSTR) : "memory");
  else if (pending == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * INSTR) : "memory");
  else if (pending == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * INSTR) : "memory");
  else if (pending == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(INSTR) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * dev::sigmoid(g) * u;
}

template <int WTB, int WCB>
struct Frags {
  bf16x8 a[WTB];   // token fragments (MFMA B operand), one per 32-row block
  bf16x8 b[WCB];   // weight fragments (MFMA A operand), one per 32-column block
};

template <bool UP, int WGM, int WGN, int WTB, int WCB, int NST, int BK>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void grouped_gemm_bf16(
    const uint16_t* __restrict__ A,       // up: X [T][Kd]; down: H [rows][Kd]
    const int32_t* __restrict__ perm,     // up: expert-major slot -> token
    const int32_t* __restrict__ table,    // tile table
    const uint16_t* __restrict__ B0,      // up: W_gate; down: W_down  ([E][Kd][N])
    const uint16_t* __restrict__ B1,      // up: W_up
    uint16_t* __restrict__ C,             // up: H [rows][N]; down: O [rows][N]
    uint16_t* __restrict__ Hpre,          // up, or NULL: pre-activations [rows][2N] (gate | up)
    int64_t T, int Kd, int N, int NT,
    const int32_t* __restrict__ offsets,  // [E+1] expert row ranges (weight-streaming blocks)
    int64_t rows_max, int stream_rows, int stream_base) {
  using G = Geo<WGM, WGN, WTB, WCB, NST, BK>;
  constexpr int kCpr = G::kCpr, kSh = G::kSh, kRowsPerCopy = 64 / kCpr;
  constexpr int KS = BK / 16;              // 16-deep MFMA sub-steps per stage
  constexpr int BM = G::BM, kAStage = G::kAStage, kStageBytes = G::kStageBytes;
  constexpr int kAInstr = G::kAInstr, kBInstr = G::kBInstr, kInstr = G::kInstr;
  constexpr int kStages = NST;
  constexpr int kHalf = WCB / 2;           // up: gate blocks (then as many up blocks)
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  // Workgroups from stream_base on are weight-streaming blocks: expert
  // bid / NB, column block bid % NB, for the experts with 1..stream_rows
  // rows (the tiles of those experts exit below).  They come after every
  // tile, so the dispatcher starts them on the CUs that tiles leave free.
  if (stream_rows > 0 && (int)blockIdx.x >= stream_base) {
    constexpr int kCols = UP ? kStreamCols / 2 : kStreamCols;
    const int NB = (N + kCols - 1) / kCols;
    const int idx = (int)blockIdx.x - stream_base;
    wstream::stream_block<UP, kStreamRows, kStreamCols, WGM * WGN>(
        A, perm, offsets, B0, B1, C, T, Kd, N, rows_max, stream_rows, idx / NB, idx - (idx / NB) * NB,
        smem);
    return;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wm = w / WGN, wn = w - (w / WGN) * WGN;
  const uint32_t lds_base = (uint32_t)(size_t)(lds_ptr_t)smem;

  // ---- tile decode.  Workgroups are dispatched to the 8 XCDs round robin
  // (workgroup b runs on XCD b%8); ids are remapped so that each XCD takes a
  // contiguous range of tiles (same expert, same token rows close together)
  // and the tiles running at once on an XCD share operands in its L2.
  const int total = table[0] * NT;
  const int bid = blockIdx.x;
  if (bid >= total) return;
  const int q8 = total >> 3, r8 = total & 7;
  const int xcd = bid & 7, j = bid >> 3;
  const int L = xcd * q8 + (xcd < r8 ? xcd : r8) + j;
  // Within an expert (c row tiles x NT column tiles, ids [first*NT,
  // (first+c)*NT)), tiles run in blocks of kColBlock columns: block by block,
  // row tile by row tile, column by column.  The c*kColBlock tiles of a block
  // are consecutive ids, so they run together on one XCD and share both the
  // token rows (across columns) and the weight slices (across row tiles).
  constexpr int kColBlock = UP ? kColBlockUp : kColBlockDown;
  const int m0 = L / NT;
  const uint32_t head = (uint32_t)table[4 * (m0 + 1)];
  const int first = table[4 * (m0 + 1) + 3];
  const int c = tile_expert_tiles(head);
  const int local = L - first * NT;
  const int blk = local / (c * kColBlock);
  const int inb = local - blk * (c * kColBlock);
  const int bw = (NT - blk * kColBlock < kColBlock) ? NT - blk * kColBlock : kColBlock;
  const int mt = first + inb / bw;
  const int nt = blk * kColBlock + (inb - (inb / bw) * bw);
  if (mt >= table[0]) return;   // only with a table cut at its capacity (inconsistent offsets)
  const int32_t* ent = table + 4 * (mt + 1);
  const int e = tile_expert((uint32_t)ent[0]), row0 = ent[1];
  const int nrows = ent[2] - row0;
  // an expert of at most stream_rows rows (one tile) is a weight-streaming block's
  if (c == 1 && nrows <= stream_rows) return;
  const int ncol0 = nt * (UP ? BN / 2 : BN);   // first output column of the tile
  // 32-row token blocks of this wave that hold any valid row (uniform per wave)
  int ntb = (nrows - wm * (WTB * 32) + 31) / 32;
  ntb = ntb < 0 ? 0 : (ntb > WTB ? WTB : ntb);

  // ---- copy source addresses
  // token tile (2*BK-byte rows): copy instruction j = kAInstr*w + i fills rows
  // kRowsPerCopy*j + lane/kCpr, slot lane%kCpr holding k chunk
  // slot^((row>>kSh)&(kCpr-1)).
  const uint16_t* asrc[kAInstr];
#pragma unroll
  for (int i = 0; i < kAInstr; ++i) {
    const int r = (w * kAInstr + i) * kRowsPerCopy + (lane / kCpr);
    const int c = (lane % kCpr) ^ ((r >> kSh) & (kCpr - 1));
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
  // weight tile (512 B rows, natural [k][n]): copy instruction j = kBInstr*w + i
  // fills rows 2j + lane/32, slot lane%32 holding column chunk slot^(4*(k&3));
  // k&3 = (2j + lane/32)&3 depends on the parity of j only.
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

  // Down projection: tile L starts its k loop at k-step L mod KT and wraps.
  // An XCD starts about one tile per k-step, so the tiles running together
  // then work on the same k slice and share it in L2 (the down projection's
  // working set per XCD, ~10 row tiles and 3 column slices, is just above
  // L2).  3% faster there; neutral for the up projection, which keeps the
  // natural order.  The order of each tile's sum is fixed by L alone, so
  // results stay bit-reproducible.
  const int KTall = Kd / BK;
  const int rot = UP ? 0 : L % KTall;
  auto issue_stage = [&](int kt) {
    const uint32_t As = lds_base + (uint32_t)((kt % kStages) * kStageBytes);
    const uint32_t Bs = As + kAStage;
    int kk = kt + rot;
    if (kk >= KTall) kk -= KTall;
#pragma unroll
    for (int i = 0; i < kAInstr; ++i) dev::lds_copy16(asrc[i] + kk * BK, As + (w * kAInstr + i) * 1024);
#pragma unroll
    for (int i = 0; i < kBInstr; ++i) {
      const int jb = w * kBInstr + i;
      dev::lds_copy16(bsrc[jb & 1] + (int64_t)(kk * BK + 2 * jb) * N, Bs + jb * 1024);
    }
  };

  // ---- fragment geometry
  // token fragment: lane -> token row wm*32*WTB + tb*32 + lane%32, k chunk 2*ks + lane/32
  int a_off[WTB][KS];
#pragma unroll
  for (int tb = 0; tb < WTB; ++tb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int r = wm * (WTB * 32) + tb * 32 + (lane & 31);
      const int c = ks * 2 + (lane >> 5);
      a_off[tb][ks] = r * (2 * BK) + ((c ^ ((r >> kSh) & (kCpr - 1))) * 16);
    }
  // weight fragment via transpose loads: group g = lane/16, lane s in group ->
  // row 16*ks + 8*(g/2) + s/4 (+4 for the second half), column 16*(g%2) + 4*(s%4)
  const int g = lane >> 4, s16 = lane & 15;
  const int tr_row = 8 * (g >> 1) + (s16 >> 2);
  int b_off[WCB][2];
#pragma unroll
  for (int cb = 0; cb < WCB; ++cb) {
    int colbase;
    if (UP) colbase = (cb < kHalf) ? (wn * kHalf * 32 + cb * 32) : (BN / 2 + wn * kHalf * 32 + (cb - kHalf) * 32);
    else colbase = wn * WCB * 32 + cb * 32;
    const int n = colbase + 16 * (g & 1) + 4 * (s16 & 3);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = tr_row + 4 * h;
      const int q = n >> 3;
      b_off[cb][h] = kAStage + k * 512 + ((q ^ (4 * (k & 3))) * 16) + ((n >> 2) & 1) * 8;
    }
  }

  auto read_frags = [&](Frags<WTB, WCB>& f, int kt, int ks) {
    const unsigned char* S = smem + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int tb = 0; tb < WTB; ++tb)
      f.a[tb] = *reinterpret_cast<const bf16x8*>(S + a_off[tb][ks]);
#pragma unroll
    for (int cb = 0; cb < WCB; ++cb) {
      i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(S + b_off[cb][0] + ks * 16 * 512));
      i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(S + b_off[cb][1] + ks * 16 * 512));
      f.b[cb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  f32x16 acc[WCB][WTB];
#pragma unroll
  for (int cb = 0; cb < WCB; ++cb)
#pragma unroll
    for (int tb = 0; tb < WTB; ++tb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[cb][tb][v] = 0.f;

  auto mma = [&](const Frags<WTB, WCB>& f) {
#pragma unroll
    for (int tb = 0; tb < WTB; ++tb)
      if (tb < ntb) {
#pragma unroll
        for (int cb = 0; cb < WCB; ++cb)
          acc[cb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[cb], f.a[tb], acc[cb][tb], 0, 0, 0);
      }
  };

  // ---- main loop: stage kt+NST-1 copies in flight while stage kt is
  // multiplied; fragments are read one 16-deep sub-step ahead of the MFMAs.
  // Order inside an iteration (pinned with sched_barrier): wait for the
  // fragments already in flight, issue the next fragment reads, then the
  // MFMAs on the landed fragments, so LDS reads overlap the matrix work.
  const int KT = Kd / BK;   // the host requires Kd % 64 == 0
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < KT) issue_stage(s);
  wait_copies<kInstr>((KT - 1 < kStages - 2) ? KT - 1 : kStages - 2);
  asm volatile("s_barrier" ::: "memory");

  Frags<WTB, WCB> cur, nxt;
  read_frags(cur, 0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + kStages - 1 < KT) issue_stage(kt + kStages - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      __builtin_amdgcn_s_waitcnt(kWaitLds);            // cur landed
      __builtin_amdgcn_sched_barrier(0);
      read_frags(nxt, kt, ks + 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(cur);
      __builtin_amdgcn_sched_barrier(0);
      // nxt landed (and, on the last sub-step, every read of stage kt is
      // done).  Waiting here, on both paths of the branch below, keeps the
      // compiler from merging the pending reads of the two paths.
      __builtin_amdgcn_s_waitcnt(kWaitLds);
      if (ks + 2 < KS) {
        read_frags(cur, kt, ks + 2);
      } else if (kt + 1 < KT) {
        // stage kt+1 must have landed (own copies), then publish it to all
        // waves; the barrier also tells every wave that stage kt is free.
        const int last = (kt + kStages - 1 < KT) ? kt + kStages - 1 : KT - 1;
        wait_copies<kInstr>(last - (kt + 1));
        asm volatile("s_barrier" ::: "memory");
        read_frags(cur, kt + 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mma(nxt);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue: the tile goes through LDS so that global stores are whole
  // rows.  A lane holds, for token row lane%32 of block tb, output columns
  // 8*(v/4) + 4*(lane/32) + v%4 of block cb (v = accumulator index); it writes
  // them as 8-byte pieces into a row-major bf16 tile whose 16-byte chunks are
  // XOR-swizzled by row, then every thread stores 16-byte chunks of whole rows.
  constexpr int OW = UP ? BN / 2 : BN;        // output columns per tile
  constexpr int kRowBytes = OW * 2;
  constexpr int kChunks = kRowBytes / 16;
  static_assert(BM * kRowBytes <= G::kLds, "output tile must fit the stage buffers");
  asm volatile("s_barrier" ::: "memory");     // every wave is done reading the last stage
#pragma unroll
  for (int tb = 0; tb < WTB; ++tb) {
    const int rloc = wm * (WTB * 32) + tb * 32 + (lane & 31);
    unsigned char* srow = smem + rloc * kRowBytes;
#pragma unroll
    for (int cb = 0; cb < (UP ? kHalf : WCB); ++cb)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int col = wn * (UP ? kHalf : WCB) * 32 + cb * 32 + 8 * v4 + 4 * (lane >> 5);
        float h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          h[r] = UP ? silu_mul(acc[cb][tb][4 * v4 + r], acc[cb + kHalf][tb][4 * v4 + r])
                    : acc[cb][tb][4 * v4 + r];
        const u32x2 pk = {dev::pack_bf16x2(h[0], h[1]), dev::pack_bf16x2(h[2], h[3])};
        const int chunk = (col >> 3) ^ (rloc & (kChunks - 1));
        *reinterpret_cast<u32x2*>(srow + chunk * 16 + ((col >> 2) & 1) * 8) = pk;
      }
  }
  __syncthreads();
  constexpr int kIters = BM * kChunks / G::kThreads;
  static_assert(kIters * G::kThreads == BM * kChunks, "store split");
#pragma unroll
  for (int i = 0; i < kIters; ++i) {
    const int idx = tid + i * G::kThreads;
    const int rloc = idx / kChunks, c = idx - (idx / kChunks) * kChunks;
    const int col = ncol0 + c * 8;
    if (rloc < nrows && col < N) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(
          smem + rloc * kRowBytes + ((c ^ (rloc & (kChunks - 1))) * 16));
      __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(C + (int64_t)(row0 + rloc) * N + col));
    }
  }
  if (UP && Hpre != nullptr) {
    // training forward: also keep the pre-activations (x W_gate | x W_up) of
    // the tile, staged the same way: a row of the tile holds its 128 gate
    // columns then the same 128 up columns.
    constexpr int kPRow = BN * 2;
    constexpr int kPChunks = kPRow / 16;
    __syncthreads();                          // the staged output tile has been read out
#pragma unroll
    for (int tb = 0; tb < WTB; ++tb) {
      const int rloc = wm * (WTB * 32) + tb * 32 + (lane & 31);
      unsigned char* srow = smem + rloc * kPRow;
#pragma unroll
      for (int cb = 0; cb < WCB; ++cb)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int colbase = (cb < kHalf) ? (wn * kHalf * 32 + cb * 32)
                                           : (BN / 2 + wn * kHalf * 32 + (cb - kHalf) * 32);
          const int col = colbase + 8 * v4 + 4 * (lane >> 5);
          const u32x2 pk = {dev::pack_bf16x2(acc[cb][tb][4 * v4], acc[cb][tb][4 * v4 + 1]),
                            dev::pack_bf16x2(acc[cb][tb][4 * v4 + 2], acc[cb][tb][4 * v4 + 3])};
          const int chunk = (col >> 3) ^ (rloc & (kPChunks - 1));
          *reinterpret_cast<u32x2*>(srow + chunk * 16 + ((col >> 2) & 1) * 8) = pk;
        }
    }
    __syncthreads();
    constexpr int kPIters = BM * kPChunks / G::kThreads;
#pragma unroll
    for (int i = 0; i < kPIters; ++i) {
      const int idx = tid + i * G::kThreads;
      const int rloc = idx / kPChunks, c = idx - (idx / kPChunks) * kPChunks;
      const int half = c / (kPChunks / 2);                // 0: gate, 1: up
      const int col = ncol0 + (c - half * (kPChunks / 2)) * 8;
      if (rloc < nrows && col < N) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(
            smem + rloc * kPRow + ((c ^ (rloc & (kPChunks - 1))) * 16));
        __builtin_nontemporal_store(
            v, reinterpret_cast<bf16x8*>(Hpre + (int64_t)(row0 + rloc) * (2 * N) + half * N + col));
      }
    }
  }
}

// stream_rows > 0 (needs offsets): experts with 1..stream_rows rows run as
// weight-streaming blocks appended to the grid, E * NB of them.
template <bool UP>
hipError_t launch_bf16(const uint16_t* A, const int32_t* perm, const int32_t* table,
                       const uint16_t* B0, const uint16_t* B1, uint16_t* C, uint16_t* Hpre,
                       int64_t T, int Kd, int N, int64_t mtiles, int E, const int32_t* offsets,
                       int64_t rows_max, int stream_rows, hipStream_t s) {
  if (stream_rows < 0 || stream_rows > kMaxStreamRows || (stream_rows > 0 && !offsets))
    return hipErrorInvalidValue;
  const int NT = (N + (UP ? BN / 2 : BN) - 1) / (UP ? BN / 2 : BN);
  const int64_t tiles = mtiles * NT;
  const int NB = (N + (UP ? kStreamCols / 2 : kStreamCols) - 1) / (UP ? kStreamCols / 2 : kStreamCols);
  const int64_t grid = tiles + (stream_rows > 0 ? (int64_t)E * NB : 0);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const int lds = (stream_rows > 0 && StreamGeo::kLds > ProdGeo::kLds) ? StreamGeo::kLds : ProdGeo::kLds;
  auto* kern = grouped_gemm_bf16<UP, kWGM, kWGN, kWTB, kWCB, kNST, kBK>;
  hipError_t err = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(ProdGeo::kThreads), (size_t)lds, s, A, perm,
                     table, B0, B1, C, Hpre, T, Kd, N, NT, offsets, rows_max, stream_rows,
                     (int)tiles);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fp32 (MFMA)
// 64-row x 64-column tiles of 4 waves, each 32 x 32 with
// v_mfma_f32_32x32x2_f32 over 32-deep k slices staged in LDS; only for the
// fp32 element type (a correctness-sized layer).  A lane supplies
// A[row lane%32][k lane/32] and B[k lane/32][col lane%32] and ends with
// columns lane%32 of rows 8*(v/4) + 4*(lane/32) + v%4 of its wave's block.
constexpr int kF32Rows = 64, kF32Cols = 64, kF32K = 32;
constexpr int kF32Sub = kGemmBM / kF32Rows;   // sub-tiles per table tile
using f32x16v = float __attribute__((ext_vector_type(16)));

template <bool UP>
__global__ __launch_bounds__(256) void grouped_gemm_f32(
    const float* __restrict__ A, const int32_t* __restrict__ perm, const int32_t* __restrict__ table,
    const float* __restrict__ B0, const float* __restrict__ B1, float* __restrict__ C, int64_t T,
    int Kd, int N, int NT) {
  constexpr int TM = kF32Rows, TN = kF32Cols, TK = kF32K;
  __shared__ float As[TM][TK + 1];
  __shared__ float Bg[TK][TN];
  __shared__ float Bu[UP ? TK : 1][TN];
  // each 256-row table tile is covered by kF32Sub sub-tiles of TM rows
  constexpr int kSub = kF32Sub;
  const int total = table[0] * kSub * NT;
  const int bid = blockIdx.x;
  if (bid >= total) return;
  const int mt = bid / (kSub * NT);
  const int rem = bid - mt * (kSub * NT);
  const int sub = rem / NT, nt = rem - (rem / NT) * NT;
  const int32_t* ent = table + 4 * (mt + 1);
  const int e = tile_expert((uint32_t)ent[0]), row0 = ent[1] + sub * TM;
  const int nrows = (ent[2] - row0 < TM) ? ent[2] - row0 : TM;
  if (nrows <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const float* Wg = B0 + (int64_t)e * Kd * N;
  const float* Wu = UP ? B1 + (int64_t)e * Kd * N : nullptr;
  f32x16v ag, au;
#pragma unroll
  for (int v = 0; v < 16; ++v) ag[v] = au[v] = 0.f;
  for (int k0 = 0; k0 < Kd; k0 += TK) {
    for (int idx = tid; idx < TM * TK; idx += 256) {
      const int r = idx / TK, c = idx - (idx / TK) * TK;
      const int rr = r < nrows ? r : nrows - 1;
      int64_t row;
      if (UP) {
        int64_t tok = perm[row0 + rr];
        row = tok < 0 ? 0 : (tok > T - 1 ? T - 1 : tok);
      } else {
        row = row0 + rr;
      }
      As[r][c] = (k0 + c < Kd) ? A[row * Kd + k0 + c] : 0.f;
    }
    for (int idx = tid; idx < TK * TN; idx += 256) {
      const int r = idx / TN, c = idx - (idx / TN) * TN;
      const int col = nt * TN + c;
      const bool ok = col < N && k0 + r < Kd;
      Bg[r][c] = ok ? Wg[(int64_t)(k0 + r) * N + col] : 0.f;
      if (UP) Bu[r][c] = ok ? Wu[(int64_t)(k0 + r) * N + col] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; kk += 2) {
      const float a = As[wm * 32 + (lane & 31)][kk + (lane >> 5)];
      ag = __builtin_amdgcn_mfma_f32_32x32x2f32(a, Bg[kk + (lane >> 5)][wn * 32 + (lane & 31)], ag, 0, 0, 0);
      if (UP)
        au = __builtin_amdgcn_mfma_f32_32x32x2f32(a, Bu[kk + (lane >> 5)][wn * 32 + (lane & 31)], au, 0, 0, 0);
    }
    __syncthreads();
  }
  const int col = nt * TN + wn * 32 + (lane & 31);
  if (col >= N) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (r >= nrows) continue;
    float out = ag[v];
    if (UP) out = out / (1.0f + expf(-out)) * au[v];
    C[(int64_t)(row0 + r) * N + col] = out;
  }
}

}  // namespace

hipError_t launch_gemm_up(const Problem& p, const void* X, const int32_t* perm,
                          const int32_t* table, const void* W_gate, const void* W_up, void* H,
                          hipStream_t s, void* Hpre, const int32_t* offsets, int stream_rows) {
  const int64_t mtiles = max_row_tiles(p, kGemmBM);
  if (p.bf16) {
    if (Hpre && stream_rows) return hipErrorInvalidValue;   // streamed rows store no pre-activations
    return launch_bf16<true>((const uint16_t*)X, perm, table, (const uint16_t*)W_gate,
                             (const uint16_t*)W_up, (uint16_t*)H, (uint16_t*)Hpre, p.T, p.d, p.n,
                             mtiles, p.E, offsets, p.rows_max, stream_rows, s);
  }
  if (Hpre) return hipErrorNotSupported;      // the training path is bf16 only
  const int NT = (p.n + kF32Cols - 1) / kF32Cols;
  hipLaunchKernelGGL(grouped_gemm_f32<true>, dim3((unsigned)(mtiles * kF32Sub * NT)), dim3(256), 0, s,
                     (const float*)X, perm, table, (const float*)W_gate, (const float*)W_up,
                     (float*)H, p.T, p.d, p.n, NT);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const Problem& p, const void* H, const int32_t* table,
                            const void* W_down, void* O, hipStream_t s, const int32_t* offsets,
                            int stream_rows) {
  const int64_t mtiles = max_row_tiles(p, kGemmBM);
  if (p.bf16)
    return launch_bf16<false>((const uint16_t*)H, nullptr, table, (const uint16_t*)W_down,
                              nullptr, (uint16_t*)O, nullptr, p.T, p.n, p.d, mtiles, p.E, offsets,
                              p.rows_max, stream_rows, s);
  const int NT = (p.d + kF32Cols - 1) / kF32Cols;
  hipLaunchKernelGGL(grouped_gemm_f32<false>, dim3((unsigned)(mtiles * kF32Sub * NT)), dim3(256), 0, s,
                     (const float*)H, nullptr, table, (const float*)W_down, nullptr, (float*)O,
                     p.T, p.n, p.d, NT);
  return hipGetLastError();
}

}  // namespace moe
