/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer library (forward and backward).
 *
 * The layer, for tokens X[T,d] and E SwiGLU experts of width n:
 *   1. router logits  l = X W_r (+ b)              (page "Routing-Free 与 OmniMoE", §1.1)
 *   2. softmax, top-K, gates renormalised over the K selected experts
 *                                                   (same page §1.1; "AI芯片如何支持MoE架构" §4.3)
 *   3-5. expert-major metadata: per-expert histogram, capacity cut in token
 *        order, exclusive scan, scatter index       (SonicMoE article §11; "算子与编译器：MoE 路由
 *                                                    与稀疏 Kernel" §3-§4; OmniMoE page §2.3)
 *   6. grouped GEMM over the gathered token rows with a SwiGLU epilogue -> H
 *   7. second grouped GEMM -> O                     (SonicMoE article §3, §6.2, §6.3)
 *   8. gate-weighted combine back to token order -> Y  (SonicMoE article §1, §6.1)
 * and, for training, its backward (SonicMoE article §6.1, §6.3, §6.4).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every call returns a moe_status; nothing throws across the ABI (an
 *   exception inside a call, such as a failed host allocation, returns
 *   MOE_ERR_HOST).  On failure moe_last_error() gives a message for the
 *   calling thread.
 * - Device entry points take device pointers owned by the caller and enqueue
 *   their kernels on `stream` (a hipStream_t passed as void*; NULL = the
 *   default stream).  They never synchronise, never copy to the host and
 *   never allocate: buffers and workspaces are the caller's.  Device faults
 *   therefore surface at the caller's next synchronisation.
 * - Debugging: with MOE_DEBUG_SYNC=1 in the environment (read at every
 *   call), each launch step synchronises `stream` and a kernel that failed
 *   is reported by that call as MOE_ERR_HIP, the message naming the step.
 *   Outputs are unchanged.  A stream being captured into a graph is not
 *   synchronised.
 * - Argument checks happen on the host before anything is enqueued; a failed
 *   check enqueues nothing.  A failed kernel launch gives MOE_ERR_HIP.
 * - Layouts are row-major and contiguous.  X, W_r, W_gate, W_up, W_down, H,
 *   O and Y have the element type desc->dtype (fp32 or bf16); logits, gates
 *   and bias are fp32 in both cases; ids, counts, offsets and slots are
 *   int32 (so T*K must stay below 2^31).  Arithmetic accumulates in fp32;
 *   H, O and Y are rounded to desc->dtype (round to nearest even).
 * - Every device pointer must be 16-byte aligned (MOE_ERR_ALIGNMENT).
 * - Supported shapes: 1 <= E <= 256, 1 <= K <= E, d and n multiples of 64
 *   (MOE_ERR_UNSUPPORTED otherwise), T >= 0 (T = 0 is a successful no-op,
 *   except that moe_backward then writes zero weight gradients).
 * - Identical inputs give bitwise identical outputs; moe_forward gives the
 *   same bits as the step-wise chain route_ws -> permute -> grouped_ffn ->
 *   combine with the same flags.  Calls sharing a workspace must not overlap
 *   in time.
 * - Inputs must be finite; non-finite values give unspecified routing.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null pointer, bad count, bad flags, non-finite factor */
  MOE_ERR_UNSUPPORTED = -2,  /* shape outside the supported set */
  MOE_ERR_ALIGNMENT = -3,    /* a device pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = -4,    /* workspace missing or smaller than moe_workspace_size */
  MOE_ERR_HIP = -5,          /* a HIP runtime call or kernel launch failed */
  MOE_ERR_HOST = -6          /* a host-side failure (an allocation on the host failed) */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Problem description (the pages' problem statement: X[T,d], W_r[d,E], K,
 * capacity factor, W_gate/W_up[E,d,n], W_down[E,n,d]). */
typedef struct {
  int64_t T;                /* tokens */
  int32_t d;                /* model width */
  int32_t E;                /* experts */
  int32_t K;                /* experts per token (run-time value, "AI芯片..." §4.3) */
  int32_t n;                /* expert FFN width */
  int32_t dtype;            /* moe_dtype of X, weights, H, O, Y */
  double capacity_factor;   /* <= 0: no cap (C = T); else C = min(T, ceil(cf*T*K/E))
                               with cf's exact binary value ("算子与编译器..." §4) */
  uint32_t flags;           /* 0, or MOE_FLAG_TILE_TABLE_READY */
} moe_desc;

/* desc->flags bit for moe_grouped_gemm_up / moe_grouped_gemm_down /
 * moe_grouped_ffn: the workspace already holds the row-tile table that a
 * previous grouped call on the same stream built from the same offsets, so
 * the call skips rebuilding it (e.g. a down-projection issued right after its
 * up-projection).  Other entry points reject the bit. */
#define MOE_FLAG_TILE_TABLE_READY 1u

/* desc->flags bits for moe_grouped_gemm_up / moe_grouped_gemm_down /
 * moe_grouped_ffn / moe_forward (bf16 only; at most one of the two): which
 * grouped-GEMM kernels run.  By default a batch that averages at most 64 rows
 * per expert (T*K <= 64*E, e.g. decode) runs the weight-streaming kernels --
 * one workgroup per expert and column block, reading each active expert's
 * weights once per 64 rows -- and larger batches run the 256x256-tiled
 * kernels, whose launch also computes every expert of at most 64 rows with a
 * weight-streaming block instead of its mostly empty tile (a skewed router
 * leaves many such experts beside a few full ones).  MOE_FLAG_GEMM_TILED
 * runs every expert by tiles; MOE_FLAG_GEMM_SKINNY every expert by weight
 * streaming.  All give results within the documented tolerance of each
 * other (they round the same fp32 sums; summation order differs).  The
 * skinny kernels need no tile table: MOE_FLAG_TILE_TABLE_READY is then
 * ignored. */
#define MOE_FLAG_GEMM_TILED 2u
#define MOE_FLAG_GEMM_SKINNY 4u

/* desc->flags bit for moe_forward: apply tile-aware token rounding
 * (moe_round_tokens) to the metadata between the permutation and the grouped
 * GEMMs.  moe_forward with it gives the same bits as route_ws -> permute ->
 * round_tokens -> grouped_ffn -> combine. */
#define MOE_FLAG_TOKEN_ROUNDING 8u

/* desc->flags bit for moe_route / moe_route_ws / moe_route_permute /
 * moe_forward / moe_forward_train: select the K experts of each token by
 * threshold bisection ("AI芯片如何支持MoE架构" §4.3, threshold-based
 * selection: try a threshold, count the scores above it, move it) instead of
 * the default sort-and-extract selection.  Both are exact: ids, their order
 * and the gates are bit-identical either way; only the kernel's work differs
 * (the bisection runs a fixed number of counting steps whatever K is, the
 * default K extraction rounds). */
#define MOE_FLAG_TOPK_THRESHOLD 16u

/* Workspace selectors for moe_workspace_size.  MOE_WS_SAVED is the state
 * that moe_forward_train keeps for moe_backward (see moe_saved_layout);
 * MOE_WS_BACKWARD is moe_backward's scratch. */
enum {
  MOE_WS_PERMUTE = 0,
  MOE_WS_GROUPED_FFN = 1,
  MOE_WS_FORWARD = 2,
  MOE_WS_ROUTE = 3,
  MOE_WS_SAVED = 4,
  MOE_WS_BACKWARD = 5,
  MOE_WS_ROUND = 6,
  MOE_WS_ROUTE_PERMUTE = 7
};

/* Byte offsets of the fields of the saved state (the `saved` buffer of
 * moe_forward_train / moe_backward), each 256-byte aligned.  Apart from the
 * internal tile table, every field is what the step-wise entry points write. */
typedef struct {
  size_t logits;      /* fp32 [T][E]: the scores the selection was made on */
  size_t topk_ids;    /* int32 [T][K] */
  size_t topk_gates;  /* fp32 [T][K] */
  size_t inv_slot;    /* int32 [T][K] (-1: dropped by the cap) */
  size_t perm_token;  /* int32 [T*K]; the first offsets[E] entries are valid */
  size_t counts;      /* int32 [E] */
  size_t offsets;     /* int32 [E+1] */
  size_t preact;      /* bf16 [moe_max_rows][2n]: row s = (x W_gate[e] | x W_up[e]) of slot s */
  size_t bytes;       /* total = moe_workspace_size(MOE_WS_SAVED) */
} moe_saved_layout;

/* ---------------------------------------------------------------- host only
 * These make no HIP call and can run on a machine without a GPU. */

/* Checks the description (counts, supported shapes, capacity factor, and that
 * flags holds only defined bits, not both GEMM-path bits).  Each device entry
 * point further rejects the bits it does not take.  The host-only queries
 * below ignore the flags.  MOE_ERR_UNSUPPORTED: E > 256, d or n not a
 * positive multiple of 64, T*K >= 2^31, or a grouped-GEMM grid of 2^31 or
 * more workgroups ((T*K/64 + 4E + 4) * ceil(max(d, 2n)/64) bounds it; no
 * problem whose buffers fit in device memory comes near). */
moe_status moe_validate(const moe_desc* desc);

/* Per-expert cap C (see moe_desc.capacity_factor); exact integer arithmetic. */
moe_status moe_capacity(const moe_desc* desc, int64_t* C_out);

/* Upper bound on kept (token, expert) assignments: min(T*K, E*C).  H and O
 * need this many rows. */
moe_status moe_max_rows(const moe_desc* desc, int64_t* rows_out);

/* Bytes of workspace that the entry point `entry` (MOE_WS_*) needs. */
moe_status moe_workspace_size(const moe_desc* desc, int32_t entry, size_t* bytes);

/* Field offsets of the saved state for this description. */
moe_status moe_saved_layout_of(const moe_desc* desc, moe_saved_layout* out);

/* Static description of a status code. */
const char* moe_status_str(moe_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* moe_last_error(void);

/* ---------------------------------------------------------------- device
 * Steps 1-2 (router GEMM, softmax, top-K, renormalised gates; page "MoE 的两个
 * 上游创新：Routing-Free 与 OmniMoE" §1.1 (Router -> Softmax -> TopK) and
 * "AI芯片如何支持MoE架构" §4.2-§4.3 (gating as dense dot products, top-K with
 * a run-time K)).
 *   X[T,d] dtype, W_r[d,E] dtype, bias[E] fp32 or NULL,
 *   logits[T,E] fp32 or NULL (when given, receives the exact scores the
 *   selection was made on), topk_ids[T,K] int32, topk_gates[T,K] fp32.
 * ids[t,:] lists the K largest scores best first; equal scores go to the
 * lower expert id and -0.0 equals +0.0.  gates[t,:] sum to 1. */
moe_status moe_route(const moe_desc* desc, const void* X, const void* W_r, const float* bias,
                     float* logits, int32_t* topk_ids, float* topk_gates, void* stream);

/* moe_route with a workspace (same passages as moe_route; MOE_WS_ROUTE bytes; may be 0, then ws may be
 * NULL).  For batches whose 64-token blocks cannot fill the GPU (bf16, E a
 * multiple of 8) the router's k range is split over several workgroups per
 * block, whose fp32 partial scores go to ws and are summed in a fixed order
 * by a second kernel, then selected as in moe_route.  The scores may differ
 * from moe_route's in the last bits (another summation order); ids and gates
 * always follow the scores this call computed (and exports). */
moe_status moe_route_ws(const moe_desc* desc, const void* X, const void* W_r, const float* bias,
                        float* logits, int32_t* topk_ids, float* topk_gates, void* ws,
                        size_t ws_bytes, void* stream);

/* Steps 3-5 (histogram, capacity cut in token order, exclusive scan, scatter;
 * SonicMoE article §11 (the metadata triple and its counting / prefix-sum /
 * scatter-index steps), "算子与编译器：MoE 路由与稀疏 Kernel" §3-§4
 * (permutation as counting + prefix sums; the capacity factor), OmniMoE page
 * §2.3 (slots ordered by expert, then token)).
 *   topk_ids[T,K] int32 with distinct ids in [0,E) per token (as moe_route writes;
 *   other ids are ignored and marked dropped),
 *   counts[E] kept per expert, offsets[E+1] exclusive scan of counts,
 *   raw_counts[E] before the cut or NULL,
 *   perm_token[T*K]: for slot s < offsets[E], the token of expert-major slot s
 *   (slots ordered by expert, then ascending token); entries past offsets[E]
 *   are left untouched,
 *   inv_slot[T*K]: slot of assignment (t,k), or -1 when the cap dropped it.
 *   ws: MOE_WS_PERMUTE bytes. */
moe_status moe_permute(const moe_desc* desc, const int32_t* topk_ids, int32_t* counts,
                       int32_t* offsets, int32_t* raw_counts, int32_t* perm_token,
                       int32_t* inv_slot, void* ws, size_t ws_bytes, void* stream);

/* Steps 1-5 in two launches ("算子与编译器：MoE 路由与稀疏 Kernel" §3: the
 * counting and prefix sums of the permutation; SonicMoE article §11: the
 * metadata triple): the router of moe_route_ws, whose selection also counts
 * each token block's choices per expert, then one permutation launch that
 * sums the counts of the blocks before each 256-token workgroup and ranks
 * that workgroup's tokens.  Outputs are exactly those of moe_route_ws
 * followed by moe_permute (same arguments; logits and raw_counts may be
 * NULL).  ws: MOE_WS_ROUTE_PERMUTE bytes.  moe_forward runs this path. */
moe_status moe_route_permute(const moe_desc* desc, const void* X, const void* W_r,
                             const float* bias, float* logits, int32_t* topk_ids,
                             float* topk_gates, int32_t* counts, int32_t* offsets,
                             int32_t* raw_counts, int32_t* perm_token, int32_t* inv_slot,
                             void* ws, size_t ws_bytes, void* stream);

/* Allocation-free moe_permute, for callers that cannot allocate device memory
 * or hand in a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments and outputs as moe_permute
 * (bit for bit) without ws/ws_bytes: its scratch (the per-block histogram and
 * block bases, and the raw counts when raw_counts is NULL) lives in a static
 * device array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one copy per
 * GPU, held until the process ends.
 *   Limit: moe_workspace_size(desc, MOE_WS_PERMUTE) must not exceed
 *   MOE_NOALLOC_SCRATCH_BYTES (for example T <= 131072 at E = 256, T <= 262144
 *   at E = 128); a larger problem gets MOE_ERR_WORKSPACE and nothing is
 *   enqueued.
 *   The call never calls hipMalloc/hipFree or any allocating routine; the
 *   first call on a device looks the array's address up once
 *   (hipGetSymbolAddress on the current device; `stream` must belong to it).
 *   Every call on one GPU shares that one array and leaves its contents
 *   behind: calls that overlap in time on the same GPU (other streams, other
 *   threads) race on it and must be serialised by the caller.  Nothing in the
 *   array has to start at zero (every scratch entry is written before it is
 *   read in each call). */
#define MOE_NOALLOC_SCRATCH_BYTES (2u << 20)
moe_status moe_permute_noalloc(const moe_desc* desc, const int32_t* topk_ids, int32_t* counts,
                               int32_t* offsets, int32_t* raw_counts, int32_t* perm_token,
                               int32_t* inv_slot, void* stream);

/* Step 6 (SonicMoE article §3 pipeline steps 3-4, §6.2 gather fused into the
 * operand load, §6.3 SwiGLU in the epilogue):
 * H[s,:] = silu(X[perm_token[s]] W_gate[e]) * (X[perm_token[s]] W_up[e])
 * for every slot s of expert e (rows gathered from X inside the GEMM; no
 * gathered copy of X is made).  offsets/perm_token as moe_permute writes them.
 *   H has moe_max_rows rows of n; ws: MOE_WS_GROUPED_FFN bytes. */
moe_status moe_grouped_gemm_up(const moe_desc* desc, const void* X, const int32_t* offsets,
                               const int32_t* perm_token, const void* W_gate, const void* W_up,
                               void* H, void* ws, size_t ws_bytes, void* stream);

/* Step 7 (SonicMoE article §3 pipeline step 5): O[s,:] = H[s,:] W_down[e] for
 * every slot s of expert e.
 *   O has moe_max_rows rows of d; ws: MOE_WS_GROUPED_FFN bytes. */
moe_status moe_grouped_gemm_down(const moe_desc* desc, const void* H, const int32_t* offsets,
                                 const void* W_down, void* O, void* ws, size_t ws_bytes,
                                 void* stream);

/* Step 5b, tile-aware token rounding (SonicMoE article §6.5: make per-expert
 * counts friendlier to the grouped GEMM's row tiles; the page gives no rule,
 * this is the library's reading).  Updates the metadata that moe_permute
 * wrote, in place: an expert with c >= 256 kept rows and c mod 256 < 128
 * keeps 256*floor(c/256) of them (the tiled GEMM's row tile is 256), dropping
 * its lowest-gate assignments (topk_gates as given; equal gates drop the
 * larger token first); other experts are unchanged.  Dropped assignments
 * get inv_slot = -1 like capacity drops (gates are not renormalised); each
 * expert's surviving slots keep ascending token order; counts and offsets
 * are rewritten; perm_token entries past the new offsets[E] are unspecified.
 *   ws: MOE_WS_ROUND bytes. */
moe_status moe_round_tokens(const moe_desc* desc, const int32_t* topk_ids, const float* topk_gates,
                            int32_t* counts, int32_t* offsets, int32_t* perm_token,
                            int32_t* inv_slot, void* ws, size_t ws_bytes, void* stream);

/* Steps 6-7 in one call (moe_grouped_gemm_up then moe_grouped_gemm_down;
 * SonicMoE article §3). */
moe_status moe_grouped_ffn(const moe_desc* desc, const void* X, const int32_t* offsets,
                           const int32_t* perm_token, const void* W_gate, const void* W_up,
                           const void* W_down, void* H, void* O, void* ws, size_t ws_bytes,
                           void* stream);

/* Step 8 (SonicMoE article §1: y = sum over the selected experts of gate x
 * expert output; §6.1: the aggregation back to token order):
 * Y[t,:] = sum over k with inv_slot[t,k] >= 0, in k order, of
 * topk_gates[t,k] * O[inv_slot[t,k],:], accumulated in fp32; a token whose
 * K assignments were all dropped gets a zero row.  No atomics. */
moe_status moe_combine(const moe_desc* desc, const void* O, const float* topk_gates,
                       const int32_t* inv_slot, void* Y, void* stream);

/* Steps 1-8 in one call (the SonicMoE article §3 GPU pipeline, forward
 * half); every intermediate lives in ws (MOE_WS_FORWARD bytes).
 * Flags: MOE_FLAG_GEMM_TILED / MOE_FLAG_GEMM_SKINNY, MOE_FLAG_TOKEN_ROUNDING. */
moe_status moe_forward(const moe_desc* desc, const void* X, const void* W_r, const float* bias,
                       const void* W_gate, const void* W_up, const void* W_down, void* Y,
                       void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- training (bf16 only)
 * The SonicMoE article (§6.1) keeps, per kept slot, only what the backward
 * cannot cheaply recompute: the routing metadata and the pre-activations
 * x W_gate | x W_up; the SwiGLU activation A and the expert outputs O are
 * never stored for the backward.  Both calls need desc->dtype == MOE_BF16
 * (MOE_ERR_UNSUPPORTED otherwise) and take flags 0 or MOE_FLAG_GEMM_TILED
 * (plus MOE_FLAG_TOPK_THRESHOLD, which only moe_forward_train's router uses):
 * the training path always runs the 256x256-tiled GEMMs. */

/* Forward that also fills `saved` (MOE_WS_SAVED bytes, layout in
 * moe_saved_layout) for moe_backward.  ws: MOE_WS_FORWARD bytes (scratch, not
 * needed afterwards).  Y has the same bits as moe_forward with
 * MOE_FLAG_GEMM_TILED. */
moe_status moe_forward_train(const moe_desc* desc, const void* X, const void* W_r,
                             const float* bias, const void* W_gate, const void* W_up,
                             const void* W_down, void* Y, void* saved, size_t saved_bytes,
                             void* ws, size_t ws_bytes, void* stream);

/* Gradients of sum(Y * dY) for the layer that moe_forward_train ran with the
 * same desc and inputs (X, W_r, W_gate, W_up, W_down unchanged since; `saved`
 * as it wrote it).  SonicMoE article §6.4 ordering: per kept slot s of
 * expert e (token t, gate g):
 *   dA'[s] = dY[t] W_down[e]^T; dS[s] = <dA'[s], A[s]> with A = silu(Hg) Hu
 *   recomputed from the saved pre-activations (no O or Y is formed);
 *   dHg = g dA' Hu silu'(Hg), dHu = g dA' silu(Hg) in the GEMM's epilogue (§6.3);
 *   dW_down[e] = sum_s (g A[s])^T dY[t];  dW_gate[e] | dW_up[e] = sum_s X[t]^T (dHg | dHu);
 *   router: dg[t,k] = dS[slot] (0 when dropped), dl = softmax-over-the-K Jacobian
 *   applied to dg (the selection itself has no gradient), dW_r = X^T dl;
 *   dX[t] = sum over kept k of (dHg W_gate^T + dHu W_up^T)[slot] + dl[t] W_r^T.
 *   dY[T,d], dX[T,d] bf16; dW_r[d,E], dW_gate/dW_up[E,d,n], dW_down[E,n,d] fp32
 *   (every element written; bias gets no gradient).  Intermediates (dH, g A,
 *   per-slot dX, dl) are rounded to bf16, sums run in fp32 in a fixed order,
 *   so identical inputs give identical bits.  ws: MOE_WS_BACKWARD bytes.
 *   T = 0 writes zero weight gradients. */
moe_status moe_backward(const moe_desc* desc, const void* X, const void* W_r, const void* W_gate,
                        const void* W_up, const void* W_down, const void* dY, const void* saved,
                        size_t saved_bytes, void* dX, float* dW_r, float* dW_gate, float* dW_up,
                        float* dW_down, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- atomic experts
 * A second layer type (page "MoE 的两个上游创新：Routing-Free 与 OmniMoE",
 * part 2): N = Nr*Nc experts, each two d-vectors, E_i(x) = silu(x . w_in_i)
 * w_out_i (§2.1; sigma taken as SiLU, the routing weight playing SwiGLU's
 * gating role), chosen by a Cartesian-product router (§2.2) and executed
 * expert by expert in (expert, token) order (§2.3).  bf16 only.
 *   X[T,d], W_r[d,Nr], W_c[d,Nc], W_in/W_out[N,d] (row i = expert i), Y[T,d].
 * Expert id i = i_r*Nc + i_c; score S = ls_r[i_r] + ls_c[i_c] with ls the
 * fp32 log-softmax of x W over each axis; the K largest S by (S desc, id
 * asc); gates = softmax over the K selected S.  The search keeps the top
 * min(K, Nr) rows and min(K, Nc) columns and then only pairs whose axis
 * ranks satisfy (i+1)(j+1) <= K, a pruning that returns the full search's
 * result.  No capacity: every task is kept.
 * Supported: 1 <= Nr, Nc <= 256, 1 <= K <= min(64, Nr*Nc), d a multiple of
 * 64 up to 4096, T*K < 2^31, dtype MOE_BF16, flags 0. */
typedef struct {
  int64_t T;
  int32_t d, Nr, Nc, K;
  int32_t dtype;            /* must be MOE_BF16 */
  uint32_t flags;           /* must be 0 */
} moe_omni_desc;

enum { MOE_OMNI_WS_ROUTE = 0, MOE_OMNI_WS_PERMUTE = 1, MOE_OMNI_WS_FORWARD = 2 };

/* Host only: checks the description; bytes of workspace for an entry point. */
moe_status moe_omni_validate(const moe_omni_desc* desc);
moe_status moe_omni_workspace_size(const moe_omni_desc* desc, int32_t entry, size_t* bytes);

/* Router: ids[T,K] int32 (best first), gates[T,K] fp32; ls_r[T,Nr] and
 * ls_c[T,Nc] (fp32 log-softmax rows the selection used) or NULL.
 * ws: MOE_OMNI_WS_ROUTE bytes. */
moe_status moe_omni_route(const moe_omni_desc* desc, const void* X, const void* W_r,
                          const void* W_c, float* ls_r, float* ls_c, int32_t* ids, float* gates,
                          void* ws, size_t ws_bytes, void* stream);

/* (expert, token) order over the N experts: counts[N], offsets[N+1],
 * perm_token[T*K] (slot -> token, ascending tokens inside an expert),
 * inv_slot[T,K] (entry -> slot).  ws: MOE_OMNI_WS_PERMUTE bytes. */
moe_status moe_omni_permute(const moe_omni_desc* desc, const int32_t* ids, int32_t* counts,
                            int32_t* offsets, int32_t* perm_token, int32_t* inv_slot, void* ws,
                            size_t ws_bytes, void* stream);

/* The whole layer: Y[t] = sum over k of g[t,k] silu(X[t] . w_in[id]) w_out[id]
 * (fp32 in k order, rounded to bf16).  ws: MOE_OMNI_WS_FORWARD bytes. */
moe_status moe_omni_forward(const moe_omni_desc* desc, const void* X, const void* W_r,
                            const void* W_c, const void* W_in, const void* W_out, void* Y,
                            void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
