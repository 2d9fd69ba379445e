// C ABI of the MI355X MoE layer library (declared in include/moe.h).
//
// Host side only: argument checks, the capacity rule, workspace carving and
// the launch order.  Every entry point enqueues on the caller's stream and
// returns without synchronising; nothing here allocates device memory.
#include "moe.h"

#include <cmath>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <string>

#include "moe_internal.hpp"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

// An exception that reached an entry point (a host allocation failed): it is
// not let across the C ABI; the message is set without allocating when possible.
moe_status caught() noexcept {
  try {
    g_last_error = "host-side failure (an allocation on the host failed)";
  } catch (...) {
  }
  return MOE_ERR_HOST;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Exact C = min(T, ceil(cf * T * K / E)) for cf > 0, with cf taken as the
// exact binary value of the double: cf = m * 2^ex, m a 53-bit integer.
int64_t exact_capacity(int64_t T, int64_t K, int64_t E, double cf) {
  if (!(cf > 0.0)) return T;
  if (T == 0) return 0;
  int ex = 0;
  const double f = std::frexp(cf, &ex);            // cf = f * 2^ex, f in [0.5, 1)
  const int64_t m = (int64_t)std::ldexp(f, 53);    // exact
  ex -= 53;                                        // cf = m * 2^ex
  if (ex >= 0) return T;                           // cf >= 2^52: above any cap
  if (-ex > 100) return 1;                         // 0 < cf*T*K/E < 1
  const __int128 num = (__int128)m * T * K;
  const __int128 den = (__int128)E << (-ex);
  const __int128 c = (num + den - 1) / den;
  return c < (__int128)T ? (int64_t)c : T;
}

moe_status check_desc(const moe_desc* d, uint32_t allowed_flags = 0) {
  if (!d) return fail(MOE_ERR_INVALID_ARG, "desc is NULL");
  if (d->flags & ~allowed_flags) return fail(MOE_ERR_INVALID_ARG, "desc->flags has a bit this entry point does not accept");
  if ((d->flags & MOE_FLAG_GEMM_TILED) && (d->flags & MOE_FLAG_GEMM_SKINNY))
    return fail(MOE_ERR_INVALID_ARG, "MOE_FLAG_GEMM_TILED and MOE_FLAG_GEMM_SKINNY are exclusive");
  if (d->T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0");
  if (d->E < 1) return fail(MOE_ERR_INVALID_ARG, "E must be >= 1");
  if (d->K < 1 || d->K > d->E) return fail(MOE_ERR_INVALID_ARG, "K must satisfy 1 <= K <= E");
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "dtype must be MOE_F32 or MOE_BF16");
  if (!std::isfinite(d->capacity_factor))
    return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be finite");
  if (d->E > 256) return fail(MOE_ERR_UNSUPPORTED, "E above 256 is not supported");
  if (d->d < 64 || d->d % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "d must be a positive multiple of 64");
  if (d->n < 64 || d->n % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "n must be a positive multiple of 64");
  // T*K < 2^31, tested by division so that no product can overflow
  if (d->T > (((int64_t)1 << 31) - 1) / d->K)
    return fail(MOE_ERR_UNSUPPORTED, "T*K must stay below 2^31 (int32 slots)");
  // every grouped-GEMM grid (forward and backward, at most one workgroup per
  // 64 rows plus four per expert, times one per 64 columns of the widest
  // operand) must fit the kernels' 32-bit tile numbering; a problem whose
  // buffers fit in device memory is far below this
  const int64_t row_blocks = d->T * (int64_t)d->K / 64 + 4 * (int64_t)d->E + 4;
  const int64_t widest = d->d > 2 * (int64_t)d->n ? d->d : 2 * (int64_t)d->n;
  if (row_blocks * ((widest + 63) / 64) >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "problem too large for one grouped-GEMM launch");
  return MOE_OK;
}

constexpr uint32_t kGemmFlags = MOE_FLAG_TILE_TABLE_READY | MOE_FLAG_GEMM_TILED | MOE_FLAG_GEMM_SKINNY;
// every defined bit (host-only queries accept them all)
constexpr uint32_t kAllFlags = kGemmFlags | MOE_FLAG_TOKEN_ROUNDING | MOE_FLAG_TOPK_THRESHOLD;

bool skinny(const moe::Problem& p, const moe_desc* d) {
  return moe::use_skinny(p, d->flags, MOE_FLAG_GEMM_TILED, MOE_FLAG_GEMM_SKINNY);
}

// Rows up to which an expert of a tiled bf16 launch is computed by a
// weight-streaming block instead of its tile (0: every expert by tiles, as
// MOE_FLAG_GEMM_TILED asks).
int stream_rows(const moe::Problem& p, const moe_desc* d) {
  return (p.bf16 && !(d->flags & MOE_FLAG_GEMM_TILED)) ? moe::kMaxStreamRows : 0;
}

moe::Problem make_problem(const moe_desc* d) {
  moe::Problem p;
  p.T = d->T;
  p.d = d->d;
  p.E = d->E;
  p.K = d->K;
  p.n = d->n;
  p.bf16 = d->dtype == MOE_BF16;
  p.C = exact_capacity(d->T, d->K, d->E, d->capacity_factor);
  const int64_t tk = d->T * (int64_t)d->K;
  const int64_t ec = (int64_t)d->E * p.C;
  p.rows_max = tk < ec ? tk : ec;
  p.sel = (d->flags & MOE_FLAG_TOPK_THRESHOLD) ? 1 : 0;
  return p;
}

size_t elem(const moe::Problem& p) { return p.bf16 ? 2 : 4; }

struct PermuteWs {
  int32_t* blockcnt;
  int32_t* blockbase;
  int32_t* raw;
};
size_t permute_ws_bytes(const moe::Problem& p) {
  const size_t nbe = (size_t)moe::permute_blocks(p.T) * p.E * sizeof(int32_t);
  return align_up(nbe) * 2 + align_up((size_t)p.E * sizeof(int32_t));
}
PermuteWs carve_permute(const moe::Problem& p, unsigned char* base) {
  const size_t nbe = align_up((size_t)moe::permute_blocks(p.T) * p.E * sizeof(int32_t));
  return {reinterpret_cast<int32_t*>(base), reinterpret_cast<int32_t*>(base + nbe),
          reinterpret_cast<int32_t*>(base + 2 * nbe)};
}

// Workspace of moe_route_permute: split-k partial scores (or none), the
// per-block expert counts, raw counts.
struct RoutePermuteWs {
  float* route_partial;
  int32_t* blockcnt;
  int32_t* raw;
  size_t bytes;
};
RoutePermuteWs carve_route_permute(const moe::Problem& p, unsigned char* base) {
  RoutePermuteWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* ptr = base ? base + off : nullptr;
    off += align_up(bytes);
    return ptr;
  };
  const size_t rp = moe::route_partial_bytes(p);
  w.route_partial = rp ? reinterpret_cast<float*>(take(rp)) : nullptr;
  w.blockcnt = reinterpret_cast<int32_t*>(take(moe::route_count_bytes(p, true)));
  w.raw = reinterpret_cast<int32_t*>(take((size_t)p.E * 4));
  w.bytes = off;
  return w;
}

struct ForwardWs {
  float* route_partial;
  int32_t* ids;
  float* gates;
  int32_t* inv;
  int32_t* perm;
  int32_t* counts;
  int32_t* offsets;
  int32_t* raw;
  int32_t* blockcnt;
  int32_t* table;
  void* H;
  void* O;
  unsigned char* round;
  size_t bytes;
};
ForwardWs carve_forward(const moe::Problem& p, unsigned char* base) {
  ForwardWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* ptr = base ? base + off : nullptr;
    off += align_up(bytes);
    return ptr;
  };
  const size_t tk = (size_t)p.T * p.K;
  const size_t rp = moe::route_partial_bytes(p);
  w.route_partial = rp ? reinterpret_cast<float*>(take(rp)) : nullptr;
  w.ids = reinterpret_cast<int32_t*>(take(tk * 4));
  w.gates = reinterpret_cast<float*>(take(tk * 4));
  w.inv = reinterpret_cast<int32_t*>(take(tk * 4));
  w.perm = reinterpret_cast<int32_t*>(take(tk * 4));
  w.counts = reinterpret_cast<int32_t*>(take((size_t)p.E * 4));
  w.offsets = reinterpret_cast<int32_t*>(take((size_t)(p.E + 1) * 4));
  w.raw = reinterpret_cast<int32_t*>(take((size_t)p.E * 4));
  w.blockcnt = reinterpret_cast<int32_t*>(take(moe::route_count_bytes(p, true)));
  w.table = reinterpret_cast<int32_t*>(take(moe::tile_table_bytes(p)));
  w.H = take((size_t)p.rows_max * p.n * elem(p));
  w.O = take((size_t)p.rows_max * p.d * elem(p));
  w.round = take(moe::round_ws_bytes(p, nullptr, nullptr));
  w.bytes = off;
  return w;
}

// State kept by moe_forward_train for moe_backward (field order as in
// moe_saved_layout, plus the row-tile table at the end).
struct Saved {
  float* logits;
  int32_t* ids;
  float* gates;
  int32_t* inv;
  int32_t* perm;
  int32_t* counts;
  int32_t* offsets;
  uint16_t* Hpre;
  int32_t* table;
  moe_saved_layout layout;
};
Saved carve_saved(const moe::Problem& p, unsigned char* base) {
  Saved w{};
  size_t off = 0;
  auto take = [&](size_t bytes, size_t* field) {
    if (field) *field = off;
    unsigned char* ptr = base ? base + off : nullptr;
    off += align_up(bytes);
    return ptr;
  };
  const size_t tk = (size_t)p.T * p.K;
  moe_saved_layout& L = w.layout;
  w.logits = reinterpret_cast<float*>(take((size_t)p.T * p.E * 4, &L.logits));
  w.ids = reinterpret_cast<int32_t*>(take(tk * 4, &L.topk_ids));
  w.gates = reinterpret_cast<float*>(take(tk * 4, &L.topk_gates));
  w.inv = reinterpret_cast<int32_t*>(take(tk * 4, &L.inv_slot));
  w.perm = reinterpret_cast<int32_t*>(take(tk * 4, &L.perm_token));
  w.counts = reinterpret_cast<int32_t*>(take((size_t)p.E * 4, &L.counts));
  w.offsets = reinterpret_cast<int32_t*>(take((size_t)(p.E + 1) * 4, &L.offsets));
  w.Hpre = reinterpret_cast<uint16_t*>(take((size_t)p.rows_max * 2 * p.n * 2, &L.preact));
  w.table = reinterpret_cast<int32_t*>(take(moe::tile_table_bytes(p), nullptr));
  L.bytes = off;
  return w;
}

bool misaligned(const void* ptr) { return ((uintptr_t)ptr & 15u) != 0; }

moe_status check_ptrs(std::initializer_list<std::pair<const void*, const char*>> required,
                      std::initializer_list<std::pair<const void*, const char*>> optional) {
  for (auto& pr : required) {
    if (!pr.first) return fail(MOE_ERR_INVALID_ARG, std::string(pr.second) + " is NULL");
    if (misaligned(pr.first))
      return fail(MOE_ERR_ALIGNMENT, std::string(pr.second) + " is not 16-byte aligned");
  }
  for (auto& pr : optional)
    if (pr.first && misaligned(pr.first))
      return fail(MOE_ERR_ALIGNMENT, std::string(pr.second) + " is not 16-byte aligned");
  return MOE_OK;
}

// MOE_DEBUG_SYNC=1 in the environment (read at every step): each launch
// step synchronises the entry point's stream and reports a kernel that
// failed as MOE_ERR_HIP naming that step, instead of leaving the error to
// the caller's next synchronisation.  Debug only; a stream that is being
// captured into a graph is not synchronised.
thread_local hipStream_t g_stream = nullptr;
thread_local bool g_in_call = false;

struct StreamScope {   // the entry point's stream, for the debug synchronisation
  hipStream_t prev;
  bool prev_in;
  explicit StreamScope(void* s) : prev(g_stream), prev_in(g_in_call) {
    g_stream = (hipStream_t)s;
    g_in_call = true;
  }
  ~StreamScope() {
    g_stream = prev;
    g_in_call = prev_in;
  }
};

bool debug_sync() {
  const char* v = std::getenv("MOE_DEBUG_SYNC");
  return v != nullptr && std::strcmp(v, "1") == 0;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess && g_in_call && debug_sync()) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(g_stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone)
      e = hipStreamSynchronize(g_stream);
  }
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define MOE_TRY(expr)                 \
  do {                                \
    const moe_status st_ = (expr);    \
    if (st_ != MOE_OK) return st_;    \
  } while (0)

// The step sequences shared by the step-wise entry points and moe_forward.
moe_status run_permute(const moe::Problem& p, const int32_t* ids, int32_t* counts,
                       int32_t* offsets, int32_t* raw, int32_t* perm, int32_t* inv,
                       unsigned char* ws, int32_t* table, hipStream_t s) {
  PermuteWs w = carve_permute(p, ws);
  if (moe::permute_blocks(p.T) == 1)
    return hip_status(moe::launch_permute_one_block(p, ids, raw ? raw : w.raw, counts, offsets,
                                                    table, perm, inv, s),
                      "permutation launch");
  MOE_TRY(hip_status(moe::launch_histogram(p, ids, w.blockcnt, s), "histogram launch"));
  MOE_TRY(hip_status(moe::launch_scan(p, w.blockcnt, w.blockbase, raw ? raw : w.raw, counts,
                                      offsets, table, s),
                     "scan launch"));
  return hip_status(moe::launch_scatter(p, ids, w.blockbase, offsets, perm, inv, s),
                    "scatter launch");
}

// Steps 1-5 of moe_forward / moe_forward_train: the router, which also
// writes per-block expert counts, then the fused permutation (one launch).
moe_status run_route_permute(const moe::Problem& p, const void* X, const void* W_r,
                             const float* bias, float* logits, int32_t* ids, float* gates,
                             float* partial, int32_t* blockcnt, int32_t* counts, int32_t* offsets,
                             int32_t* raw, int32_t* perm, int32_t* inv, int32_t* table,
                             hipStream_t s) {
  const bool split = partial != nullptr;
  if (moe::permute_blocks(p.T) == 1) {
    // one token block (decode-sized): the one-workgroup permutation counts
    // for itself, so the router writes no per-block counts (5.7 instead of
    // 14.6 us for the permutation at T = 64)
    MOE_TRY(hip_status(moe::launch_route(p, X, W_r, bias, logits, ids, gates, partial, s),
                       "route launch"));
    return hip_status(moe::launch_permute_one_block(p, ids, raw, counts, offsets, table, perm, inv,
                                                    s),
                      "permutation launch");
  }
  MOE_TRY(hip_status(moe::launch_route(p, X, W_r, bias, logits, ids, gates, partial, s, blockcnt),
                     "route launch"));
  return hip_status(moe::launch_permute_fused(p, ids, blockcnt, moe::route_count_block(p, split),
                                              moe::route_count_ld(p, split), raw, counts, offsets,
                                              table, perm, inv, s),
                    "permutation launch");
}

moe_status check_omni(const moe_omni_desc* d) {
  if (!d) return fail(MOE_ERR_INVALID_ARG, "desc is NULL");
  if (d->flags != 0) return fail(MOE_ERR_INVALID_ARG, "desc->flags must be 0");
  if (d->T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0");
  if (d->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the atomic-expert layer is bf16 only");
  if (d->Nr < 1 || d->Nc < 1) return fail(MOE_ERR_INVALID_ARG, "Nr and Nc must be >= 1");
  if (d->Nr > 256 || d->Nc > 256) return fail(MOE_ERR_UNSUPPORTED, "Nr and Nc above 256 are not supported");
  if (d->K < 1 || (int64_t)d->K > (int64_t)d->Nr * d->Nc)
    return fail(MOE_ERR_INVALID_ARG, "K must satisfy 1 <= K <= Nr*Nc");
  if (d->K > 64) return fail(MOE_ERR_UNSUPPORTED, "K above 64 is not supported");
  if (d->d < 64 || d->d % 64 != 0 || d->d > 4096)
    return fail(MOE_ERR_UNSUPPORTED, "d must be a multiple of 64 up to 4096");
  // T*K < 2^31, tested by division so that no product can overflow
  if (d->T > (((int64_t)1 << 31) - 1) / d->K)
    return fail(MOE_ERR_UNSUPPORTED, "T*K must stay below 2^31 (int32 slots)");
  return MOE_OK;
}

moe::OmniProblem omni_problem(const moe_omni_desc* d) {
  moe::OmniProblem p;
  p.T = d->T;
  p.d = d->d;
  p.Nr = d->Nr;
  p.Nc = d->Nc;
  p.K = d->K;
  return p;
}

struct OmniForwardWs {
  unsigned char* route;
  int32_t* ids;
  float* gates;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  unsigned char* permute;
  float* a;
  size_t bytes;
};
OmniForwardWs carve_omni_forward(const moe::OmniProblem& p, unsigned char* base) {
  OmniForwardWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* ptr = base ? base + off : nullptr;
    off += align_up(bytes);
    return ptr;
  };
  const size_t tk = (size_t)p.T * p.K, N = (size_t)p.Nr * p.Nc;
  w.route = take(moe::omni_route_ws_bytes(p, nullptr, nullptr));
  w.ids = reinterpret_cast<int32_t*>(take(tk * 4));
  w.gates = reinterpret_cast<float*>(take(tk * 4));
  w.counts = reinterpret_cast<int32_t*>(take(N * 4));
  w.offsets = reinterpret_cast<int32_t*>(take((N + 1) * 4));
  w.perm = reinterpret_cast<int32_t*>(take(tk * 4));
  w.inv = reinterpret_cast<int32_t*>(take(tk * 4));
  w.permute = take(moe::omni_permute_ws_bytes(p, nullptr, nullptr));
  w.a = reinterpret_cast<float*>(take(tk * 4));
  w.bytes = off;
  return w;
}

}  // namespace

extern "C" {

moe_status moe_omni_validate(const moe_omni_desc* desc) try {
  g_last_error.clear();
  return check_omni(desc);
} catch (...) {
  return caught();
}

moe_status moe_omni_workspace_size(const moe_omni_desc* desc, int32_t entry, size_t* bytes) try {
  MOE_TRY(check_omni(desc));
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  const moe::OmniProblem p = omni_problem(desc);
  switch (entry) {
    case MOE_OMNI_WS_ROUTE: *bytes = moe::omni_route_ws_bytes(p, nullptr, nullptr); return MOE_OK;
    case MOE_OMNI_WS_PERMUTE: *bytes = moe::omni_permute_ws_bytes(p, nullptr, nullptr); return MOE_OK;
    case MOE_OMNI_WS_FORWARD: *bytes = carve_omni_forward(p, nullptr).bytes; return MOE_OK;
    default: return fail(MOE_ERR_INVALID_ARG, "unknown workspace selector");
  }
} catch (...) {
  return caught();
}

moe_status moe_omni_route(const moe_omni_desc* desc, const void* X, const void* W_r,
                          const void* W_c, float* ls_r, float* ls_c, int32_t* ids, float* gates,
                          void* ws, size_t ws_bytes, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_omni(desc));
  if (desc->T == 0) return MOE_OK;
  MOE_TRY(check_ptrs({{X, "X"}, {W_r, "W_r"}, {W_c, "W_c"}, {ids, "ids"}, {gates, "gates"},
                      {ws, "ws"}},
                     {{ls_r, "ls_r"}, {ls_c, "ls_c"}}));
  const moe::OmniProblem p = omni_problem(desc);
  if (ws_bytes < moe::omni_route_ws_bytes(p, nullptr, nullptr))
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_omni_workspace_size(MOE_OMNI_WS_ROUTE)");
  moe::OmniRouteWs w;
  moe::omni_route_ws_bytes(p, &w, static_cast<unsigned char*>(ws));
  return hip_status(moe::launch_omni_route(p, X, W_r, W_c, ls_r, ls_c, ids, gates, w,
                                           (hipStream_t)stream),
                    "atomic-expert router launch");
} catch (...) {
  return caught();
}

moe_status moe_omni_permute(const moe_omni_desc* desc, const int32_t* ids, int32_t* counts,
                            int32_t* offsets, int32_t* perm_token, int32_t* inv_slot, void* ws,
                            size_t ws_bytes, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_omni(desc));
  if (desc->T == 0) return MOE_OK;
  MOE_TRY(check_ptrs({{ids, "ids"}, {counts, "counts"}, {offsets, "offsets"},
                      {perm_token, "perm_token"}, {inv_slot, "inv_slot"}, {ws, "ws"}},
                     {}));
  const moe::OmniProblem p = omni_problem(desc);
  if (ws_bytes < moe::omni_permute_ws_bytes(p, nullptr, nullptr))
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_omni_workspace_size(MOE_OMNI_WS_PERMUTE)");
  moe::OmniPermuteWs w;
  moe::omni_permute_ws_bytes(p, &w, static_cast<unsigned char*>(ws));
  return hip_status(moe::launch_omni_permute(p, ids, counts, offsets, perm_token, inv_slot, w,
                                             (hipStream_t)stream),
                    "atomic-expert permutation launch");
} catch (...) {
  return caught();
}

moe_status moe_omni_forward(const moe_omni_desc* desc, const void* X, const void* W_r,
                            const void* W_c, const void* W_in, const void* W_out, void* Y,
                            void* ws, size_t ws_bytes, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_omni(desc));
  if (desc->T == 0) return MOE_OK;
  MOE_TRY(check_ptrs({{X, "X"}, {W_r, "W_r"}, {W_c, "W_c"}, {W_in, "W_in"}, {W_out, "W_out"},
                      {Y, "Y"}, {ws, "ws"}},
                     {}));
  const moe::OmniProblem p = omni_problem(desc);
  if (ws_bytes < carve_omni_forward(p, nullptr).bytes)
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_omni_workspace_size(MOE_OMNI_WS_FORWARD)");
  const OmniForwardWs w = carve_omni_forward(p, static_cast<unsigned char*>(ws));
  hipStream_t s = (hipStream_t)stream;
  moe::OmniRouteWs rw;
  moe::omni_route_ws_bytes(p, &rw, w.route);
  // the selection counts the entries per expert, so the permutation does
  // not, and records each entry's place in its expert's arrival order in the
  // buffer of the expert activations a (written only after the permutation)
  int32_t* tpos = reinterpret_cast<int32_t*>(w.a);
  MOE_TRY(hip_status(moe::launch_omni_route(p, X, W_r, W_c, nullptr, nullptr, w.ids, w.gates, rw, s,
                                            w.counts, tpos),
                     "atomic-expert router launch"));
  moe::OmniPermuteWs pw;
  moe::omni_permute_ws_bytes(p, &pw, w.permute);
  MOE_TRY(hip_status(moe::launch_omni_permute(p, w.ids, w.counts, w.offsets, w.perm, w.inv, pw, s,
                                              true, tpos),
                     "atomic-expert permutation launch"));
  return hip_status(moe::launch_omni_experts(p, X, W_in, W_out, w.ids, w.gates, w.offsets, w.perm,
                                             w.inv, w.a, Y, s),
                    "atomic-expert launch");
} catch (...) {
  return caught();
}


moe_status moe_validate(const moe_desc* desc) try {
  g_last_error.clear();
  return check_desc(desc, kAllFlags);
} catch (...) {
  return caught();
}

moe_status moe_capacity(const moe_desc* desc, int64_t* C_out) try {
  MOE_TRY(check_desc(desc, kAllFlags));
  if (!C_out) return fail(MOE_ERR_INVALID_ARG, "C_out is NULL");
  *C_out = make_problem(desc).C;
  return MOE_OK;
} catch (...) {
  return caught();
}

moe_status moe_max_rows(const moe_desc* desc, int64_t* rows_out) try {
  MOE_TRY(check_desc(desc, kAllFlags));
  if (!rows_out) return fail(MOE_ERR_INVALID_ARG, "rows_out is NULL");
  *rows_out = make_problem(desc).rows_max;
  return MOE_OK;
} catch (...) {
  return caught();
}

moe_status moe_workspace_size(const moe_desc* desc, int32_t entry, size_t* bytes) try {
  MOE_TRY(check_desc(desc, kAllFlags));
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  const moe::Problem p = make_problem(desc);
  switch (entry) {
    case MOE_WS_PERMUTE:
      *bytes = permute_ws_bytes(p);
      return MOE_OK;
    case MOE_WS_GROUPED_FFN:
      *bytes = align_up(moe::tile_table_bytes(p));
      return MOE_OK;
    case MOE_WS_FORWARD:
      *bytes = carve_forward(p, nullptr).bytes;
      return MOE_OK;
    case MOE_WS_ROUTE:
      *bytes = align_up(moe::route_partial_bytes(p));
      return MOE_OK;
    case MOE_WS_SAVED:
      *bytes = carve_saved(p, nullptr).layout.bytes;
      return MOE_OK;
    case MOE_WS_BACKWARD:
      *bytes = moe::backward_ws_bytes(p, nullptr, nullptr);
      return MOE_OK;
    case MOE_WS_ROUND:
      *bytes = moe::round_ws_bytes(p, nullptr, nullptr);
      return MOE_OK;
    case MOE_WS_ROUTE_PERMUTE:
      *bytes = carve_route_permute(p, nullptr).bytes;
      return MOE_OK;
    default:
      return fail(MOE_ERR_INVALID_ARG, "unknown workspace selector");
  }
} catch (...) {
  return caught();
}

moe_status moe_saved_layout_of(const moe_desc* desc, moe_saved_layout* out) try {
  MOE_TRY(check_desc(desc, kAllFlags));
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  *out = carve_saved(make_problem(desc), nullptr).layout;
  return MOE_OK;
} catch (...) {
  return caught();
}

const char* moe_status_str(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_ALIGNMENT: return "MOE_ERR_ALIGNMENT";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_HOST: return "MOE_ERR_HOST";
    default: return "unknown moe_status";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_route(const moe_desc* desc, const void* X, const void* W_r, const float* bias,
                     float* logits, int32_t* topk_ids, float* topk_gates, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_desc(desc, MOE_FLAG_TOPK_THRESHOLD));
  if (desc->T == 0) return MOE_OK;  // no-op; empty tensors may carry NULL
  MOE_TRY(check_ptrs({{X, "X"}, {W_r, "W_r"}, {topk_ids, "topk_ids"}, {topk_gates, "topk_gates"}},
                     {{bias, "bias"}, {logits, "logits"}}));
  const moe::Problem p = make_problem(desc);
  return hip_status(moe::launch_route(p, X, W_r, bias, logits, topk_ids, topk_gates, nullptr,
                                      (hipStream_t)stream),
                    "route launch");
} catch (...) {
  return caught();
}

moe_status moe_route_ws(const moe_desc* desc, const void* X, const void* W_r, const float* bias,
                        float* logits, int32_t* topk_ids, float* topk_gates, void* ws,
                        size_t ws_bytes, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_desc(desc, MOE_FLAG_TOPK_THRESHOLD));
  if (desc->T == 0) return MOE_OK;  // no-op; empty tensors may carry NULL
  MOE_TRY(check_ptrs({{X, "X"}, {W_r, "W_r"}, {topk_ids, "topk_ids"}, {topk_gates, "topk_gates"}},
                     {{bias, "bias"}, {logits, "logits"}, {ws, "ws"}}));
  const moe::Problem p = make_problem(desc);
  const size_t need = moe::route_partial_bytes(p);
  if (need && (!ws || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size(MOE_WS_ROUTE)");
  return hip_status(moe::launch_route(p, X, W_r, bias, logits, topk_ids, topk_gates,
                                      need ? static_cast<float*>(ws) : nullptr,
                                      (hipStream_t)stream),
                    "route launch");
} catch (...) {
  return caught();
}

moe_status moe_permute(const moe_desc* desc, const int32_t* topk_ids, int32_t* counts,
                       int32_t* offsets, int32_t* raw_counts, int32_t* perm_token,
                       int32_t* inv_slot, void* ws, size_t ws_bytes, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_desc(desc));
  if (desc->T == 0) return MOE_OK;  // no-op; empty tensors may carry NULL
  MOE_TRY(check_ptrs({{topk_ids, "topk_ids"}, {counts, "counts"}, {offsets, "offsets"},
                      {perm_token, "perm_token"}, {inv_slot, "inv_slot"}},
                     {{raw_counts, "raw_counts"}, {ws, "ws"}}));
  const moe::Problem p = make_problem(desc);
  if (!ws || ws_bytes < permute_ws_bytes(p))
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size(MOE_WS_PERMUTE)");
  return run_permute(p, topk_ids, counts, offsets, raw_counts, perm_token, inv_slot,
                     static_cast<unsigned char*>(ws), nullptr, (hipStream_t)stream);
} catch (...) {
  return caught();
}

moe_status moe_route_permute(const moe_desc* desc, const void* X, const void* W_r,
                             const float* bias, float* logits, int32_t* topk_ids,
                             float* topk_gates, int32_t* counts, int32_t* offsets,
                             int32_t* raw_counts, int32_t* perm_token, int32_t* inv_slot,
                             void* ws, size_t ws_bytes, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_desc(desc, MOE_FLAG_TOPK_THRESHOLD));
  if (desc->T == 0) return MOE_OK;  // no-op; empty tensors may carry NULL
  MOE_TRY(check_ptrs({{X, "X"}, {W_r, "W_r"}, {topk_ids, "topk_ids"}, {topk_gates, "topk_gates"},
                      {counts, "counts"}, {offsets, "offsets"}, {perm_token, "perm_token"},
                      {inv_slot, "inv_slot"}, {ws, "ws"}},
                     {{bias, "bias"}, {logits, "logits"}, {raw_counts, "raw_counts"}}));
  const moe::Problem p = make_problem(desc);
  if (ws_bytes < carve_route_permute(p, nullptr).bytes)
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size(MOE_WS_ROUTE_PERMUTE)");
  const RoutePermuteWs w = carve_route_permute(p, static_cast<unsigned char*>(ws));
  return run_route_permute(p, X, W_r, bias, logits, topk_ids, topk_gates, w.route_partial,
                           w.blockcnt, counts, offsets, raw_counts ? raw_counts : w.raw,
                           perm_token, inv_slot, nullptr, (hipStream_t)stream);
} catch (...) {
  return caught();
}

static_assert(moe::kNoallocScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "scratch size in moe.h");

moe_status moe_permute_noalloc(const moe_desc* desc, const int32_t* topk_ids, int32_t* counts,
                               int32_t* offsets, int32_t* raw_counts, int32_t* perm_token,
                               int32_t* inv_slot, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_desc(desc));
  if (desc->T == 0) return MOE_OK;  // no-op; empty tensors may carry NULL
  MOE_TRY(check_ptrs({{topk_ids, "topk_ids"}, {counts, "counts"}, {offsets, "offsets"},
                      {perm_token, "perm_token"}, {inv_slot, "inv_slot"}},
                     {{raw_counts, "raw_counts"}}));
  const moe::Problem p = make_problem(desc);
  if (permute_ws_bytes(p) > moe::kNoallocScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "moe_permute_noalloc: the permutation needs " + std::to_string(permute_ws_bytes(p)) +
                    " bytes of scratch, above the static MOE_NOALLOC_SCRATCH_BYTES (" +
                    std::to_string(moe::kNoallocScratchBytes) + "); use moe_permute with a workspace");
  void* scratch = nullptr;
  MOE_TRY(hip_status(moe::noalloc_scratch(&scratch), "static scratch address"));
  return run_permute(p, topk_ids, counts, offsets, raw_counts, perm_token, inv_slot,
                     static_cast<unsigned char*>(scratch), nullptr, (hipStream_t)stream);
} catch (...) {
  return caught();
}

moe_status moe_round_tokens(const moe_desc* desc, const int32_t* topk_ids, const float* topk_gates,
                            int32_t* counts, int32_t* offsets, int32_t* perm_token,
                            int32_t* inv_slot, void* ws, size_t ws_bytes, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_desc(desc));
  if (desc->T == 0) return MOE_OK;  // no-op; empty tensors may carry NULL
  MOE_TRY(check_ptrs({{topk_ids, "topk_ids"}, {topk_gates, "topk_gates"}, {counts, "counts"},
                      {offsets, "offsets"}, {perm_token, "perm_token"}, {inv_slot, "inv_slot"},
                      {ws, "ws"}},
                     {}));
  const moe::Problem p = make_problem(desc);
  if (ws_bytes < moe::round_ws_bytes(p, nullptr, nullptr))
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size(MOE_WS_ROUND)");
  moe::RoundWs w;
  moe::round_ws_bytes(p, &w, static_cast<unsigned char*>(ws));
  return hip_status(moe::launch_round(p, topk_ids, topk_gates, counts, offsets, perm_token,
                                      inv_slot, w, (hipStream_t)stream),
                    "token rounding launch");
} catch (...) {
  return caught();
}

moe_status moe_grouped_gemm_up(const moe_desc* desc, const void* X, const int32_t* offsets,
                               const int32_t* perm_token, const void* W_gate, const void* W_up,
                               void* H, void* ws, size_t ws_bytes, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_desc(desc, kGemmFlags));
  if (desc->T == 0) return MOE_OK;  // no-op; empty tensors may carry NULL
  MOE_TRY(check_ptrs({{X, "X"}, {offsets, "offsets"}, {perm_token, "perm_token"},
                      {W_gate, "W_gate"}, {W_up, "W_up"}, {H, "H"}},
                     {{ws, "ws"}}));
  const moe::Problem p = make_problem(desc);
  if (!ws || ws_bytes < moe::tile_table_bytes(p))
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size(MOE_WS_GROUPED_FFN)");
  hipStream_t s = (hipStream_t)stream;
  if (skinny(p, desc))
    return hip_status(moe::launch_gemm_up_skinny(p, X, perm_token, offsets, W_gate, W_up, H, s),
                      "grouped GEMM (up, weight-streaming) launch");
  int32_t* table = static_cast<int32_t*>(ws);
  if (!(desc->flags & MOE_FLAG_TILE_TABLE_READY))
    MOE_TRY(hip_status(moe::launch_tile_table(p, offsets, table, s), "tile table launch"));
  return hip_status(moe::launch_gemm_up(p, X, perm_token, table, W_gate, W_up, H, s, nullptr,
                                        offsets, stream_rows(p, desc)),
                    "grouped GEMM (up) launch");
} catch (...) {
  return caught();
}

moe_status moe_grouped_gemm_down(const moe_desc* desc, const void* H, const int32_t* offsets,
                                 const void* W_down, void* O, void* ws, size_t ws_bytes,
                                 void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_desc(desc, kGemmFlags));
  if (desc->T == 0) return MOE_OK;  // no-op; empty tensors may carry NULL
  MOE_TRY(check_ptrs({{H, "H"}, {offsets, "offsets"}, {W_down, "W_down"}, {O, "O"}}, {{ws, "ws"}}));
  const moe::Problem p = make_problem(desc);
  if (!ws || ws_bytes < moe::tile_table_bytes(p))
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size(MOE_WS_GROUPED_FFN)");
  hipStream_t s = (hipStream_t)stream;
  if (skinny(p, desc))
    return hip_status(moe::launch_gemm_down_skinny(p, H, offsets, W_down, O, s),
                      "grouped GEMM (down, weight-streaming) launch");
  int32_t* table = static_cast<int32_t*>(ws);
  if (!(desc->flags & MOE_FLAG_TILE_TABLE_READY))
    MOE_TRY(hip_status(moe::launch_tile_table(p, offsets, table, s), "tile table launch"));
  return hip_status(moe::launch_gemm_down(p, H, table, W_down, O, s, offsets, stream_rows(p, desc)),
                    "grouped GEMM (down) launch");
} catch (...) {
  return caught();
}

moe_status moe_grouped_ffn(const moe_desc* desc, const void* X, const int32_t* offsets,
                           const int32_t* perm_token, const void* W_gate, const void* W_up,
                           const void* W_down, void* H, void* O, void* ws, size_t ws_bytes,
                           void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_desc(desc, kGemmFlags));
  if (desc->T == 0) return MOE_OK;  // no-op; empty tensors may carry NULL
  MOE_TRY(check_ptrs({{X, "X"}, {offsets, "offsets"}, {perm_token, "perm_token"},
                      {W_gate, "W_gate"}, {W_up, "W_up"}, {W_down, "W_down"}, {H, "H"}, {O, "O"}},
                     {{ws, "ws"}}));
  const moe::Problem p = make_problem(desc);
  if (!ws || ws_bytes < moe::tile_table_bytes(p))
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size(MOE_WS_GROUPED_FFN)");
  hipStream_t s = (hipStream_t)stream;
  if (skinny(p, desc)) {
    MOE_TRY(hip_status(moe::launch_gemm_up_skinny(p, X, perm_token, offsets, W_gate, W_up, H, s),
                       "grouped GEMM (up, weight-streaming) launch"));
    return hip_status(moe::launch_gemm_down_skinny(p, H, offsets, W_down, O, s),
                      "grouped GEMM (down, weight-streaming) launch");
  }
  int32_t* table = static_cast<int32_t*>(ws);
  if (!(desc->flags & MOE_FLAG_TILE_TABLE_READY))
    MOE_TRY(hip_status(moe::launch_tile_table(p, offsets, table, s), "tile table launch"));
  const int sr = stream_rows(p, desc);
  MOE_TRY(hip_status(moe::launch_gemm_up(p, X, perm_token, table, W_gate, W_up, H, s, nullptr,
                                         offsets, sr),
                     "grouped GEMM (up) launch"));
  return hip_status(moe::launch_gemm_down(p, H, table, W_down, O, s, offsets, sr),
                    "grouped GEMM (down) launch");
} catch (...) {
  return caught();
}

moe_status moe_combine(const moe_desc* desc, const void* O, const float* topk_gates,
                       const int32_t* inv_slot, void* Y, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_desc(desc));
  if (desc->T == 0) return MOE_OK;  // no-op; empty tensors may carry NULL
  MOE_TRY(check_ptrs({{O, "O"}, {topk_gates, "topk_gates"}, {inv_slot, "inv_slot"}, {Y, "Y"}}, {}));
  const moe::Problem p = make_problem(desc);
  return hip_status(moe::launch_combine(p, O, topk_gates, inv_slot, Y, (hipStream_t)stream),
                    "combine launch");
} catch (...) {
  return caught();
}

moe_status moe_forward(const moe_desc* desc, const void* X, const void* W_r, const float* bias,
                       const void* W_gate, const void* W_up, const void* W_down, void* Y,
                       void* ws, size_t ws_bytes, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_desc(desc, MOE_FLAG_GEMM_TILED | MOE_FLAG_GEMM_SKINNY | MOE_FLAG_TOKEN_ROUNDING |
                               MOE_FLAG_TOPK_THRESHOLD));
  if (desc->T == 0) return MOE_OK;  // no-op; empty tensors may carry NULL
  MOE_TRY(check_ptrs({{X, "X"}, {W_r, "W_r"}, {W_gate, "W_gate"}, {W_up, "W_up"},
                      {W_down, "W_down"}, {Y, "Y"}},
                     {{bias, "bias"}, {ws, "ws"}}));
  const moe::Problem p = make_problem(desc);
  const ForwardWs size_only = carve_forward(p, nullptr);
  if (!ws || ws_bytes < size_only.bytes)
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size(MOE_WS_FORWARD)");
  hipStream_t s = (hipStream_t)stream;
  ForwardWs w = carve_forward(p, static_cast<unsigned char*>(ws));
  const bool rounding = (desc->flags & MOE_FLAG_TOKEN_ROUNDING) != 0;
  MOE_TRY(run_route_permute(p, X, W_r, bias, nullptr, w.ids, w.gates, w.route_partial, w.blockcnt,
                            w.counts, w.offsets, w.raw, w.perm, w.inv, rounding ? nullptr : w.table,
                            s));
  if (rounding) {
    moe::RoundWs rw;
    moe::round_ws_bytes(p, &rw, w.round);
    MOE_TRY(hip_status(moe::launch_round(p, w.ids, w.gates, w.counts, w.offsets, w.perm, w.inv,
                                         rw, s),
                       "token rounding launch"));
    if (!skinny(p, desc))
      MOE_TRY(hip_status(moe::launch_tile_table(p, w.offsets, w.table, s), "tile table launch"));
  }
  if (skinny(p, desc)) {
    MOE_TRY(hip_status(moe::launch_gemm_up_skinny(p, X, w.perm, w.offsets, W_gate, W_up, w.H, s),
                       "grouped GEMM (up, weight-streaming) launch"));
    MOE_TRY(hip_status(moe::launch_gemm_down_skinny(p, w.H, w.offsets, W_down, w.O, s),
                       "grouped GEMM (down, weight-streaming) launch"));
  } else {
    const int sr = stream_rows(p, desc);
    MOE_TRY(hip_status(moe::launch_gemm_up(p, X, w.perm, w.table, W_gate, W_up, w.H, s, nullptr,
                                           w.offsets, sr),
                       "grouped GEMM (up) launch"));
    MOE_TRY(hip_status(moe::launch_gemm_down(p, w.H, w.table, W_down, w.O, s, w.offsets, sr),
                       "grouped GEMM (down) launch"));
  }
  return hip_status(moe::launch_combine(p, w.O, w.gates, w.inv, Y, s), "combine launch");
} catch (...) {
  return caught();
}

moe_status moe_forward_train(const moe_desc* desc, const void* X, const void* W_r,
                             const float* bias, const void* W_gate, const void* W_up,
                             const void* W_down, void* Y, void* saved, size_t saved_bytes,
                             void* ws, size_t ws_bytes, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_desc(desc, MOE_FLAG_GEMM_TILED | MOE_FLAG_TOPK_THRESHOLD));
  if (desc->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the training path is bf16 only");
  if (desc->T == 0) return MOE_OK;  // no-op; empty tensors may carry NULL
  MOE_TRY(check_ptrs({{X, "X"}, {W_r, "W_r"}, {W_gate, "W_gate"}, {W_up, "W_up"},
                      {W_down, "W_down"}, {Y, "Y"}, {saved, "saved"}, {ws, "ws"}},
                     {{bias, "bias"}}));
  const moe::Problem p = make_problem(desc);
  if (saved_bytes < carve_saved(p, nullptr).layout.bytes)
    return fail(MOE_ERR_WORKSPACE, "saved smaller than moe_workspace_size(MOE_WS_SAVED)");
  if (ws_bytes < carve_forward(p, nullptr).bytes)
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size(MOE_WS_FORWARD)");
  hipStream_t s = (hipStream_t)stream;
  const Saved sv = carve_saved(p, static_cast<unsigned char*>(saved));
  const ForwardWs w = carve_forward(p, static_cast<unsigned char*>(ws));
  MOE_TRY(run_route_permute(p, X, W_r, bias, sv.logits, sv.ids, sv.gates, w.route_partial,
                            w.blockcnt, sv.counts, sv.offsets, w.raw, sv.perm, sv.inv, sv.table,
                            s));
  MOE_TRY(hip_status(moe::launch_gemm_up(p, X, sv.perm, sv.table, W_gate, W_up, w.H, s, sv.Hpre),
                     "grouped GEMM (up) launch"));
  MOE_TRY(hip_status(moe::launch_gemm_down(p, w.H, sv.table, W_down, w.O, s),
                     "grouped GEMM (down) launch"));
  return hip_status(moe::launch_combine(p, w.O, sv.gates, sv.inv, Y, s), "combine launch");
} catch (...) {
  return caught();
}

moe_status moe_backward(const moe_desc* desc, const void* X, const void* W_r, const void* W_gate,
                        const void* W_up, const void* W_down, const void* dY, const void* saved,
                        size_t saved_bytes, void* dX, float* dW_r, float* dW_gate, float* dW_up,
                        float* dW_down, void* ws, size_t ws_bytes, void* stream) try {
  const StreamScope scope_(stream);
  g_last_error.clear();
  MOE_TRY(check_desc(desc, MOE_FLAG_GEMM_TILED | MOE_FLAG_TOPK_THRESHOLD));  // the latter: no effect here
  if (desc->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the training path is bf16 only");
  MOE_TRY(check_ptrs({{dW_r, "dW_r"}, {dW_gate, "dW_gate"}, {dW_up, "dW_up"}, {dW_down, "dW_down"}},
                     {}));
  const moe::Problem p = make_problem(desc);
  hipStream_t s = (hipStream_t)stream;
  if (desc->T == 0)   // no tokens: the weight gradients are zero
    return hip_status(moe::launch_zero_grads(p, dW_r, dW_gate, dW_up, dW_down, s),
                      "zero-gradient launch");
  MOE_TRY(check_ptrs({{X, "X"}, {W_r, "W_r"}, {W_gate, "W_gate"}, {W_up, "W_up"},
                      {W_down, "W_down"}, {dY, "dY"}, {saved, "saved"}, {dX, "dX"}, {ws, "ws"}},
                     {}));
  if (saved_bytes < carve_saved(p, nullptr).layout.bytes)
    return fail(MOE_ERR_WORKSPACE, "saved smaller than moe_workspace_size(MOE_WS_SAVED)");
  if (ws_bytes < moe::backward_ws_bytes(p, nullptr, nullptr))
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size(MOE_WS_BACKWARD)");
  const Saved sv = carve_saved(p, static_cast<unsigned char*>(const_cast<void*>(saved)));
  moe::BackwardWs w;
  moe::backward_ws_bytes(p, &w, static_cast<unsigned char*>(ws));
  return hip_status(moe::launch_backward(p, X, W_r, W_gate, W_up, W_down, dY, sv.ids, sv.gates,
                                         sv.inv, sv.perm, sv.offsets, sv.table, sv.Hpre, dX, dW_r,
                                         dW_gate, dW_up, dW_down, w, s),
                    "backward launch");
} catch (...) {
  return caught();
}

}  // extern "C"
