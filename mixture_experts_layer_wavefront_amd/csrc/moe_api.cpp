// C ABI of the MoE FFN layer forward pass: argument validation, workspace
// carving and the kernel sequence.  Declarations and the contract of every
// entry point are in include/moe.h.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <mutex>

#include "launch.h"

namespace {

constexpr int kMaxE = 256;
constexpr int kMaxK = 32;
constexpr int kMaxT = 1 << 24;
constexpr int kMaxDim = 1 << 20;

size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

bool is_bf16(const moe_problem_t* p) { return p->act_dtype == MOE_BF16; }
bool out_bf16(const moe_problem_t* p) { return p->out_dtype == MOE_BF16; }
size_t act_bytes(const moe_problem_t* p) { return is_bf16(p) ? 2 : 4; }

// fp8_ok: FP8 expert weights (with bf16 activations) are accepted: the
// scaled entry points and the workspace-size queries.
moe_status_t validate(const moe_problem_t* p, bool fp8_ok = false) {
  if (p == nullptr) return MOE_ERR_INVALID_ARG;
  if (p->T < 0 || p->d_model <= 0 || p->E <= 0 || p->top_k <= 0 || p->d_ff <= 0)
    return MOE_ERR_INVALID_ARG;
  if (p->top_k > p->E) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(p->capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (p->act_dtype != MOE_F32 && p->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (p->w_dtype != MOE_F32 && p->w_dtype != MOE_BF16 && p->w_dtype != MOE_FP8_E4M3)
    return MOE_ERR_INVALID_ARG;
  if (p->act_dtype == MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  if (p->gating != MOE_TOPK_THEN_SOFTMAX && p->gating != MOE_SOFTMAX_THEN_TOPK)
    return MOE_ERR_INVALID_ARG;
  if (p->out_dtype != MOE_F32 && p->out_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (p->E > kMaxE || p->top_k > kMaxK || p->T >= kMaxT) return MOE_ERR_UNSUPPORTED;
  if (p->d_model % 8 != 0 || p->d_ff % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (p->d_model > kMaxDim || p->d_ff > kMaxDim) return MOE_ERR_UNSUPPORTED;
  if (p->w_dtype == MOE_FP8_E4M3) {
    if (!fp8_ok || p->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (p->d_model % 16 != 0 || p->d_ff % 16 != 0) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
  }
  if (p->act_dtype != p->w_dtype) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

bool is_fp8(const moe_problem_t* p) { return p->w_dtype == MOE_FP8_E4M3; }

// C as an int for the kernels: INT_MAX when unlimited.
int capacity_int(const moe_problem_t* p) {
  const int64_t C = moe_capacity(p);
  return C < 0 ? INT_MAX : (int)C;
}

// Mean rows per expert, known on the host without reading device data; it
// picks the grouped GEMM's tile shape.
int mean_rows_per_expert(const moe_problem_t* p) {
  double mean = (double)p->T * p->top_k / p->E;
  const int64_t C = moe_capacity(p);
  if (C >= 0 && (double)C < mean) mean = (double)C;
  return (int)std::ceil(mean);
}

// bf16 layers: the grouped FFN reads the tokens' rows of X through row_token
// (one 32-bit buffer range over X), so no permuted copy of X is made.
bool gather_input(const moe_problem_t* p) {
  return is_bf16(p) && (int64_t)p->T * p->d_model * 2 <= INT32_MAX;
}

struct ForwardLayout {
  size_t topk_idx, topk_w, route_scratch, perm_scratch, stats, dest_row, row_token,
      x_perm, ffn_scratch, y_perm, total;
};

ForwardLayout forward_layout(const moe_problem_t* p, bool router_stats = false) {
  const size_t Tk = (size_t)p->T * p->top_k;
  const size_t R = (size_t)moe_rows_bound(p);
  ForwardLayout L{};
  size_t o = 0;
  L.topk_idx = o; o += a256(Tk * 4);
  L.topk_w = o; o += a256(Tk * 4);
  L.route_scratch = o;
  o += a256(moe::route_scratch_bytes(p->T, p->E, p->d_model, is_bf16(p), router_stats));
  L.perm_scratch = o; o += a256(moe::permute_scratch_bytes(p->T, p->top_k, p->E));
  L.stats = o; o += a256((size_t)(2 * p->E + 2) * 4);
  L.dest_row = o; o += a256(Tk * 4);
  L.row_token = o; o += a256(R * 4);
  L.x_perm = o; o += gather_input(p) ? 0 : a256(R * p->d_model * act_bytes(p));
  L.ffn_scratch = o;
  o += a256(moe::ffn_scratch_bytes((int64_t)R, p->E, p->d_model, p->d_ff, is_bf16(p),
                                   mean_rows_per_expert(p)));
  L.y_perm = o; o += a256(R * p->d_model * 4);
  L.total = o;
  return L;
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Shared expert region, after the routed layer's workspace.
struct SharedLayout {
  size_t offsets, ffn_scratch, y_shared, total;
};

SharedLayout shared_layout(const moe_problem_t* p, int sdff, size_t base) {
  SharedLayout S{};
  size_t o = base;
  S.offsets = o; o += 256;
  S.ffn_scratch = o;
  o += a256(moe::ffn_scratch_bytes(p->T, 1, p->d_model, sdff, is_bf16(p), p->T));
  S.y_shared = o; o += a256((size_t)p->T * p->d_model * 4);
  S.total = o;
  return S;
}

moe_status_t validate_shared(int sdff) {
  if (sdff <= 0) return MOE_ERR_INVALID_ARG;
  if (sdff % 8 != 0 || sdff > kMaxDim) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Route, permute and the grouped FFN of the whole layer on `stream`; the
// combine's inputs are left in the workspace (see forward_layout).
struct RoutedOut {
  int32_t* dest_row;
  float* topk_w;
  float* y_perm;
  float* y_half;  // second K half of a split down projection (the combine adds it), or null
};

// side_ok: the grouped FFN may run its two classes of experts concurrently on
// the library's side stream (not for moe_forward_noalloc, which makes no
// stream).
hipError_t enqueue_routed(const moe_problem_t* p, const void* X, const float* W_r,
                          const float* bias, const void* W_gate, const void* W_up,
                          const void* W_down, int32_t* stats, float* router_stats,
                          char* ws, const ForwardLayout& L, hipStream_t stream,
                          RoutedOut* r, const float* w_scales = nullptr, bool side_ok = true) {
  int32_t* topk_idx = reinterpret_cast<int32_t*>(ws + L.topk_idx);
  float* topk_w = reinterpret_cast<float*>(ws + L.topk_w);
  int32_t* st_buf = stats ? stats : reinterpret_cast<int32_t*>(ws + L.stats);
  int32_t* counts = st_buf;
  int32_t* offsets = st_buf + p->E;
  int32_t* dropped = st_buf + 2 * p->E + 1;
  int32_t* dest_row = reinterpret_cast<int32_t*>(ws + L.dest_row);
  int32_t* row_token = reinterpret_cast<int32_t*>(ws + L.row_token);
  void* x_perm = ws + L.x_perm;
  float* y_perm = reinterpret_cast<float*>(ws + L.y_perm);
  const bool bf = is_bf16(p);
  *r = RoutedOut{dest_row, topk_w, y_perm,
                 moe::ffn_half_sums(ws + L.ffn_scratch, moe_rows_bound(p), p->E, p->d_model,
                                    p->d_ff, bf, mean_rows_per_expert(p))};

  hipError_t e = moe::launch_route(X, bf, W_r, bias, p->T, p->d_model, p->E, p->top_k,
                                   (int)p->gating, topk_idx, topk_w, ws + L.route_scratch,
                                   router_stats, stream);
  if (e != hipSuccess) return e;
  // the permute also writes the FFN's tile schedule(s) (start of its scratch)
  const int rows = mean_rows_per_expert(p);
  const bool fp8 = w_scales != nullptr;
  hipStream_t side = (side_ok && moe::ffn_two_class(bf, fp8, p->E, rows, p->d_model, p->d_ff))
                         ? moe::ffn_side_stream(stream)
                         : nullptr;
  const int bm = moe::ffn_tile_code(bf, rows, fp8, side != nullptr);
  int32_t* mt_prefix = bm > 0 ? reinterpret_cast<int32_t*>(ws + L.ffn_scratch) : nullptr;
  const bool gather = gather_input(p);
  e = moe::launch_permute(X, bf, topk_idx, p->T, p->d_model, p->E, p->top_k,
                          capacity_int(p), counts, offsets, dropped, dest_row, row_token,
                          gather ? nullptr : x_perm, ws + L.perm_scratch, mt_prefix, bm, stream,
                          moe::ffn_tile_code2(side != nullptr));
  if (e != hipSuccess) return e;
  return moe::launch_grouped_ffn(gather ? X : x_perm, bf, offsets, W_gate, W_up, W_down,
                                 moe_rows_bound(p), p->d_model, p->E, p->d_ff, rows, y_perm,
                                 ws + L.ffn_scratch, mt_prefix != nullptr, stream, w_scales,
                                 /*defer_half_sum=*/true, gather ? row_token : nullptr, p->T,
                                 side);
}

// The side stream for a stage-level grouped FFN call on `stream` (nullptr:
// one class of experts).
hipStream_t ffn_side(const moe_problem_t* p, bool fp8, hipStream_t stream) {
  return moe::ffn_two_class(is_bf16(p), fp8, p->E, mean_rows_per_expert(p), p->d_model, p->d_ff)
             ? moe::ffn_side_stream(stream)
             : nullptr;
}

// The whole layer with its intermediates carved from `ws` (L.total bytes).
moe_status_t enqueue_forward(const moe_problem_t* p, const void* X, const float* W_r,
                             const float* bias, const void* W_gate, const void* W_up,
                             const void* W_down, void* out, int32_t* stats, char* ws,
                             const ForwardLayout& L, hipStream_t stream, bool side_ok = true) {
  RoutedOut r{};
  hipError_t e = enqueue_routed(p, X, W_r, bias, W_gate, W_up, W_down, stats, nullptr, ws, L,
                                stream, &r, nullptr, side_ok);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_combine(r.y_perm, r.dest_row, r.topk_w, p->T, p->d_model, p->top_k,
                          nullptr, out_bf16(p), out, stream, r.y_half);
  return hip_status(e);
}

// ---- the workspace of moe_forward_noalloc ----------------------------------
// A fixed device array in this library's code object: each GPU that loads
// the library holds its own copy until the process ends.  Host code never
// passes `scratch` itself to a kernel (on the host the name only stands in
// for the symbol); it looks up the array's device address on the current
// device once and passes that address.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_addr[kMaxDevices];  // device address of `scratch`, per device

// The device address of `scratch` on the current device (looked up on the
// first call on that device, then kept).
hipError_t scratch_address(char** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (a == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = static_cast<char*>(a);
  }
  *addr = g_scratch_addr[dev];
  return hipSuccess;
}

// ---- training ---------------------------------------------------------------
// Training supports bf16 layers.  The backward GEMMs address a weight
// matrix, or an expert's rows of a saved activation, with one 32-bit buffer
// range.
moe_status_t validate_train(const moe_problem_t* p) {
  const moe_status_t st = validate(p);
  if (st != MOE_OK) return st;
  if (!is_bf16(p)) return MOE_ERR_UNSUPPORTED;
  const int64_t w_bytes = (int64_t)p->d_model * p->d_ff * 2;
  const int64_t row_bytes = (int64_t)std::max(p->d_model, 2 * p->d_ff) * 2;
  if (w_bytes >= (int64_t(1) << 31) || moe_rows_bound(p) * row_bytes >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// What moe_forward_train keeps for moe_backward.
struct TrainState {
  size_t topk_idx, topk_w, stats, dest_row, row_token, x_perm, g, u, h, y_perm, total;
};

TrainState train_state_layout(const moe_problem_t* p) {
  const size_t Tk = (size_t)p->T * p->top_k;
  const size_t R = (size_t)moe_rows_bound(p);
  const size_t d = p->d_model, dff = p->d_ff;
  TrainState S{};
  size_t o = 0;
  S.topk_idx = o; o += a256(Tk * 4);
  S.topk_w = o; o += a256(Tk * 4);
  S.stats = o; o += a256((size_t)(2 * p->E + 2) * 4);
  S.dest_row = o; o += a256(Tk * 4);
  S.row_token = o; o += a256(R * 4);
  S.x_perm = o; o += a256(R * d * 2);
  S.g = o; o += a256(R * dff * 2);
  S.u = o; o += a256(R * dff * 2);
  S.h = o; o += a256(R * dff * 2);
  S.y_perm = o; o += a256(R * d * 4);
  S.total = o;
  return S;
}

struct BackwardLayout {
  size_t dy, dgu, dxp, dl, mtp, rw, total;
};

BackwardLayout backward_layout(const moe_problem_t* p) {
  const size_t Tk = (size_t)p->T * p->top_k;
  const size_t R = (size_t)moe_rows_bound(p);
  const size_t d = p->d_model, dff = p->d_ff, E = p->E;
  BackwardLayout B{};
  size_t o = 0;
  B.dy = o; o += a256(R * d * 2);
  B.dgu = o; o += a256(R * 2 * dff * 2);
  B.dxp = o; o += a256(2 * R * d * 4);
  B.dl = o; o += a256(Tk * 4);
  B.mtp = o; o += a256((E + 1) * 4);
  B.rw = o; o += a256(moe::router_wgrad_scratch_bytes(p->T, p->d_model, p->E));
  B.total = o;
  return B;
}

}  // namespace

extern "C" {

int64_t moe_capacity(const moe_problem_t* p) {
  if (validate(p, true) != MOE_OK) return -1;
  if (!(p->capacity_factor > 0.f)) return -1;
  const double c = std::ceil((double)p->capacity_factor * p->T * p->top_k / p->E);
  return c < (double)p->T ? (int64_t)c : (int64_t)p->T;
}

int64_t moe_rows_bound(const moe_problem_t* p) {
  if (validate(p, true) != MOE_OK) return 0;
  const int64_t Tk = (int64_t)p->T * p->top_k;
  const int64_t C = moe_capacity(p);
  if (C < 0) return Tk;
  const int64_t EC = (int64_t)p->E * C;
  return EC < Tk ? EC : Tk;
}

size_t moe_route_workspace_bytes(const moe_problem_t* p) {
  if (validate(p, true) != MOE_OK) return 0;
  return a256(moe::route_scratch_bytes(p->T, p->E, p->d_model, is_bf16(p), false));
}

size_t moe_permute_workspace_bytes(const moe_problem_t* p) {
  if (validate(p, true) != MOE_OK) return 0;
  return a256(moe::permute_scratch_bytes(p->T, p->top_k, p->E));
}

size_t moe_grouped_ffn_workspace_bytes(const moe_problem_t* p) {
  if (validate(p, true) != MOE_OK) return 0;
  return a256(moe::ffn_scratch_bytes(moe_rows_bound(p), p->E, p->d_model, p->d_ff, is_bf16(p),
                                     mean_rows_per_expert(p)));
}

size_t moe_workspace_bytes(const moe_problem_t* p) {
  if (validate(p, true) != MOE_OK) return 0;
  return forward_layout(p).total;
}

moe_status_t moe_route(const moe_problem_t* p, const void* X, const float* W_r,
                       const float* bias, int32_t* topk_idx, float* topk_w,
                       void* workspace, size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = validate(p, true);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!X || !W_r || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_route_workspace_bytes(p);
  if (need > 0 && (!workspace || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_route(X, is_bf16(p), W_r, bias, p->T, p->d_model, p->E,
                                      p->top_k, (int)p->gating, topk_idx, topk_w, workspace,
                                      nullptr, stream));
}

size_t moe_route_stats_workspace_bytes(const moe_problem_t* p) {
  if (validate(p, true) != MOE_OK) return 0;
  return a256(moe::route_scratch_bytes(p->T, p->E, p->d_model, is_bf16(p), true));
}

moe_status_t moe_route_stats(const moe_problem_t* p, const void* X, const float* W_r,
                             const float* bias, int32_t* topk_idx, float* topk_w,
                             float* router_stats, void* workspace, size_t ws_bytes,
                             hipStream_t stream) {
  moe_status_t st = validate(p, true);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!X || !W_r || !topk_idx || !topk_w || !router_stats) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_route_stats_workspace_bytes(p);
  if (!workspace || ws_bytes < need) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_route(X, is_bf16(p), W_r, bias, p->T, p->d_model, p->E,
                                      p->top_k, (int)p->gating, topk_idx, topk_w, workspace,
                                      router_stats, stream));
}

moe_status_t moe_permute(const moe_problem_t* p, const void* X,
                         const int32_t* topk_idx, int32_t* expert_counts,
                         int32_t* expert_offsets, int32_t* num_dropped,
                         int32_t* dest_row, int32_t* row_token, void* X_perm,
                         void* workspace, size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = validate(p, true);
  if (st != MOE_OK) return st;
  if (!expert_counts || !expert_offsets || !num_dropped) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!X || !topk_idx || !dest_row || !row_token)) return MOE_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < moe_permute_workspace_bytes(p)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_permute(X, is_bf16(p), topk_idx, p->T, p->d_model, p->E,
                                        p->top_k, capacity_int(p), expert_counts,
                                        expert_offsets, num_dropped, dest_row, row_token,
                                        X_perm, workspace, nullptr, 0, stream));
}

moe_status_t moe_grouped_ffn(const moe_problem_t* p, const void* X_perm,
                             const int32_t* expert_offsets, const void* W_gate,
                             const void* W_up, const void* W_down, float* Y_perm,
                             void* workspace, size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = validate(p);
  if (st != MOE_OK) return st;
  const int64_t R = moe_rows_bound(p);
  if (R == 0) return MOE_OK;
  if (!X_perm || !expert_offsets || !W_gate || !W_up || !W_down || !Y_perm)
    return MOE_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < moe_grouped_ffn_workspace_bytes(p)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_grouped_ffn(X_perm, is_bf16(p), expert_offsets, W_gate, W_up,
                                            W_down, R, p->d_model, p->E, p->d_ff,
                                            mean_rows_per_expert(p), Y_perm, workspace, false,
                                            stream, nullptr, false, nullptr, 0,
                                            ffn_side(p, false, stream)));
}

moe_status_t moe_grouped_ffn_rows(const moe_problem_t* p, const void* X,
                                  const int32_t* row_token, const int32_t* expert_offsets,
                                  const void* W_gate, const void* W_up, const void* W_down,
                                  const float* w_scales, float* Y_perm, void* workspace,
                                  size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = validate(p, true);
  if (st != MOE_OK) return st;
  if (!gather_input(p)) return MOE_ERR_UNSUPPORTED;
  const int64_t R = moe_rows_bound(p);
  if (R == 0) return MOE_OK;
  if (!X || !row_token || !expert_offsets || !W_gate || !W_up || !W_down || !Y_perm)
    return MOE_ERR_INVALID_ARG;
  if (is_fp8(p) != (w_scales != nullptr)) return MOE_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < moe_grouped_ffn_workspace_bytes(p)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_grouped_ffn(X, true, expert_offsets, W_gate, W_up, W_down, R,
                                            p->d_model, p->E, p->d_ff,
                                            mean_rows_per_expert(p), Y_perm, workspace, false,
                                            stream, w_scales, false, row_token, p->T,
                                            ffn_side(p, w_scales != nullptr, stream)));
}

moe_status_t moe_combine(const moe_problem_t* p, const float* Y_perm,
                         const int32_t* dest_row, const float* topk_w, void* out,
                         hipStream_t stream) {
  moe_status_t st = validate(p, true);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!Y_perm || !dest_row || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine(Y_perm, dest_row, topk_w, p->T, p->d_model,
                                        p->top_k, nullptr, out_bf16(p), out, stream));
}

moe_status_t moe_forward(const moe_problem_t* p, const void* X, const float* W_r,
                         const float* bias, const void* W_gate, const void* W_up,
                         const void* W_down, void* out, int32_t* stats,
                         void* workspace, size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = validate(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!X || !W_r || !W_gate || !W_up || !W_down || !out) return MOE_ERR_INVALID_ARG;
  const ForwardLayout L = forward_layout(p);
  if (!workspace || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return enqueue_forward(p, X, W_r, bias, W_gate, W_up, W_down, out, stats,
                         static_cast<char*>(workspace), L, stream);
}

moe_status_t moe_forward_noalloc(const moe_problem_t* p, const void* X, const float* W_r,
                                 const float* bias, const void* W_gate, const void* W_up,
                                 const void* W_down, void* out, int32_t* stats,
                                 hipStream_t stream) {
  moe_status_t st = validate(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!X || !W_r || !W_gate || !W_up || !W_down || !out) return MOE_ERR_INVALID_ARG;
  const ForwardLayout L = forward_layout(p);
  if (L.total > kScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
  char* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return MOE_ERR_HIP;
  return enqueue_forward(p, X, W_r, bias, W_gate, W_up, W_down, out, stats, ws, L, stream,
                         /*side_ok=*/false);
}

size_t moe_forward_stats_workspace_bytes(const moe_problem_t* p) {
  if (validate(p) != MOE_OK) return 0;
  return forward_layout(p, true).total;
}

moe_status_t moe_forward_stats(const moe_problem_t* p, const void* X, const float* W_r,
                               const float* bias, const void* W_gate, const void* W_up,
                               const void* W_down, void* out, int32_t* stats,
                               float* router_stats, void* workspace, size_t ws_bytes,
                               hipStream_t stream) {
  moe_status_t st = validate(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!X || !W_r || !W_gate || !W_up || !W_down || !out || !router_stats)
    return MOE_ERR_INVALID_ARG;
  const ForwardLayout L = forward_layout(p, true);
  if (!workspace || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  RoutedOut r{};
  hipError_t e = enqueue_routed(p, X, W_r, bias, W_gate, W_up, W_down, stats, router_stats, ws,
                                L, stream, &r);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_combine(r.y_perm, r.dest_row, r.topk_w, p->T, p->d_model, p->top_k,
                          nullptr, out_bf16(p), out, stream, r.y_half);
  return hip_status(e);
}

size_t moe_forward_shared_workspace_bytes(const moe_problem_t* p, int32_t shared_d_ff) {
  if (validate(p) != MOE_OK || validate_shared(shared_d_ff) != MOE_OK) return 0;
  return shared_layout(p, shared_d_ff, forward_layout(p).total).total;
}

moe_status_t moe_forward_shared(const moe_problem_t* p, int32_t shared_d_ff,
                                const void* X, const float* W_r, const float* bias,
                                const void* W_gate, const void* W_up, const void* W_down,
                                const void* Ws_gate, const void* Ws_up, const void* Ws_down,
                                void* out, int32_t* stats, void* workspace, size_t ws_bytes,
                                hipStream_t stream, hipStream_t side_stream) {
  moe_status_t st = validate(p);
  if (st != MOE_OK) return st;
  if ((st = validate_shared(shared_d_ff)) != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!X || !W_r || !W_gate || !W_up || !W_down || !Ws_gate || !Ws_up || !Ws_down || !out)
    return MOE_ERR_INVALID_ARG;
  const ForwardLayout L = forward_layout(p);
  const SharedLayout S = shared_layout(p, shared_d_ff, L.total);
  if (!workspace || ws_bytes < S.total) return MOE_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  int32_t* s_offsets = reinterpret_cast<int32_t*>(ws + S.offsets);
  float* y_shared = reinterpret_cast<float*>(ws + S.y_shared);

  // fork: the shared FFN on side_stream after what `stream` already holds
  hipEvent_t fork = nullptr, join = nullptr;
  hipStream_t ss = stream;
  hipError_t e = hipSuccess;
  if (side_stream != nullptr) {
    ss = side_stream;
    if ((e = hipEventCreateWithFlags(&fork, hipEventDisableTiming)) == hipSuccess &&
        (e = hipEventCreateWithFlags(&join, hipEventDisableTiming)) == hipSuccess &&
        (e = hipEventRecord(fork, stream)) == hipSuccess)
      e = hipStreamWaitEvent(side_stream, fork, 0);
  }
  if (e == hipSuccess) e = moe::launch_dense_offsets(s_offsets, p->T, ss);
  if (e == hipSuccess)
    e = moe::launch_grouped_ffn(X, is_bf16(p), s_offsets, Ws_gate, Ws_up, Ws_down, p->T,
                                p->d_model, 1, shared_d_ff, p->T, y_shared,
                                ws + S.ffn_scratch, false, ss);
  if (e == hipSuccess && side_stream != nullptr) e = hipEventRecord(join, side_stream);
  RoutedOut r{};
  if (e == hipSuccess)
    e = enqueue_routed(p, X, W_r, bias, W_gate, W_up, W_down, stats, nullptr, ws, L, stream, &r);
  // join before the combine adds the shared rows
  if (e == hipSuccess && side_stream != nullptr) e = hipStreamWaitEvent(stream, join, 0);
  if (e == hipSuccess)
    e = moe::launch_combine(r.y_perm, r.dest_row, r.topk_w, p->T, p->d_model, p->top_k,
                            y_shared, out_bf16(p), out, stream, r.y_half);
  if (fork) (void)hipEventDestroy(fork);
  if (join) (void)hipEventDestroy(join);
  return hip_status(e);
}

moe_status_t moe_grouped_ffn_scaled(const moe_problem_t* p, const void* X_perm,
                                    const int32_t* expert_offsets, const void* W_gate,
                                    const void* W_up, const void* W_down,
                                    const float* w_scales, float* Y_perm, void* workspace,
                                    size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = validate(p, true);
  if (st != MOE_OK) return st;
  if (!is_fp8(p)) return MOE_ERR_UNSUPPORTED;
  const int64_t R = moe_rows_bound(p);
  if (R == 0) return MOE_OK;
  if (!X_perm || !expert_offsets || !W_gate || !W_up || !W_down || !w_scales || !Y_perm)
    return MOE_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < moe_grouped_ffn_workspace_bytes(p)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_grouped_ffn(X_perm, true, expert_offsets, W_gate, W_up, W_down,
                                            R, p->d_model, p->E, p->d_ff,
                                            mean_rows_per_expert(p), Y_perm, workspace, false,
                                            stream, w_scales));
}

moe_status_t moe_forward_scaled(const moe_problem_t* p, const void* X, const float* W_r,
                                const float* bias, const void* W_gate, const void* W_up,
                                const void* W_down, const float* w_scales, void* out,
                                int32_t* stats, void* workspace, size_t ws_bytes,
                                hipStream_t stream) {
  moe_status_t st = validate(p, true);
  if (st != MOE_OK) return st;
  if (!is_fp8(p)) return MOE_ERR_UNSUPPORTED;
  if (p->T == 0) return MOE_OK;
  if (!X || !W_r || !W_gate || !W_up || !W_down || !w_scales || !out)
    return MOE_ERR_INVALID_ARG;
  const ForwardLayout L = forward_layout(p);
  if (!workspace || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  RoutedOut r{};
  hipError_t e = enqueue_routed(p, X, W_r, bias, W_gate, W_up, W_down, stats, nullptr, ws, L,
                                stream, &r, w_scales);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_combine(r.y_perm, r.dest_row, r.topk_w, p->T, p->d_model, p->top_k,
                          nullptr, out_bf16(p), out, stream, r.y_half);
  return hip_status(e);
}

size_t moe_train_state_bytes(const moe_problem_t* p) {
  if (validate_train(p) != MOE_OK) return 0;
  return train_state_layout(p).total;
}

moe_status_t moe_forward_train(const moe_problem_t* p, const void* X, const float* W_r,
                               const float* bias, const void* W_gate, const void* W_up,
                               const void* W_down, void* out, int32_t* stats, void* state,
                               size_t state_bytes, void* workspace, size_t ws_bytes,
                               hipStream_t stream) {
  moe_status_t st = validate_train(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!X || !W_r || !W_gate || !W_up || !W_down || !out) return MOE_ERR_INVALID_ARG;
  const TrainState S = train_state_layout(p);
  if (!state || state_bytes < S.total) return MOE_ERR_INVALID_ARG;
  const ForwardLayout L = forward_layout(p);
  if (!workspace || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  char* sb = static_cast<char*>(state);
  char* ws = static_cast<char*>(workspace);
  int32_t* topk_idx = reinterpret_cast<int32_t*>(sb + S.topk_idx);
  float* topk_w = reinterpret_cast<float*>(sb + S.topk_w);
  int32_t* st_buf = reinterpret_cast<int32_t*>(sb + S.stats);
  int32_t* dest_row = reinterpret_cast<int32_t*>(sb + S.dest_row);
  int32_t* row_token = reinterpret_cast<int32_t*>(sb + S.row_token);
  float* y_perm = reinterpret_cast<float*>(sb + S.y_perm);
  const int rows = mean_rows_per_expert(p);
  hipError_t e = moe::launch_route(X, true, W_r, bias, p->T, p->d_model, p->E, p->top_k,
                                   (int)p->gating, topk_idx, topk_w, ws + L.route_scratch,
                                   nullptr, stream);
  const int bm = moe::ffn_train_tile_code(rows);
  int32_t* mt_prefix = reinterpret_cast<int32_t*>(ws + L.ffn_scratch);
  if (e == hipSuccess)
    e = moe::launch_permute(X, true, topk_idx, p->T, p->d_model, p->E, p->top_k,
                            capacity_int(p), st_buf, st_buf + p->E, st_buf + 2 * p->E + 1,
                            dest_row, row_token, sb + S.x_perm, ws + L.perm_scratch, mt_prefix,
                            bm, stream);
  if (e == hipSuccess)
    e = moe::launch_grouped_ffn_train(sb + S.x_perm, st_buf + p->E, W_gate, W_up, W_down,
                                      moe_rows_bound(p), p->d_model, p->E, p->d_ff, rows,
                                      mt_prefix, true, sb + S.h, sb + S.g, sb + S.u, y_perm,
                                      stream);
  if (e == hipSuccess)
    e = moe::launch_combine(y_perm, dest_row, topk_w, p->T, p->d_model, p->top_k, nullptr,
                            out_bf16(p), out, stream);
  if (e == hipSuccess && stats)
    e = hipMemcpyAsync(stats, st_buf, (size_t)(2 * p->E + 2) * 4, hipMemcpyDeviceToDevice,
                       stream);
  return hip_status(e);
}

size_t moe_backward_workspace_bytes(const moe_problem_t* p) {
  if (validate_train(p) != MOE_OK) return 0;
  return backward_layout(p).total;
}

moe_status_t moe_backward(const moe_problem_t* p, const void* X, const float* W_r,
                          const void* W_gate, const void* W_up, const void* W_down,
                          const void* state, size_t state_bytes, const float* dout, float* dX,
                          float* dW_r, float* dbias, float* dW_gate, float* dW_up,
                          float* dW_down, void* workspace, size_t ws_bytes,
                          hipStream_t stream) {
  moe_status_t st = validate_train(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!X || !W_r || !W_gate || !W_up || !W_down || !dout || !dX || !dW_r || !dW_gate ||
      !dW_up || !dW_down)
    return MOE_ERR_INVALID_ARG;
  const TrainState S = train_state_layout(p);
  if (!state || state_bytes < S.total) return MOE_ERR_INVALID_ARG;
  const BackwardLayout B = backward_layout(p);
  if (!workspace || ws_bytes < B.total) return MOE_ERR_WORKSPACE;
  const char* sb = static_cast<const char*>(state);
  char* ws = static_cast<char*>(workspace);
  const int T = p->T, d = p->d_model, E = p->E, k = p->top_k, dff = p->d_ff;
  const int64_t R = moe_rows_bound(p);
  const int32_t* topk_idx = reinterpret_cast<const int32_t*>(sb + S.topk_idx);
  const float* topk_w = reinterpret_cast<const float*>(sb + S.topk_w);
  const int32_t* offsets = reinterpret_cast<const int32_t*>(sb + S.stats) + E;
  const int32_t* dest_row = reinterpret_cast<const int32_t*>(sb + S.dest_row);
  const float* y_perm = reinterpret_cast<const float*>(sb + S.y_perm);
  float* dl = reinterpret_cast<float*>(ws + B.dl);
  int32_t* mtp = reinterpret_cast<int32_t*>(ws + B.mtp);
  float* dxp = reinterpret_cast<float*>(ws + B.dxp);

  // combine and gate weights
  hipError_t e =
      moe::launch_bwd_combine(dout, y_perm, dest_row, topk_w, T, d, k, ws + B.dy, dl, stream);
  // experts, data gradients (SwiGLU backward in the dH epilogue)
  if (e == hipSuccess)
    e = moe::launch_ffn_dgrad(ws + B.dy, offsets, W_gate, W_up, W_down, sb + S.g, sb + S.u, R,
                              d, E, dff, mean_rows_per_expert(p), mtp, ws + B.dgu, dxp, stream);
  // permute and router
  if (e == hipSuccess)
    e = moe::launch_bwd_gather(dxp, R, dest_row, topk_idx, dl, W_r, T, d, k, dX, stream);
  if (e == hipSuccess)
    e = moe::launch_router_wgrad(X, topk_idx, dl, T, d, E, k, dW_r, dbias, ws + B.rw, stream);
  // experts, weight gradients over each expert's rows:
  // dW_down = dY^T H, [dW_gate ; dW_up] = [dG | dU]^T X_perm
  if (e == hipSuccess)
    e = moe::launch_wgrad(ws + B.dy, d, d, sb + S.h, dff, dff, offsets, E, d, dW_down, nullptr,
                          stream);
  if (e == hipSuccess)
    e = moe::launch_wgrad(ws + B.dgu, 2 * dff, 2 * dff, sb + S.x_perm, d, d, offsets, E, dff,
                          dW_gate, dW_up, stream);
  return hip_status(e);
}

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: outside the supported envelope";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a kernel launch failed";
    case MOE_ERR_SCRATCH_LIMIT:
      return "MOE_ERR_SCRATCH_LIMIT: the problem needs more workspace than the library's "
             "static scratch holds (MOE_NOALLOC_SCRATCH_BYTES, 64 MiB)";
  }
  return "unknown moe_status_t";
}

}  // extern "C"
