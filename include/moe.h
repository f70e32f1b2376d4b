/*
 * moe.h -- C ABI of the MI355X (gfx950) forward pass of one sparsely-gated
 * mixture-of-experts FFN layer.
 *
 * The layer, as the method page states it ("Sparsely-Gated MoE 구현 관점에서
 * 살펴보기: Router, Top-k, 부하 분산", section "순전파 과정(forward pass)은
 * 디스패치와 결합(combine)을 포함" -- the five-step forward pipeline):
 *   1. router logits  l = X @ W_r^T (+ bias)                    -> moe_route
 *   2. top-k experts per token and their renormalised weights   -> moe_route
 *   3. per-expert capacity slots (overflowing copies dropped)   -> moe_permute
 *   4. permute token copies into expert-contiguous order        -> moe_permute
 *   5. each expert's FFN on its rows, as one grouped GEMM       -> moe_grouped_ffn
 *      (or moe_grouped_ffn_rows, which reads the rows from X through
 *      the permute's row map instead of a permuted copy)
 *   6. un-permute and combine with the gate weights             -> moe_combine
 * moe_forward runs all of them (bf16 layers: steps 3-4 assign rows without
 * copying them, and step 5 reads them from X).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers (HIP device memory), row-major
 *   and contiguous, 16-byte aligned.  Host pointers: only `const
 *   moe_problem_t*`.
 * - Weights are stored [E, out, in], so every product is A @ W^T:
 *     W_r    [E, d_model]          fp32
 *     W_gate [E, d_ff, d_model]    act dtype
 *     W_up   [E, d_ff, d_model]    act dtype
 *     W_down [E, d_model, d_ff]    act dtype
 *   This is the packed one-tensor-per-projection layout of "MoonEP의 계획
 *   코드를 직접 돌려봤습니다" (thakicloud.com), section "설치 및 통합".
 * - Ownership: the caller owns every buffer, including the workspace.  The
 *   library never allocates device memory, frees or synchronises.  Global
 *   state: moe_forward_noalloc's fixed per-GPU scratch array, and one side
 *   stream with two events per GPU for grouped FFNs that run two classes of
 *   experts (bf16 layers of at least 64 experts averaging more than 256 rows
 *   each; see moe_grouped_ffn), made on the first such call that is not
 *   inside a graph capture and kept until the process ends.  Calls on
 *   distinct streams with distinct buffers and workspaces may run
 *   concurrently.
 * - Every call only enqueues work on `stream` and returns; no host
 *   synchronisation happens inside any call (no per-expert size is read
 *   back: the grouped GEMM schedules its tiles from device-side offsets).
 *   Two-class grouped FFNs fork part of their work onto the side stream
 *   after what `stream` holds and join it back into `stream` before they
 *   return, so later work on `stream` sees every result and a graph capture
 *   of the call holds both branches.
 * - Errors: arguments are validated on the host before anything is
 *   enqueued.  An invalid argument returns a negative status and writes
 *   nothing.  A failed launch returns MOE_ERR_HIP.  Faults inside kernels
 *   surface at the caller's next synchronisation.
 * - Supported envelope: 0 <= T < 2^24, 1 <= top_k <= E <= 256, top_k <= 32,
 *   d_model and d_ff multiples of 8 (16-byte rows), act/weight dtype pairs
 *   (F32,F32) and (BF16,BF16), out_dtype F32 or BF16.  T == 0 is a valid
 *   no-op.  Anything else is
 *   MOE_ERR_UNSUPPORTED (or MOE_ERR_INVALID_ARG for nonsense such as a
 *   negative size or a NULL required pointer).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* NULL required pointer, negative size, k > E */
  MOE_ERR_UNSUPPORTED = -2, /* outside the supported envelope above */
  MOE_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than required */
  MOE_ERR_HIP = -4,         /* a kernel launch failed */
  MOE_ERR_SCRATCH_LIMIT = -5 /* moe_forward_noalloc: the problem's workspace
                                exceeds MOE_NOALLOC_SCRATCH_BYTES */
} moe_status_t;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8_E4M3 = 2 /* expert weights only: OCP E4M3 codes, with scales
                      (moe_grouped_ffn_scaled / moe_forward_scaled) */
} moe_dtype_t;

/* Order of softmax and top-k ("Sparsely-Gated MoE 구현 관점에서 살펴보기",
 * section "Top-2 라우팅의 수치 예시": implementations either take the top-k
 * and renormalise the selected logits with a softmax, or take a softmax over
 * all experts first, then the top-k, then renormalise).  Selection is always
 * on the logits (ties to the lower expert id). */
typedef enum {
  MOE_TOPK_THEN_SOFTMAX = 0, /* w_j = exp(l_j - m) / sum_sel exp(l - m) */
  MOE_SOFTMAX_THEN_TOPK = 1  /* p = softmax(l over E); w_j = p_j / sum_sel p */
} moe_gating_t;

/* Shape of the problem (host struct, read synchronously during the call). */
typedef struct {
  int32_t T;               /* tokens (batch x sequence flattened)           */
  int32_t d_model;         /* hidden size                                   */
  int32_t E;               /* number of experts                             */
  int32_t top_k;           /* experts per token                             */
  int32_t d_ff;            /* expert FFN inner size                         */
  float capacity_factor;   /* <= 0: unlimited; else C = min(T, ceil(cf*T*k/E)) */
  moe_dtype_t act_dtype;   /* X, X_perm, H                                  */
  moe_dtype_t w_dtype;     /* W_gate, W_up, W_down (W_r, bias: always fp32);
                              equal to act_dtype, or FP8_E4M3 with BF16
                              activations in the _scaled entry points      */
  moe_gating_t gating;
  moe_dtype_t out_dtype;   /* out: F32 (no rounding beyond fp32) or BF16    */
} moe_problem_t;

/* Per-expert capacity C of the problem, or -1 when unlimited.  The capacity
 * bounds how many token copies one expert takes ("Sparsely-Gated MoE 구현
 * 관점에서 살펴보기", section "로드 밸런싱 손실과 용량은 별개"); the printed
 * formula is lost, the reading is C = min(T, ceil(cf * T * k / E)). */
int64_t moe_capacity(const moe_problem_t* p);

/* R: static upper bound on the number of kept token copies, the row count
 * of X_perm and Y_perm: T*k without capacity, else min(T*k, E*C). */
int64_t moe_rows_bound(const moe_problem_t* p);

/* Workspace bytes needed by moe_route, moe_permute, moe_grouped_ffn and
 * moe_forward (0 for an invalid problem; moe_route needs none for fp32
 * layers).  Workspaces are plain device memory, 256-byte aligned, with no
 * state kept between calls. */
size_t moe_route_workspace_bytes(const moe_problem_t* p);
size_t moe_permute_workspace_bytes(const moe_problem_t* p);
size_t moe_grouped_ffn_workspace_bytes(const moe_problem_t* p);
size_t moe_workspace_bytes(const moe_problem_t* p);

/* Step 1-2: router logits, top-k and gate weights.
 * "Sparsely-Gated MoE 구현 관점에서 살펴보기", sections "Router를 텐서
 * 형태에서 추적하기" (logits X @ W_r^T per token, T x E) and "Top-2 라우팅의
 * 수치 예시" (top-k, renormalised weights).
 *   X        [T, d_model]  act dtype
 *   W_r      [E, d_model]  fp32
 *   bias     [E] fp32, or NULL for none (added to the fp32 logits)
 *   topk_idx [T, top_k] int32 out: expert ids, by descending logit, ties to
 *                                  the lower id
 *   topk_w   [T, top_k] fp32  out: gate weights (sum to 1 per token)
 *   workspace >= moe_route_workspace_bytes(p) bytes (may be NULL when that
 *            is 0)
 * Logits are fp32.  bf16 layers: X is exactly bf16 and W_r is split exactly
 * into three bf16 terms, so the matrix cores form every product exactly and
 * accumulate in fp32; partial sums over K-slices are added in a fixed order.
 * fp32 layers: fp32 FMA accumulation. */
moe_status_t moe_route(const moe_problem_t* p, const void* X, const float* W_r,
                       const float* bias, int32_t* topk_idx, float* topk_w,
                       void* workspace, size_t ws_bytes, hipStream_t stream);

/* Step 3-4: histogram, capacity, offsets and the stable counting-sort
 * permute.  Copy (t, j) of expert e = topk_idx[t, j] gets rank
 * #{t' < t : e in topk_idx[t', :]}; it is kept iff rank < C and then goes to
 * row expert_offsets[e] + rank.  ("Sparsely-Gated MoE 구현 관점에서
 * 살펴보기", forward pipeline steps 2-3; counts and offsets are the
 * tokens_per_expert and cu_seqlens of "MoonEP의 계획 코드를 직접
 * 돌려봤습니다", section "설치 및 통합".)
 *   X              [T, d_model] act dtype
 *   topk_idx       [T, top_k] int32, every id in [0, E) (not checked on the
 *                  device; ids out of range are undefined behaviour)
 *   expert_counts  [E]   int32 out: copies routed to each expert (pre-capacity)
 *   expert_offsets [E+1] int32 out: exclusive prefix sum of min(count, C)
 *   num_dropped    [1]   int32 out: copies dropped by capacity
 *   dest_row       [T, top_k] int32 out: row in X_perm, -1 if dropped
 *   row_token      [R] int32 out: token of each row (rows >= offsets[E]
 *                  are not written)
 *   X_perm         [R, d_model] act dtype out: X_perm[r] = X[row_token[r]];
 *                  or NULL: no row is copied (for moe_grouped_ffn_rows,
 *                  which reads the rows of X through row_token)
 *   workspace      >= moe_permute_workspace_bytes(p) bytes */
moe_status_t moe_permute(const moe_problem_t* p, const void* X,
                         const int32_t* topk_idx, int32_t* expert_counts,
                         int32_t* expert_offsets, int32_t* num_dropped,
                         int32_t* dest_row, int32_t* row_token, void* X_perm,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

/* Step 5: every expert's SwiGLU FFN over its rows [offsets[e], offsets[e+1])
 * of X_perm, as one grouped GEMM pair ("5.3 Expert Parallelism", section
 * "최적화 2: GroupGEMM"; "Sparsely-Gated MoE 구현 관점에서 살펴보기",
 * forward pipeline step 4):
 *   Y[r] = (silu(X_perm[r] Wg_e^T) * (X_perm[r] Wu_e^T)) Wd_e^T
 * with silu(z) = z / (1 + exp(-z)).  bf16 inputs use bf16 MFMA with fp32
 * accumulation; the SwiGLU product is formed in fp32 and rounded once to
 * the act dtype.  With bf16 weights, at least 64 experts and more than 256
 * rows per expert on average, each expert's tile height is chosen on the
 * device from its row count (experts of at most 160 rows on 160-row tiles,
 * on the library's side stream, beside the others' taller tiles); each
 * row's sums run in the same order either way, so the result is the same
 * bit pattern.
 *   X_perm         [R, d_model] act dtype
 *   expert_offsets [E+1] int32 (device; never read back to the host)
 *   Y_perm         [R, d_model] fp32 out (rows >= offsets[E] not written)
 *   workspace      >= moe_grouped_ffn_workspace_bytes(p) bytes */
moe_status_t moe_grouped_ffn(const moe_problem_t* p, const void* X_perm,
                             const int32_t* expert_offsets, const void* W_gate,
                             const void* W_up, const void* W_down,
                             float* Y_perm, void* workspace, size_t ws_bytes,
                             hipStream_t stream);

/* Step 5 without the permuted copy of the input: moe_grouped_ffn with
 * X_perm[r] read as X[row_token[r]] (the same steps as above; the expert
 * rows are fetched from X by the gate/up GEMM's own loads, so the reorder of
 * step 4 only assigns rows).  Same result as moe_grouped_ffn on the X_perm
 * that moe_permute writes, bit for bit (and, with FP8 expert weights, as
 * moe_grouped_ffn_scaled).  bf16 activations with T * d_model * 2 < 2^31
 * bytes (else MOE_ERR_UNSUPPORTED).
 *   X              [T, d_model] bf16
 *   row_token      [R] int32: token of each row r < offsets[E] (moe_permute)
 *   expert_offsets [E+1] int32 (device)
 *   w_scales       [E, 3] fp32 when p->w_dtype is MOE_FP8_E4M3 (as in
 *                  moe_grouped_ffn_scaled), else NULL; a mismatch is
 *                  MOE_ERR_INVALID_ARG
 *   Y_perm         [R, d_model] fp32 out (rows >= offsets[E] not written)
 *   workspace      >= moe_grouped_ffn_workspace_bytes(p) bytes */
moe_status_t moe_grouped_ffn_rows(const moe_problem_t* p, const void* X,
                                  const int32_t* row_token, const int32_t* expert_offsets,
                                  const void* W_gate, const void* W_up, const void* W_down,
                                  const float* w_scales, float* Y_perm, void* workspace,
                                  size_t ws_bytes, hipStream_t stream);

/* Step 6: out[t] = sum over j ascending with dest_row[t, j] >= 0 of
 * topk_w[t, j] * Y_perm[dest_row[t, j]], accumulated in fp32 and stored in
 * out_dtype (one rounding when that is BF16).  A token with every copy dropped gets a zero row.
 * ("Sparsely-Gated MoE 구현 관점에서 살펴보기", section "Router를 텐서
 * 형태에서 추적하기": the output is the weighted sum of the selected
 * experts' outputs; forward pipeline step 5: un-permute and combine.)
 *   Y_perm   [R, d_model] fp32
 *   dest_row [T, top_k] int32, topk_w [T, top_k] fp32
 *   out      [T, d_model] out_dtype out */
moe_status_t moe_combine(const moe_problem_t* p, const float* Y_perm,
                         const int32_t* dest_row, const float* topk_w,
                         void* out, hipStream_t stream);

/* The whole layer: moe_route, moe_permute, moe_grouped_ffn, moe_combine in
 * order on `stream`, intermediates carved from the workspace.  bf16 layers
 * (T * d_model * 2 < 2^31 bytes) run the permute without its row copy and
 * moe_grouped_ffn_rows in place of moe_grouped_ffn (same result, bit for bit).
 *   out   [T, d_model] out_dtype out
 *   stats [E + (E+1) + 1] int32 out, or NULL: expert_counts | expert_offsets
 *         | num_dropped (routing statistics for monitoring)
 *   workspace >= moe_workspace_bytes(p) bytes */
moe_status_t moe_forward(const moe_problem_t* p, const void* X,
                         const float* W_r, const float* bias,
                         const void* W_gate, const void* W_up,
                         const void* W_down, void* out, int32_t* stats,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

/* moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results as moe_forward (bit for bit), without
 * the workspace: the intermediates live in a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library, one per GPU, held
 * from the library's first use on that GPU until the process ends.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * its first call on a device looks up the array's address there (the
 * current device must be the one `stream` belongs to).
 *   Limit: a problem whose moe_workspace_bytes(p) exceeds
 *   MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_SCRATCH_LIMIT (nothing is
 *   enqueued); e.g. decode batches and prefill chunks of a few hundred
 *   tokens at d_model 2048 fit.
 *   Concurrency: every call on one GPU shares that GPU's array, and each
 *   call leaves its intermediates there.  Calls that may overlap on one GPU
 *   (other streams, other threads) race on it: order them on one stream or
 *   use moe_forward with separate workspaces.  Nothing in the array needs to
 *   start at zero. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_forward_noalloc(const moe_problem_t* p, const void* X,
                                 const float* W_r, const float* bias,
                                 const void* W_gate, const void* W_up,
                                 const void* W_down, void* out, int32_t* stats,
                                 hipStream_t stream);

/* Router statistics for monitoring (forward values only), computed by the
 * router's selection kernel while it reads the logits and reduced in a fixed
 * order ("Sparsely-Gated MoE 구현 관점에서 살펴보기", section "로드 밸런싱
 * 손실과 용량은 별개": importance and load of the Sparsely-Gated MoE
 * auxiliary loss, GShard's dispatch fraction and mean gate, ST-MoE's router
 * z-loss).  router_stats [2E + 2] fp32 out:
 *   [0, E)   importance[e] = sum over tokens of the gate weight given to e
 *   [E, 2E)  mean_prob[e]  = mean over tokens of softmax(logits)[e] over all E
 *   [2E]     aux_loss      = E * sum_e (count[e] / (T k)) * mean_prob[e],
 *                            count[e] = tokens selecting e (before capacity)
 *   [2E+1]   z_loss        = mean over tokens of logsumexp(logits)^2
 * (logits are the fp32 router logits, bias included).  Routing outputs are
 * identical to moe_route's / moe_forward's.
 *   workspace >= moe_route_stats_workspace_bytes(p) (route), or
 *   >= moe_forward_stats_workspace_bytes(p) (whole layer) bytes */
size_t moe_route_stats_workspace_bytes(const moe_problem_t* p);
moe_status_t moe_route_stats(const moe_problem_t* p, const void* X,
                             const float* W_r, const float* bias,
                             int32_t* topk_idx, float* topk_w,
                             float* router_stats, void* workspace,
                             size_t ws_bytes, hipStream_t stream);
size_t moe_forward_stats_workspace_bytes(const moe_problem_t* p);
moe_status_t moe_forward_stats(const moe_problem_t* p, const void* X,
                               const float* W_r, const float* bias,
                               const void* W_gate, const void* W_up,
                               const void* W_down, void* out, int32_t* stats,
                               float* router_stats, void* workspace,
                               size_t ws_bytes, hipStream_t stream);

/* The layer with a shared expert (the DeepSeek-V3 layer form; "5.3 Expert
 * Parallelism", section "최적화 1: 공유 전문가를 통한 연산-통신 오버랩": next
 * to the routed experts one shared expert processes every token, and its
 * computation overlaps the routed experts' dispatch on another stream).
 *   out[t] = shared(X[t]) + moe(X)[t], shared = the same SwiGLU FFN on every
 *   row, with weights
 *     Ws_gate, Ws_up [shared_d_ff, d_model], Ws_down [d_model, shared_d_ff]
 *     (act dtype, like the expert weights).
 * The shared FFN's output (fp32) is the first term of each output row's fp32
 * sum, then the routed copies in slot order; one rounding at the store.
 * side_stream: NULL runs everything on `stream`; otherwise the shared FFN runs
 * on side_stream, ordered after the work already queued on `stream` and
 * joined back into `stream` before the combine (two events created and
 * released inside the call).  The result is bit-identical either way.
 * shared_d_ff: 8 <= shared_d_ff <= 2^20, a multiple of 8, else
 * MOE_ERR_UNSUPPORTED.  stats as in moe_forward.
 *   workspace >= moe_forward_shared_workspace_bytes(p, shared_d_ff) bytes */
size_t moe_forward_shared_workspace_bytes(const moe_problem_t* p,
                                          int32_t shared_d_ff);
moe_status_t moe_forward_shared(const moe_problem_t* p, int32_t shared_d_ff,
                                const void* X, const float* W_r,
                                const float* bias, const void* W_gate,
                                const void* W_up, const void* W_down,
                                const void* Ws_gate, const void* Ws_up,
                                const void* Ws_down, void* out, int32_t* stats,
                                void* workspace, size_t ws_bytes,
                                hipStream_t stream, hipStream_t side_stream);

/* FP8 expert weights with a scale per expert and projection
 * ("Expert를 똑같이 나눴는데도 GPU가 대기하는 이유: MoE의 토큰 쏠림", sections
 * "Weight Loading에서 텐서 구조 맞추기" and "적재 변환과 양자화 조합하기":
 * a per-expert quantisation step fits into loading the packed expert
 * weights).  p->w_dtype = MOE_FP8_E4M3, p->act_dtype = MOE_BF16; W_gate,
 * W_up, W_down hold one byte per weight (OCP FP8 E4M3 codes, same [E, out,
 * in] layout) and
 *   w_scales [E, 3] fp32 (device): gate, up, down scale of each expert,
 * so that expert e's weight is w_scales[e, proj] * decode(code).  The codes
 * are decoded exactly to bf16 for the bf16 MFMAs; the scale multiplies the
 * fp32 accumulator.  Same results and outputs as moe_grouped_ffn /
 * moe_forward on the decoded weights (up to fp32 rounding); half the weight
 * bytes.  d_model and d_ff must be multiples of 16 (else
 * MOE_ERR_UNSUPPORTED).  Workspace: moe_grouped_ffn_workspace_bytes(p) /
 * moe_workspace_bytes(p) of the FP8 problem.  moe_route(_stats),
 * moe_permute and moe_combine take FP8 problems too (they do not read expert
 * weights); moe_grouped_ffn and the moe_forward variants without scales
 * return MOE_ERR_UNSUPPORTED for them. */
moe_status_t moe_grouped_ffn_scaled(const moe_problem_t* p, const void* X_perm,
                                    const int32_t* expert_offsets,
                                    const void* W_gate, const void* W_up,
                                    const void* W_down, const float* w_scales,
                                    float* Y_perm, void* workspace,
                                    size_t ws_bytes, hipStream_t stream);
moe_status_t moe_forward_scaled(const moe_problem_t* p, const void* X,
                                const float* W_r, const float* bias,
                                const void* W_gate, const void* W_up,
                                const void* W_down, const float* w_scales,
                                void* out, int32_t* stats, void* workspace,
                                size_t ws_bytes, hipStream_t stream);

/* Training: the forward pass that keeps what the backward needs, and the
 * backward pass of the layer ("Expert를 똑같이 나눴는데도 GPU가 대기하는
 * 이유: MoE의 토큰 쏠림", section "Unsloth와의 MoE 학습 경로": training
 * runs the same grouped expert GEMMs; "가장 바쁜 랭크가 속도를 정합니다",
 * section "이 기술은 무엇인가": the expert weights' gradients come back in
 * the backward pass).  bf16 layers only (act_dtype = w_dtype = MOE_BF16,
 * else MOE_ERR_UNSUPPORTED); rows bound R = moe_rows_bound(p) must satisfy
 * R + 63 E < 2^22 - 64 (else MOE_ERR_UNSUPPORTED).
 *
 * moe_forward_train: moe_forward (same arguments, same out and stats) that
 * also fills `state` (device, >= moe_train_state_bytes(p) bytes, else
 * MOE_ERR_INVALID_ARG): routing, assignment, X_perm and the experts'
 * G = X Wg^T, U = X Wu^T, H (bf16) and Y_perm (fp32).  The state's layout is
 * private to the library; it stays valid until the caller reuses it.
 * workspace >= moe_workspace_bytes(p) bytes.
 *
 * moe_backward: gradients of a loss L given dout = dL/d(out) [T, d_model]
 * fp32, with the routing of the forward that wrote `state` held fixed (the
 * top-k selection and the capacity assignment are piecewise constant):
 *   dX [T, d_model], dW_r [E, d_model], dbias [E] (NULL: not computed),
 *   dW_gate, dW_up [E, d_ff, d_model], dW_down [E, d_model, d_ff],
 * all fp32, written (not accumulated).  X, W_r and the expert weights must
 * be the forward's.  The gate weights are the softmax of the selected
 * logits in both gating orders, so dl = w (dw - <w, dw>) at the selected
 * experts and 0 elsewhere, with dw[t,j] = <dout[t], Y_perm[dest[t,j]]>
 * (0 for a dropped copy).  The expert GEMMs take bf16 operands (G, U, H,
 * w dout, dG, dU) with fp32 accumulation; every sum has a fixed order.
 * workspace >= moe_backward_workspace_bytes(p) bytes: it holds w dout in
 * bf16 [R, d_model], dG | dU in bf16 [R, 2 d_ff], the two fp32 partial sums
 * of dX_perm [2, R, d_model], the logit gradients [T, top_k], the tile
 * schedule and the router weight gradient's partial sums (no copy of any
 * weight).  T = 0: nothing is written. */
size_t moe_train_state_bytes(const moe_problem_t* p);
moe_status_t moe_forward_train(const moe_problem_t* p, const void* X,
                               const float* W_r, const float* bias,
                               const void* W_gate, const void* W_up,
                               const void* W_down, void* out, int32_t* stats,
                               void* state, size_t state_bytes,
                               void* workspace, size_t ws_bytes,
                               hipStream_t stream);
size_t moe_backward_workspace_bytes(const moe_problem_t* p);
moe_status_t moe_backward(const moe_problem_t* p, const void* X,
                          const float* W_r, const void* W_gate,
                          const void* W_up, const void* W_down,
                          const void* state, size_t state_bytes,
                          const float* dout, float* dX, float* dW_r,
                          float* dbias, float* dW_gate, float* dW_up,
                          float* dW_down, void* workspace, size_t ws_bytes,
                          hipStream_t stream);

/* Static string naming a status code. */
const char* moe_status_string(moe_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
