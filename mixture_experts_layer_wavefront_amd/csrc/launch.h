// Internal launchers of the gfx950 kernels (not part of the C ABI).
// Each enqueues its kernels on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Router: logits (bf16 X: split-bf16 MFMA, or K-split FMA for few tokens,
// with partial sums in `scratch`; fp32 X: fused FMA kernel, no scratch),
// wavefront top-k, softmax.  router_stats != nullptr also writes the router
// statistics [2E + 2] (importance | mean probability | aux loss | z-loss);
// the scratch size depends on whether statistics are wanted.
size_t route_scratch_bytes(int T, int E, int d, bool x_bf16, bool stats);
hipError_t launch_route(const void* X, bool x_bf16, const float* W_r,
                        const float* bias, int T, int d, int E, int k,
                        int gating, int32_t* topk_idx, float* topk_w,
                        void* scratch, float* router_stats, hipStream_t stream);

// Permute, three kernels: per-block counts and in-block ranks; one-block
// scan with capacity; destination rows and the row copy (one kernel for few
// copies).  With mt_prefix != nullptr it also writes the grouped FFN's tile
// schedule: M-tiles per expert under tile_code (m_tiles; see launch_grouped_ffn).
// X_perm == nullptr: no row is copied (dest_row and row_token only, for a
// grouped FFN that gathers its input rows through row_token).  tile_code2 !=
// 0: a second schedule under it at mt_prefix + E + 1 (the two-class FFN).
size_t permute_scratch_bytes(int T, int k, int E);
hipError_t launch_permute(const void* X, bool x_bf16, const int32_t* topk_idx,
                          int T, int d, int E, int k, int C,
                          int32_t* counts, int32_t* offsets, int32_t* dropped,
                          int32_t* dest_row, int32_t* row_token, void* X_perm,
                          void* scratch, int32_t* mt_prefix, int tile_code,
                          hipStream_t stream, int tile_code2 = 0);

// Grouped SwiGLU FFN.  `rows_per_expert` (the mean, known on the host from
// the shape alone) picks the tile shape: ffn_tile_rows() rows per tile (64
// for fp32 layers, whose FMA kernels take 64 x 64 tiles).  The tile schedule
// (exclusive prefix over experts of their tile counts, E + 1 ints; a region
// of 2 (E + 1) ints) lives at the start of `scratch`; with prefix_ready the
// caller has already written it there.  w_scales !=
// nullptr: the weights are FP8 E4M3 codes with scales [E, 3] (bf16 layers).
// The down projection runs as two K halves (their sums added afterwards) for
// shapes whose 256 x 256 tiles fill the chip only a few times; the second
// half's partial sums need R d fp32 more scratch.  gather != nullptr (bf16
// layers, gather_rows * d * 2 < 2^31): X_perm is the layer's input X itself
// ([gather_rows, d]) and row r of the expert-grouped order is its row
// gather[r] (the permute's row_token), so the permuted copy is never made.
// side != nullptr (from ffn_side_stream) and ffn_two_class: the experts run
// in two classes, the few-row one on `side` (forked from and joined back
// into `stream`); the schedule region holds two prefixes, 2 (E + 1) ints.
int ffn_tile_rows(bool bf16, int rows_per_expert, bool fp8 = false);
// The M-tile code of moe_forward's grouped FFN (m_tiles): ffn_tile_rows, or
// 256-row tiles that take remainders of up to 64 rows (256-row tiles with
// more than 256 rows per expert, bf16 or FP8 weights).  With two_class: the
// schedule of the experts of at most kClassRows rows on 160-row tiles, and
// ffn_tile_code2 that of the others on tall tiles (0: no second schedule).
int ffn_tile_code(bool bf16, int rows_per_expert, bool fp8 = false, bool two_class = false);
int ffn_tile_code2(bool two_class);
// Whether the shape runs the grouped FFN in two classes of experts (tall
// tiles over at least 64 experts): the experts' rows decide each expert's
// class on the device, the few-row class runs on a side stream beside the
// other (ffn_side_stream).
bool ffn_two_class(bool bf16, bool fp8, int E, int rows_per_expert, int d, int d_ff);
// The library's side stream for the current device (made on the first call
// that is not inside a graph capture of `stream`, kept until the process
// ends), or nullptr where there is none: then the FFN runs in one class.
hipStream_t ffn_side_stream(hipStream_t stream);
// The M-tile code of the training forward's and the backward's GEMMs (their
// own tile shapes: 32-row, 256-row or tall tiles).
int ffn_train_tile_code(int rows_per_expert);
bool ffn_split_down(bool bf16, int E, int rows_per_expert, int d, int d_ff);
size_t ffn_scratch_bytes(int64_t R, int E, int d, int d_ff, bool bf16, int rows_per_expert);
hipError_t launch_grouped_ffn(const void* X_perm, bool bf16,
                              const int32_t* offsets, const void* W_gate,
                              const void* W_up, const void* W_down,
                              int64_t R, int d, int E, int d_ff, int rows_per_expert,
                              float* Y_perm, void* scratch, bool prefix_ready,
                              hipStream_t stream, const float* w_scales = nullptr,
                              bool defer_half_sum = false, const int32_t* gather = nullptr,
                              int gather_rows = 0, hipStream_t side = nullptr);

// Where a split down projection leaves its second K half (inside `scratch`),
// or nullptr when it is not split.
float* ffn_half_sums(void* scratch, int64_t R, int E, int d, int d_ff, bool bf16,
                     int rows_per_expert);

// Training forward (bf16 layers): the grouped FFN that also keeps
// G = X Wg^T and U = X Wu^T (bf16 [R, d_ff]) and H (bf16 [R, d_ff]) for the
// backward; mt_prefix holds E + 1 ints (written unless prefix_ready).
hipError_t launch_grouped_ffn_train(const void* X_perm, const int32_t* offsets,
                                    const void* W_gate, const void* W_up, const void* W_down,
                                    int64_t R, int d, int E, int d_ff, int rows_per_expert,
                                    int32_t* mt_prefix, bool prefix_ready, void* H, void* G,
                                    void* U, float* Y_perm, hipStream_t stream);

// Backward, data gradients of the experts: dGU [R, 2 d_ff] bf16 = (dG | dU)
// from dH = dY_perm Wd and the saved G, U; dX_perm [2, R, d] fp32 holds the
// two partial sums dG Wg and dU Wu (their sum is the rows' gradient).
// The weights are read as stored ([E, out, in]), along their rows.
hipError_t launch_ffn_dgrad(const void* dY_perm, const int32_t* offsets, const void* W_gate,
                            const void* W_up, const void* W_down, const void* G, const void* U,
                            int64_t R, int d, int E, int d_ff, int rows_per_expert,
                            int32_t* mt_prefix, void* dGU, float* dX_perm, hipStream_t stream);

// Weight gradients: for every expert e, C_e = A_e^T B_e over the expert's
// rows [offsets[e], offsets[e + 1]) of A [R, lda] (M columns used) and
// B [R, ldb] (N columns), bf16; rows m < msplit of C_e go to
// C0 [E, msplit, N], the others to C1 [E, M - msplit, N] (fp32).
hipError_t launch_wgrad(const void* A, int lda, int M, const void* B, int ldb, int N,
                        const int32_t* offsets, int E, int msplit, float* C0, float* C1,
                        hipStream_t stream);

// Backward kernels that are not GEMMs (bf16 layers).
hipError_t launch_bwd_combine(const float* dout, const float* Y_perm, const int32_t* dest,
                              const float* topk_w, int T, int d, int k, void* dY_perm,
                              float* dl_sel, hipStream_t stream);
hipError_t launch_bwd_gather(const float* dX_perm, int64_t R, const int32_t* dest,
                             const int32_t* idx, const float* dl_sel, const float* W_r, int T,
                             int d, int k, float* dX, hipStream_t stream);
size_t router_wgrad_scratch_bytes(int T, int d, int E);
hipError_t launch_router_wgrad(const void* X, const int32_t* idx, const float* dl_sel, int T,
                               int d, int E, int k, float* dW_r, float* dbias, void* scratch,
                               hipStream_t stream);

// Expert offsets {0, T} of a dense FFN over all T rows (one "expert").
hipError_t launch_dense_offsets(int32_t* offsets, int T, hipStream_t stream);

// Gate-weighted gather-combine back to token order.  add_rows ([T, d] fp32 or
// nullptr) is the first term of every output row's sum; Y_half ([R, d] or
// nullptr): second partial sums of the expert rows, added to Y_perm's.
hipError_t launch_combine(const float* Y_perm, const int32_t* dest_row,
                          const float* topk_w, int T, int d, int k,
                          const float* add_rows, bool out_bf16, void* out,
                          hipStream_t stream, const float* Y_half = nullptr);

}  // namespace moe
