// Backward pass of the MoE FFN layer: the kernels that are not GEMMs.
//
// Method: the chain rule through each forward step (the pages print no
// backward formula; "Expert를 똑같이 나눴는데도 GPU가 대기하는 이유"
// (portfolio.ywsung.com), section "Unsloth와의 MoE 학습 경로": training runs
// the same grouped expert GEMMs with gradients).  With the top-k selection
// and the capacity assignment held fixed:
//   combine   dY_perm[r] = w[t,j] dout[t],  dw[t,j] = <dout[t], Y_perm[r]>
//             (r = dest[t,j]; a dropped copy has dw = 0)
//   gate      dl[t, idx[t,j]] = w[t,j] (dw[t,j] - sum_i w[t,i] dw[t,i])
//             (both gating orders: the gate weights are the softmax of the
//             selected logits)
//   permute   dX[t] = sum over kept copies of dX_perm[dest[t,j]]
//   router    dX[t] += sum_j dl[t,j] W_r[idx[t,j]],  dW_r = dl^T X,
//             dbias = sum_t dl[t]
// The expert GEMMs (dgrad and wgrad) run on the grouped GEMM kernel; their
// transposed operands are written here.  Every sum runs in a fixed order,
// so the same inputs give the same bits.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kTokPerBlock = 4;  // one wavefront per token, 256 threads

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// One wavefront per token.  For each slot j (in order) with a kept copy
// r = dest[t, j]: lanes take 4 consecutive columns per step, dw is their
// per-lane fp32 sum reduced by a butterfly, and dY_perm[r] = bf16(w dout[t]).
// Then dl[t, j] = w_j (dw_j - sum_i w_i dw_i), the sum in slot order.
__global__ __launch_bounds__(256) void bwd_combine_kernel(
    const float* __restrict__ dout, const float* __restrict__ Y_perm,
    const int32_t* __restrict__ dest, const float* __restrict__ w, int T, int d,
    int k, uint16_t* __restrict__ dY_perm, float* __restrict__ dl_sel) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  const float4* g = reinterpret_cast<const float4*>(dout + (int64_t)t * d);
  const int d4 = d / 4;
  float my_dw = 0.f, my_w = 0.f;  // lane j < k keeps slot j's values
  for (int j = 0; j < k; ++j) {
    const int r = dest[(int64_t)t * k + j];
    const float wt = w[(int64_t)t * k + j];
    float s = 0.f;
    if (r >= 0) {
      const float4* y = reinterpret_cast<const float4*>(Y_perm + (int64_t)r * d);
      uint2* o = reinterpret_cast<uint2*>(dY_perm + (int64_t)r * d);
      for (int c = lane; c < d4; c += kWave) {
        const float4 a = g[c], b = y[c];
        s = fmaf(a.x, b.x, s);
        s = fmaf(a.y, b.y, s);
        s = fmaf(a.z, b.z, s);
        s = fmaf(a.w, b.w, s);
        o[c] = make_uint2(pack_bf16x2(wt * a.x, wt * a.y), pack_bf16x2(wt * a.z, wt * a.w));
      }
      s = wave_sum(s);
    }
    if (lane == j) {
      my_dw = s;
      my_w = wt;
    }
  }
  float sw = 0.f;
  for (int j = 0; j < k; ++j) sw = fmaf(__shfl(my_w, j, kWave), __shfl(my_dw, j, kWave), sw);
  if (lane < k) dl_sel[(int64_t)t * k + lane] = my_w * (my_dw - sw);
}

// dX[t, c] = sum over kept slots j of dX_perm[dest[t,j], c], then
// + sum over slots j of dl[t,j] W_r[idx[t,j], c] (both in slot order).  One
// wavefront per (token, 512-column slice); each lane 8 columns.
__global__ __launch_bounds__(256) void bwd_gather_kernel(
    const float* __restrict__ dX_perm, const int32_t* __restrict__ dest,
    const int32_t* __restrict__ idx, const float* __restrict__ dl_sel,
    const float* __restrict__ W_r, int T, int d, int k, float* __restrict__ dX) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  const int c0 = blockIdx.y * 512 + lane * 8;
  if (c0 >= d) return;  // d % 8 == 0: all 8 columns are in range
  float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
  for (int j = 0; j < k; ++j) {
    const int r = dest[(int64_t)t * k + j];
    if (r < 0) continue;
    const float4* p = reinterpret_cast<const float4*>(dX_perm + (int64_t)r * d + c0);
    const float4 u = p[0], v = p[1];
    a0.x += u.x; a0.y += u.y; a0.z += u.z; a0.w += u.w;
    a1.x += v.x; a1.y += v.y; a1.z += v.z; a1.w += v.w;
  }
  for (int j = 0; j < k; ++j) {
    const float l = dl_sel[(int64_t)t * k + j];
    const float4* p =
        reinterpret_cast<const float4*>(W_r + (int64_t)idx[(int64_t)t * k + j] * d + c0);
    const float4 u = p[0], v = p[1];
    a0.x = fmaf(l, u.x, a0.x); a0.y = fmaf(l, u.y, a0.y);
    a0.z = fmaf(l, u.z, a0.z); a0.w = fmaf(l, u.w, a0.w);
    a1.x = fmaf(l, v.x, a1.x); a1.y = fmaf(l, v.y, a1.y);
    a1.z = fmaf(l, v.z, a1.z); a1.w = fmaf(l, v.w, a1.w);
  }
  float4* o = reinterpret_cast<float4*>(dX + (int64_t)t * d + c0);
  o[0] = a0;
  o[1] = a1;
}

// dW_r[e, c] = sum_t dl[t, e] X[t, c] and dbias[e] = sum_t dl[t, e], with dl
// the sparse logit gradient (dl_sel at the selected ids).  Block: 256
// columns x ET experts; each thread one column and ET accumulators.  Tokens
// go 32 at a time: the block scatters their selections into a dense
// [32 x ET] LDS tile, then every thread runs the tile in token order.
template <int ET>
__global__ __launch_bounds__(256) void router_wgrad_kernel(
    const uint16_t* __restrict__ X, const int32_t* __restrict__ idx,
    const float* __restrict__ dl_sel, int T, int d, int E, int k,
    float* __restrict__ dW_r, float* __restrict__ dbias) {
  constexpr int TT = 32;
  __shared__ float s_dl[TT][ET];
  const int tid = threadIdx.x;
  const int c = blockIdx.x * 256 + tid;
  const int e0 = blockIdx.y * ET;
  float acc[ET];
#pragma unroll
  for (int i = 0; i < ET; ++i) acc[i] = 0.f;
  float bacc = 0.f;
  for (int t0 = 0; t0 < T; t0 += TT) {
    for (int i = tid; i < TT * ET; i += 256) (&s_dl[0][0])[i] = 0.f;
    __syncthreads();
    const int nt = min(TT, T - t0);
    for (int p = tid; p < nt * k; p += 256) {
      const int64_t q = (int64_t)t0 * k + p;
      const int e = idx[q] - e0;
      if (e >= 0 && e < ET) s_dl[p / k][e] = dl_sel[q];  // ids of a token are distinct
    }
    __syncthreads();
    if (c < d) {
      for (int tl = 0; tl < nt; ++tl) {
        const float x = bf16_bits_to_f32(X[(int64_t)(t0 + tl) * d + c]);
#pragma unroll
        for (int i = 0; i < ET; ++i) acc[i] = fmaf(s_dl[tl][i], x, acc[i]);
      }
    }
    if (blockIdx.x == 0 && tid < ET)
      for (int tl = 0; tl < nt; ++tl) bacc += s_dl[tl][tid];
    __syncthreads();
  }
  if (c < d) {
#pragma unroll
    for (int i = 0; i < ET; ++i)
      if (e0 + i < E) dW_r[(int64_t)(e0 + i) * d + c] = acc[i];
  }
  if (dbias != nullptr && blockIdx.x == 0 && tid < ET && e0 + tid < E) dbias[e0 + tid] = bacc;
}

// 64 x 64 tile transpose through LDS (bf16).  Source: rows i < 64 at
// src_rows + i * C (rows i >= nrows read as zero), columns [c0, c0 + 64) of
// C.  Destination: dst[(c0 + c) * ldo + i] for i < nout and c0 + c < C.
// C, ldo and the destination's column offset are multiples of 8, so every
// access is one 16-byte chunk.
__device__ __forceinline__ void transpose_tile(const uint16_t* __restrict__ src_rows,
                                               int nrows, int C, int c0,
                                               uint16_t* __restrict__ dst, int64_t ldo,
                                               int nout) {
  __shared__ uint16_t s[64][66];
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = tid + 256 * h;
    const int row = p / 8, cc = (p % 8) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < nrows && c0 + cc < C)
      v = *reinterpret_cast<const uint4*>(src_rows + (int64_t)row * C + c0 + cc);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[row][cc + 2 * i] = (uint16_t)(w[i] & 0xFFFF);
      s[row][cc + 2 * i + 1] = (uint16_t)(w[i] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = tid + 256 * h;
    const int oc = p / 8, rc = (p % 8) * 8;
    if (c0 + oc >= C || rc >= nout) continue;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)s[rc + 2 * i][oc] | ((uint32_t)s[rc + 2 * i + 1][oc] << 16);
    *reinterpret_cast<uint4*>(dst + (int64_t)(c0 + oc) * ldo + rc) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Batched weight transpose: src [B, R, C] -> dst[b] [C, ldo] at column
// offset co (dst[b][c][co + r] = src[b][r][c]).  Grid (C/64, R/64, B).
__global__ __launch_bounds__(256) void transpose_weights_kernel(
    const uint16_t* __restrict__ src, int R, int C, uint16_t* __restrict__ dst,
    int ldo, int co) {
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int64_t b = blockIdx.z;
  transpose_tile(src + (b * R + r0) * (int64_t)C, min(64, R - r0), C, c0,
                 dst + b * (int64_t)C * ldo + co + r0, ldo, min(64, R - r0));
}

// Padded expert offsets: poff[e + 1] = poff[e] + roundup(rows of e, 64).
__global__ __launch_bounds__(256) void pad_offsets_kernel(const int32_t* __restrict__ offsets,
                                                          int E, int32_t* __restrict__ poff) {
  __shared__ int32_t s[256];
  const int e = threadIdx.x;
  s[e] = e < E ? (offsets[e + 1] - offsets[e] + 63) / 64 * 64 : 0;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = e >= o ? s[e - o] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  if (e == 0) poff[0] = 0;
  if (e < E) poff[e + 1] = s[e];
}

// Rows grouped by expert -> transposed, padded segments: dst[c][p] for p in
// [poff[e], poff[e + 1]) is src[offsets[e] + p - poff[e]][c], zero past the
// expert's rows.  Grid (ld / 64, C / 64); a 64-column block of dst lies in
// one expert's segment (segments are multiples of 64 wide).
__global__ __launch_bounds__(256) void transpose_segments_kernel(
    const uint16_t* __restrict__ src, int C, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ poff, int E, uint16_t* __restrict__ dst, int ld) {
  const int p0 = blockIdx.x * 64;
  if (p0 >= poff[E]) return;
  int lo = 0, hi = E;  // poff[lo] <= p0 < poff[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (poff[mid] <= p0) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int r0 = offsets[e] + (p0 - poff[e]);
  const int nrows = max(0, min(64, offsets[e + 1] - r0));
  transpose_tile(src + (int64_t)r0 * C, nrows, C, blockIdx.y * 64, dst + p0, ld, 64);
}

}  // namespace

hipError_t launch_bwd_combine(const float* dout, const float* Y_perm, const int32_t* dest,
                              const float* topk_w, int T, int d, int k, void* dY_perm,
                              float* dl_sel, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  bwd_combine_kernel<<<(T + kTokPerBlock - 1) / kTokPerBlock, 256, 0, stream>>>(
      dout, Y_perm, dest, topk_w, T, d, k, static_cast<uint16_t*>(dY_perm), dl_sel);
  return hipGetLastError();
}

hipError_t launch_bwd_gather(const float* dX_perm, const int32_t* dest, const int32_t* idx,
                             const float* dl_sel, const float* W_r, int T, int d, int k,
                             float* dX, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + kTokPerBlock - 1) / kTokPerBlock, (d + 511) / 512);
  bwd_gather_kernel<<<grid, 256, 0, stream>>>(dX_perm, dest, idx, dl_sel, W_r, T, d, k, dX);
  return hipGetLastError();
}

hipError_t launch_router_wgrad(const void* X, const int32_t* idx, const float* dl_sel, int T,
                               int d, int E, int k, float* dW_r, float* dbias,
                               hipStream_t stream) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const unsigned gx = (d + 255) / 256;
  if (E <= 8) {
    router_wgrad_kernel<8><<<dim3(gx, 1), 256, 0, stream>>>(x, idx, dl_sel, T, d, E, k, dW_r, dbias);
  } else if (E <= 32) {
    router_wgrad_kernel<32><<<dim3(gx, 1), 256, 0, stream>>>(x, idx, dl_sel, T, d, E, k, dW_r, dbias);
  } else {
    router_wgrad_kernel<64><<<dim3(gx, (E + 63) / 64), 256, 0, stream>>>(x, idx, dl_sel, T, d, E,
                                                                         k, dW_r, dbias);
  }
  return hipGetLastError();
}

hipError_t launch_transpose_weights(const void* src, int B, int R, int C, void* dst, int ldo,
                                    int co, hipStream_t stream) {
  const dim3 grid((C + 63) / 64, (R + 63) / 64, B);
  transpose_weights_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(src), R, C,
                                                    static_cast<uint16_t*>(dst), ldo, co);
  return hipGetLastError();
}

hipError_t launch_pad_offsets(const int32_t* offsets, int E, int32_t* poff, hipStream_t stream) {
  pad_offsets_kernel<<<1, 256, 0, stream>>>(offsets, E, poff);
  return hipGetLastError();
}

hipError_t launch_transpose_segments(const void* src, int C, const int32_t* offsets,
                                     const int32_t* poff, int E, void* dst, int ld,
                                     hipStream_t stream) {
  const dim3 grid(ld / 64, (C + 63) / 64);
  transpose_segments_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(src), C,
                                                     offsets, poff, E,
                                                     static_cast<uint16_t*>(dst), ld);
  return hipGetLastError();
}

}  // namespace moe
