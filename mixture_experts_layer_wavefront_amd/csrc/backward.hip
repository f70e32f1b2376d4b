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
// The expert GEMMs (dgrad and wgrad) run on the grouped GEMM kernel, which
// reads the weights and the saved activations as stored.  Every sum runs in
// a fixed order, so the same inputs give the same bits.
#include "common.h"

#include <algorithm>

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

// dX[t, c] = sum over kept slots j of (P0 + P1)[dest[t,j], c], then
// + sum over slots j of dl[t,j] W_r[idx[t,j], c] (both in slot order), with
// P0 = dX_perm and P1 = dX_perm + R d the two K halves of the experts' data
// gradient.  One wavefront per (token, 512-column slice); each lane 8
// columns.
__global__ __launch_bounds__(256) void bwd_gather_kernel(
    const float* __restrict__ dX_perm, int64_t R, const int32_t* __restrict__ dest,
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
    const float4* p2 = reinterpret_cast<const float4*>(dX_perm + (R + r) * d + c0);
    const float4 u = p[0], v = p[1], u2 = p2[0], v2 = p2[1];
    a0.x += u.x + u2.x; a0.y += u.y + u2.y; a0.z += u.z + u2.z; a0.w += u.w + u2.w;
    a1.x += v.x + v2.x; a1.y += v.y + v2.y; a1.z += v.z + v2.z; a1.w += v.w + v2.w;
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
// the sparse logit gradient (dl_sel at the selected ids), in two passes.
// Pass 1: block (column slice of 256, ET experts, token chunk s) sums its
// chunk's tokens in order into part[s] ([E, d], and [E] for the bias): each
// thread one column and ET accumulators; tokens go 32 at a time, their
// selections scattered into a dense [32 x ET] LDS tile first.  Pass 2 adds
// the chunks' partial sums in chunk order.
template <int ET>
__global__ __launch_bounds__(256) void router_wgrad_part_kernel(
    const uint16_t* __restrict__ X, const int32_t* __restrict__ idx,
    const float* __restrict__ dl_sel, int T, int d, int E, int k, int chunk,
    float* __restrict__ part, float* __restrict__ part_b) {
  constexpr int TT = 32;
  __shared__ float s_dl[TT][ET];
  const int tid = threadIdx.x;
  const int c = blockIdx.x * 256 + tid;
  const int e0 = blockIdx.y * ET;
  const int s = blockIdx.z;
  const int t_beg = s * chunk, t_end = min(T, t_beg + chunk);
  float acc[ET];
#pragma unroll
  for (int i = 0; i < ET; ++i) acc[i] = 0.f;
  float bacc = 0.f;
  for (int t0 = t_beg; t0 < t_end; t0 += TT) {
    for (int i = tid; i < TT * ET; i += 256) (&s_dl[0][0])[i] = 0.f;
    __syncthreads();
    const int nt = min(TT, t_end - t0);
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
  float* ps = part + (int64_t)s * E * d;
  if (c < d) {
#pragma unroll
    for (int i = 0; i < ET; ++i)
      if (e0 + i < E) ps[(int64_t)(e0 + i) * d + c] = acc[i];
  }
  if (blockIdx.x == 0 && tid < ET && e0 + tid < E) part_b[(int64_t)s * E + e0 + tid] = bacc;
}

__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ part_b, int S, int E, int d,
    float* __restrict__ dW_r, float* __restrict__ dbias) {
  const int64_t n = (int64_t)E * d;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += part[(int64_t)s * n + i];
    dW_r[i] = v;
  }
  if (dbias != nullptr && blockIdx.x == 0 && threadIdx.x < E) {
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += part_b[(int64_t)s * E + threadIdx.x];
    dbias[threadIdx.x] = v;
  }
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

hipError_t launch_bwd_gather(const float* dX_perm, int64_t R, const int32_t* dest,
                             const int32_t* idx, const float* dl_sel, const float* W_r, int T,
                             int d, int k, float* dX, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + kTokPerBlock - 1) / kTokPerBlock, (d + 511) / 512);
  bwd_gather_kernel<<<grid, 256, 0, stream>>>(dX_perm, R, dest, idx, dl_sel, W_r, T, d, k, dX);
  return hipGetLastError();
}

int router_wgrad_chunks(int T, int d, int E) {
  const int et = E <= 8 ? 8 : (E <= 32 ? 32 : 64);
  const int blocks = ((d + 255) / 256) * ((E + et - 1) / et);
  const int max_chunks = (T + 31) / 32;
  return std::max(1, std::min(max_chunks, (1024 + blocks - 1) / blocks));
}

size_t router_wgrad_scratch_bytes(int T, int d, int E) {
  const size_t S = (size_t)router_wgrad_chunks(T, d, E);
  return S * E * d * 4 + ((S * E * 4 + 255) & ~size_t(255));
}

hipError_t launch_router_wgrad(const void* X, const int32_t* idx, const float* dl_sel, int T,
                               int d, int E, int k, float* dW_r, float* dbias, void* scratch,
                               hipStream_t stream) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const int S = router_wgrad_chunks(T, d, E);
  const int chunk = ((T + S - 1) / S + 31) / 32 * 32;
  float* part_b = static_cast<float*>(scratch);
  float* part = part_b + ((size_t)S * E + 63) / 64 * 64;
  const unsigned gx = (d + 255) / 256;
  if (E <= 8) {
    router_wgrad_part_kernel<8><<<dim3(gx, 1, S), 256, 0, stream>>>(x, idx, dl_sel, T, d, E, k,
                                                                   chunk, part, part_b);
  } else if (E <= 32) {
    router_wgrad_part_kernel<32><<<dim3(gx, 1, S), 256, 0, stream>>>(x, idx, dl_sel, T, d, E, k,
                                                                    chunk, part, part_b);
  } else {
    router_wgrad_part_kernel<64><<<dim3(gx, (E + 63) / 64, S), 256, 0, stream>>>(
        x, idx, dl_sel, T, d, E, k, chunk, part, part_b);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t n = (int64_t)E * d;
  router_wgrad_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(part, part_b, S, E,
                                                                             d, dW_r, dbias);
  return hipGetLastError();
}

}  // namespace moe
