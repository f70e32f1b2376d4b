// Router: logits l = X W_r^T (+ bias) in fp32, top-k per token by
// wavefront-wide argmax rounds, then the gate weights.
//
// Method: "Sparsely-Gated MoE 구현 관점에서 살펴보기: Router, Top-k, 부하 분산"
// (molayo1419.me), sections "Router를 텐서 형태에서 추적하기" (T x E
// logits from X @ W_r^T), "Top-2 라우팅의 수치 예시" (top-k; the selected
// logits renormalised by a softmax, or a softmax over all experts followed
// by top-k and renormalisation) and "pure Python으로 Top-k Router
// 확인하기" (the largest selected logit is subtracted before exponentiating).
//
// One workgroup (4 wavefronts) owns TT tokens and all E <= 256 experts.  The
// [TT x E] logit tile is accumulated in registers from LDS-staged fp32
// slices of X and W_r, then parked in LDS; it never goes to HBM.  Each
// wavefront then takes one token at a time: every lane holds up to four of
// the E logits, and k rounds of a 64-lane butterfly argmax (ties to the
// lower expert id) pick the experts in descending-logit order.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;
constexpr int kRouterDK = 32;

template <typename XT>
struct XLoad;
template <>
struct XLoad<float> {
  static constexpr int VE = 4;  // elements per 16-byte chunk
  __device__ static void load(const float* p, float* out) {
    f32x4 v = *reinterpret_cast<const f32x4*>(p);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  }
};
template <>
struct XLoad<uint16_t> {
  static constexpr int VE = 8;
  __device__ static void load(const uint16_t* p, float* out) {
    i32x4 v = *reinterpret_cast<const i32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w = (uint32_t)v[i];
      out[2 * i] = __uint_as_float(w << 16);
      out[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u);
    }
  }
};

// TX threads across experts (expert e = tx + TX*j, j < RE), TY = 256/TX
// threads across tokens (token row = ty + TY*i, i < RT).
template <int TX, int RE, int RT, typename XT>
__global__ __launch_bounds__(kRouterThreads) void router_topk_kernel(
    const XT* __restrict__ X, const float* __restrict__ W_r,
    const float* __restrict__ bias, int T, int d, int E, int k, int gating,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  constexpr int TY = kRouterThreads / TX;
  constexpr int TT = TY * RT;
  constexpr int EP = TX * RE;
  constexpr int DK = kRouterDK;
  constexpr int VE = XLoad<XT>::VE;
  constexpr int CPR = DK / VE;  // 16-byte chunks per X row slice
  constexpr int VPL = (EP + kWave - 1) / kWave;

  __shared__ float Xs[DK][TT + 1];
  __shared__ float Ws[DK][EP + 1];
  __shared__ float Ls[TT][EP + 1];

  const int tid = threadIdx.x;
  const int tx = tid % TX;
  const int ty = tid / TX;
  const int t0 = blockIdx.x * TT;

  float acc[RT][RE];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < RE; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < d; k0 += DK) {
    // stage X[t0:t0+TT, k0:k0+DK] transposed into Xs (zero outside)
    for (int c = tid; c < TT * CPR; c += kRouterThreads) {
      const int row = c / CPR, kc = c % CPR;
      const int t = t0 + row, kk = k0 + kc * VE;
      float v[VE];
      if (t < T && kk < d) {
        XLoad<XT>::load(X + (int64_t)t * d + kk, v);
      } else {
#pragma unroll
        for (int i = 0; i < VE; ++i) v[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < VE; ++i) Xs[kc * VE + i][row] = v[i];
    }
    // stage W_r[:, k0:k0+DK] transposed into Ws (zero outside)
    for (int c = tid; c < EP * (DK / 4); c += kRouterThreads) {
      const int e = c / (DK / 4), kc = c % (DK / 4);
      const int kk = k0 + kc * 4;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (e < E && kk < d) v = *reinterpret_cast<const f32x4*>(W_r + (int64_t)e * d + kk);
#pragma unroll
      for (int i = 0; i < 4; ++i) Ws[kc * 4 + i][e] = v[i];
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < DK; ++kk) {
      float xv[RT], wv[RE];
#pragma unroll
      for (int i = 0; i < RT; ++i) xv[i] = Xs[kk][ty + TY * i];
#pragma unroll
      for (int j = 0; j < RE; ++j) wv[j] = Ws[kk][tx + TX * j];
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < RE; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }

  // logits (+ bias, an fp32 add) into LDS
#pragma unroll
  for (int j = 0; j < RE; ++j) {
    const int e = tx + TX * j;
    const float b = (bias != nullptr && e < E) ? bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < RT; ++i) Ls[ty + TY * i][e] = acc[i][j] + b;
  }
  __syncthreads();

  const int lane = tid % kWave;
  const int wave = tid / kWave;
  for (int row = wave; row < TT; row += kRouterThreads / kWave) {
    const int t = t0 + row;
    if (t >= T) break;
    float v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + kWave * i;
      v[i] = (e < E) ? Ls[row][e] : -INFINITY;
    }
    float my_s = -INFINITY;
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
      float bv = v[0];
      int be = lane;
#pragma unroll
      for (int i = 1; i < VPL; ++i)
        if (v[i] > bv) { bv = v[i]; be = lane + kWave * i; }
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oe = __shfl_xor(be, o, kWave);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      if (lane == j) { my_s = bv; my_id = be; }
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (be == lane + kWave * i) v[i] = -INFINITY;
    }
    const float m = __shfl(my_s, 0, kWave);  // the largest logit of the token
    float w;
    if (gating == 0) {
      const float ex = (lane < k) ? expf(my_s - m) : 0.f;
      w = ex / wave_sum(ex);
    } else {
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + kWave * i;
        if (e < E) z += expf(Ls[row][e] - m);
      }
      const float Z = wave_sum(z);
      const float p = (lane < k) ? expf(my_s - m) / Z : 0.f;
      w = p / wave_sum(p);
    }
    if (lane < k) {
      topk_idx[(int64_t)t * k + lane] = my_id;
      topk_w[(int64_t)t * k + lane] = w;
    }
  }
}

template <int TX, int RE, int RT>
hipError_t launch_cfg(const void* X, bool x_bf16, const float* W_r,
                      const float* bias, int T, int d, int E, int k, int gating,
                      int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  constexpr int TT = (kRouterThreads / TX) * RT;
  const dim3 grid((T + TT - 1) / TT);
  if (x_bf16)
    router_topk_kernel<TX, RE, RT, uint16_t><<<grid, kRouterThreads, 0, stream>>>(
        static_cast<const uint16_t*>(X), W_r, bias, T, d, E, k, gating, topk_idx, topk_w);
  else
    router_topk_kernel<TX, RE, RT, float><<<grid, kRouterThreads, 0, stream>>>(
        static_cast<const float*>(X), W_r, bias, T, d, E, k, gating, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const void* X, bool x_bf16, const float* W_r,
                        const float* bias, int T, int d, int E, int k,
                        int gating, int32_t* topk_idx, float* topk_w,
                        hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (E <= 8) return launch_cfg<8, 1, 1>(X, x_bf16, W_r, bias, T, d, E, k, gating, topk_idx, topk_w, stream);
  if (E <= 16) return launch_cfg<16, 1, 1>(X, x_bf16, W_r, bias, T, d, E, k, gating, topk_idx, topk_w, stream);
  if (E <= 32) return launch_cfg<32, 1, 2>(X, x_bf16, W_r, bias, T, d, E, k, gating, topk_idx, topk_w, stream);
  if (E <= 64) return launch_cfg<64, 1, 4>(X, x_bf16, W_r, bias, T, d, E, k, gating, topk_idx, topk_w, stream);
  if (E <= 128) return launch_cfg<64, 2, 4>(X, x_bf16, W_r, bias, T, d, E, k, gating, topk_idx, topk_w, stream);
  return launch_cfg<64, 4, 4>(X, x_bf16, W_r, bias, T, d, E, k, gating, topk_idx, topk_w, stream);
}

}  // namespace moe
