// Combine: un-permute the expert outputs and add them with the gate weights,
// out[t] = sum_{j ascending, dest_row[t,j] >= 0} topk_w[t,j] * Y_perm[dest_row[t,j]].
//
// Method: "Sparsely-Gated MoE 구현 관점에서 살펴보기: Router, Top-k, 부하 분산"
// (molayo1419.me), section "Router를 텐서 형태에서 추적하기" (the layer output
// is the weighted sum of the selected experts' outputs; unselected experts
// add nothing) and forward-pipeline step 5 (un-permute, combine with the
// router weights, original token order).
//
// A gather-reduce rather than a scatter-add: each output row is owned by one
// wavefront that reads its k source rows in slot order, so the sum order is
// fixed and no atomics are needed.  fp32 accumulation, one rounding at the
// store.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kTokPerBlock = 4;

template <bool OUT_BF16>
__global__ __launch_bounds__(kTokPerBlock * kWave) void combine_kernel(
    const float* __restrict__ Y, const int32_t* __restrict__ dest_row,
    const float* __restrict__ topk_w, int T, int d, int k,
    void* __restrict__ out) {
  __shared__ int32_t s_dest[kTokPerBlock][32];
  __shared__ float s_w[kTokPerBlock][32];
  const int lane = threadIdx.x % kWave;
  const int wv = threadIdx.x / kWave;
  const int t = blockIdx.x * kTokPerBlock + wv;
  if (t >= T) return;  // uniform per wavefront; no block-wide barrier below
  // the token's (row, weight) pairs go through LDS: the column loop below
  // leaves lanes idle when d/8 < 64, so cross-lane shuffles there would read
  // inactive lanes
  if (lane < k) {
    s_dest[wv][lane] = dest_row[(int64_t)t * k + lane];
    s_w[wv][lane] = topk_w[(int64_t)t * k + lane];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  // 8 columns per lane step: two 16-byte fp32 loads per source row
  const int nchunk = d / 8;
  for (int c = lane; c < nchunk; c += kWave) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = s_dest[wv][j];
      const float w = s_w[wv][j];
      if (r < 0) continue;
      const f32x4* src = reinterpret_cast<const f32x4*>(Y + (int64_t)r * d) + 2 * c;
      const f32x4 a = src[0], b = src[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] = fmaf(w, a[i], acc[i]);
        acc[4 + i] = fmaf(w, b[i], acc[4 + i]);
      }
    }
    if constexpr (OUT_BF16) {
      i32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = (int)((uint32_t)f32_to_bf16_bits(acc[2 * i]) |
                     ((uint32_t)f32_to_bf16_bits(acc[2 * i + 1]) << 16));
      reinterpret_cast<i32x4*>(static_cast<uint16_t*>(out) + (int64_t)t * d)[c] = o;
    } else {
      f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(out) + (int64_t)t * d) + 2 * c;
      dst[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
      dst[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
  }
}

}  // namespace

hipError_t launch_combine(const float* Y_perm, const int32_t* dest_row,
                          const float* topk_w, int T, int d, int k,
                          bool out_bf16, void* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + kTokPerBlock - 1) / kTokPerBlock);
  if (out_bf16)
    combine_kernel<true><<<grid, kTokPerBlock * kWave, 0, stream>>>(Y_perm, dest_row, topk_w, T, d, k, out);
  else
    combine_kernel<false><<<grid, kTokPerBlock * kWave, 0, stream>>>(Y_perm, dest_row, topk_w, T, d, k, out);
  return hipGetLastError();
}

}  // namespace moe
