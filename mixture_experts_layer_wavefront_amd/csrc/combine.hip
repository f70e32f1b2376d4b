// Combine: un-permute the expert outputs and add them with the gate weights,
// out[t] = sum_{j ascending, dest_row[t,j] >= 0} topk_w[t,j] * Y_perm[dest_row[t,j]].
//
// Method: "Sparsely-Gated MoE 구현 관점에서 살펴보기: Router, Top-k, 부하 분산"
// (molayo1419.me), section "Router를 텐서 형태에서 추적하기" (the layer output
// is the weighted sum of the selected experts' outputs; unselected experts
// add nothing) and forward-pipeline step 5 (un-permute, combine with the
// router weights, original token order).
//
// A gather-reduce rather than a scatter-add: each slice of an output row is
// owned by one wavefront that reads its k source rows and adds them in slot
// order, so the sum order is fixed and no atomics are needed.  fp32
// accumulation, one rounding at the store.  When the down projection ran as
// two K halves, Y2 holds the second half's partial sums and each source row
// is Y[r] + Y2[r] (the same fp32 add the grouped FFN's own sum performs).
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kTokPerBlock = 4;
constexpr int kColsPerWave = 8 * kWave;  // 8 columns per lane

// One wavefront per (token, slice of kColsPerWave columns): blockIdx.x picks
// kTokPerBlock tokens, blockIdx.y the column slice.  The k source rows are
// read eight slots at a time (all loads issued before the FMAs, which run in
// slot order).
template <bool OUT_BF16>
__global__ __launch_bounds__(kTokPerBlock * kWave) void combine_kernel(
    const float* __restrict__ Y, const float* __restrict__ Y2,
    const int32_t* __restrict__ dest_row, const float* __restrict__ topk_w, int T, int d,
    int k, const float* __restrict__ add_rows, void* __restrict__ out) {
  __shared__ int32_t s_dest[kTokPerBlock][32];
  __shared__ float s_w[kTokPerBlock][32];
  const int lane = threadIdx.x % kWave;
  const int wv = threadIdx.x / kWave;
  const int t = blockIdx.x * kTokPerBlock + wv;
  if (t >= T) return;  // uniform per wavefront; no block-wide barrier below
  // the token's (row, weight) pairs go through LDS: lanes past the row's end
  // are idle when d is small, so cross-lane shuffles could read inactive lanes
  if (lane < k) {
    s_dest[wv][lane] = dest_row[(int64_t)t * k + lane];
    s_w[wv][lane] = topk_w[(int64_t)t * k + lane];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const int c = blockIdx.y * kWave + lane;  // 8-column chunk
  if (c >= d / 8) return;
  float acc[8];
  if (add_rows != nullptr) {
    const f32x4* a0 = reinterpret_cast<const f32x4*>(add_rows + (int64_t)t * d) + 2 * c;
    const f32x4 u = a0[0], v = a0[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] = u[i];
      acc[4 + i] = v[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  }
  for (int j0 = 0; j0 < k; j0 += 8) {
    f32x4 a[8], b[8];
    int r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      r[u] = (j0 + u < k) ? s_dest[wv][j0 + u] : -1;
      if (r[u] >= 0) {
        const f32x4* src = reinterpret_cast<const f32x4*>(Y + (int64_t)r[u] * d) + 2 * c;
        a[u] = src[0];
        b[u] = src[1];
      }
    }
    if (Y2 != nullptr) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (r[u] < 0) continue;
        const f32x4* src = reinterpret_cast<const f32x4*>(Y2 + (int64_t)r[u] * d) + 2 * c;
        const f32x4 a2 = src[0], b2 = src[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[u][i] = a[u][i] + a2[i];
          b[u][i] = b[u][i] + b2[i];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (r[u] < 0) continue;
      const float w = s_w[wv][j0 + u];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] = fmaf(w, a[u][i], acc[i]);
        acc[4 + i] = fmaf(w, b[u][i], acc[4 + i]);
      }
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

}  // namespace

hipError_t launch_combine(const float* Y_perm, const int32_t* dest_row,
                          const float* topk_w, int T, int d, int k,
                          const float* add_rows, bool out_bf16, void* out,
                          hipStream_t stream, const float* Y_half) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + kTokPerBlock - 1) / kTokPerBlock, (d + kColsPerWave - 1) / kColsPerWave);
  if (out_bf16)
    combine_kernel<true><<<grid, kTokPerBlock * kWave, 0, stream>>>(Y_perm, Y_half, dest_row, topk_w, T, d, k, add_rows, out);
  else
    combine_kernel<false><<<grid, kTokPerBlock * kWave, 0, stream>>>(Y_perm, Y_half, dest_row, topk_w, T, d, k, add_rows, out);
  return hipGetLastError();
}

}  // namespace moe
