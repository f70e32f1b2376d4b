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

constexpr int kMaxWavesPerBlock = 4;
constexpr int kColsPerWave = 8 * kWave;  // 8 columns per lane

// One wavefront per (token, slice of kColsPerWave columns).  A workgroup
// holds wpb consecutive slices of one token (wpb divides the slice count, so
// no wave is idle), and consecutive workgroups walk a token's row before the
// next token: the k source rows of a token are read whole, one after the
// other, instead of one slice of many tokens' rows at a time (measured:
// DeepSeek-V3 combine 199 -> 185 us, Qwen3 capacity 86 -> 68, gpt-oss 88 ->
// 83, Mixtral 41 -> 37).  A slice is 128 chunks of four fp32 columns; lane l owns chunks l and
// l + 64, so every load and store instruction of the wave covers 1 KB of
// contiguous memory.  The k
// source rows are read eight slots at a time (all loads issued before the
// FMAs, which run in slot order); each source row is read once, past the
// caches (non-temporal).  The token's destination rows and gate weights are
// the same for the whole wavefront: scalar loads fetch them, so the row
// loads start without a round trip through the LDS.
template <bool OUT_BF16>
__global__ __launch_bounds__(kMaxWavesPerBlock * kWave) void combine_kernel(
    const float* __restrict__ Y, const float* __restrict__ Y2,
    const int32_t* __restrict__ dest_row, const float* __restrict__ topk_w, int T, int d,
    int k, int groups, const float* __restrict__ add_rows, void* __restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t = blockIdx.x / groups;  // groups = slices per token / waves per block
  const int slice = (blockIdx.x - t * groups) * (blockDim.x / kWave) + wv;
  if (t >= T) return;  // uniform per wavefront; no block-wide barrier below
  // the token's (row, weight) pairs: the same for the whole wavefront
  const int32_t* __restrict__ td = dest_row + (int64_t)t * k;
  const float* __restrict__ tw = topk_w + (int64_t)t * k;
  const int nq = d / 4;                                // chunks of 4 columns per row
  const int q0 = slice * (2 * kWave) + lane;           // this lane's chunks: q0, q1
  const int q1 = q0 + kWave;
  if (q0 >= nq) return;
  const bool has1 = q1 < nq;
  f32x4 acc0, acc1;
  if (add_rows != nullptr) {
    const f32x4* a0 = reinterpret_cast<const f32x4*>(add_rows + (int64_t)t * d);
    acc0 = a0[q0];
    acc1 = has1 ? a0[q1] : f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1 = acc0;
  }
  for (int j0 = 0; j0 < k; j0 += 8) {
    f32x4 a[8], b[8];
    int r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      r[u] = (j0 + u < k) ? td[j0 + u] : -1;
      if (r[u] >= 0) {
        const f32x4* src = reinterpret_cast<const f32x4*>(Y + (int64_t)r[u] * d);
        a[u] = __builtin_nontemporal_load(src + q0);
        b[u] = has1 ? __builtin_nontemporal_load(src + q1) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    if (Y2 != nullptr) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (r[u] < 0) continue;
        const f32x4* src = reinterpret_cast<const f32x4*>(Y2 + (int64_t)r[u] * d);
        const f32x4 a2 = __builtin_nontemporal_load(src + q0);
        const f32x4 b2 = has1 ? __builtin_nontemporal_load(src + q1) : f32x4{0.f, 0.f, 0.f, 0.f};
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
      const float w = tw[j0 + u];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc0[i] = fmaf(w, a[u][i], acc0[i]);
        acc1[i] = fmaf(w, b[u][i], acc1[i]);
      }
    }
  }
  if constexpr (OUT_BF16) {
    uint2* o = reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (int64_t)t * d);
    auto pack = [](f32x4 v) {
      return uint2{(uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16),
                   (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16)};
    };
    o[q0] = pack(acc0);
    if (has1) o[q1] = pack(acc1);
  } else {
    f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(out) + (int64_t)t * d);
    o[q0] = acc0;
    if (has1) o[q1] = acc1;
  }
}

}  // namespace

hipError_t launch_combine(const float* Y_perm, const int32_t* dest_row,
                          const float* topk_w, int T, int d, int k,
                          const float* add_rows, bool out_bf16, void* out,
                          hipStream_t stream, const float* Y_half) {
  if (T == 0) return hipSuccess;
  const int nslices = (d + kColsPerWave - 1) / kColsPerWave;
  int wpb = kMaxWavesPerBlock;  // waves per block: the largest divisor of the slice count
  while (nslices % wpb != 0) --wpb;
  const int groups = nslices / wpb;
  const int64_t blocks = (int64_t)T * groups;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (out_bf16)
    combine_kernel<true><<<(unsigned)blocks, wpb * kWave, 0, stream>>>(Y_perm, Y_half, dest_row, topk_w, T, d, k, groups, add_rows, out);
  else
    combine_kernel<false><<<(unsigned)blocks, wpb * kWave, 0, stream>>>(Y_perm, Y_half, dest_row, topk_w, T, d, k, groups, add_rows, out);
  return hipGetLastError();
}

}  // namespace moe
