// Wavefront top-k and gate weights of one token's router logits, shared by
// the router's selection kernels and the few-token routing-and-assignment
// kernel.  "Sparsely-Gated MoE 구현 관점에서 살펴보기" (molayo1419.me),
// sections "Top-2 라우팅의 수치 예시" (top-k; softmax over the selected
// logits, or over all experts followed by renormalisation over the selected
// ones) and "pure Python으로 Top-k Router 확인하기" (the largest logit is
// subtracted before exponentiating).
#pragma once

#include "common.h"

namespace moe {

// All-lane reductions over a wavefront whose result does not depend on the
// reduction tree (a maximum; an argmax under the total order "larger value,
// then lower id"): lanes 1, 2 apart and the mirrored halves of 8 and 16
// lanes through DPP moves, then 16 and 32 apart through cross-lane
// permutes, so each step costs a few cycles instead of an LDS round trip.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ void argmax_take(float& bv, int& be, float ov, int oe) {
  if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
}
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& bv, int& be) {
  const float ov = __int_as_float(dpp_mov<CTRL>(__float_as_int(bv)));
  const int oe = dpp_mov<CTRL>(be);
  argmax_take(bv, be, ov, oe);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane l of 8 <- 7 - l
constexpr int kDppMirror = 0x140;      // lane l of 16 <- 15 - l
__device__ __forceinline__ void wave_argmax(float& bv, int& be) {
  argmax_dpp<kDppXor1>(bv, be);
  argmax_dpp<kDppXor2>(bv, be);
  argmax_dpp<kDppHalfMirror>(bv, be);
  argmax_dpp<kDppMirror>(bv, be);
#pragma unroll
  for (int o = 16; o < kWave; o <<= 1) argmax_take(bv, be, __shfl_xor(bv, o, kWave), __shfl_xor(be, o, kWave));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, __int_as_float(dpp_mov<kDppXor1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_mov<kDppXor2>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_mov<kDppHalfMirror>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_mov<kDppMirror>(__float_as_int(v))));
#pragma unroll
  for (int o = 16; o < kWave; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Top-k of one token's logits held across a wavefront (lane l holds experts
// l, l+64, ...; -inf beyond E), then its gate weights; lanes j < k store slot
// j.  k rounds of a 64-lane butterfly argmax pick the experts in descending
// logit order, ties to the lower id.
template <int VPL>
__device__ __forceinline__ void topk_softmax_store(float (&v)[VPL], int E, int k, int gating,
                                                   int lane, int32_t* __restrict__ idx_out,
                                                   float* __restrict__ w_out,
                                                   int* sel_id = nullptr, float* sel_w = nullptr) {
  // softmax over all experts needs the untouched logits: its denominator first
  float M = v[0];
#pragma unroll
  for (int i = 1; i < VPL; ++i) M = fmaxf(M, v[i]);
  M = wave_max_dpp(M);
  float Z = 0.f;
  if (gating != 0) {
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + kWave * i < E) z += expf(v[i] - M);
    Z = wave_sum(z);
  }
  float my_s = -INFINITY;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = v[0];
    int be = lane;
#pragma unroll
    for (int i = 1; i < VPL; ++i)
      if (v[i] > bv) { bv = v[i]; be = lane + kWave * i; }
    wave_argmax(bv, be);
    if (lane == j) { my_s = bv; my_id = be; }
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (be == lane + kWave * i) v[i] = -INFINITY;
  }
  float w;
  if (gating == 0) {
    // softmax over the selected logits, shifted by the largest of them
    const float ex = (lane < k) ? expf(my_s - M) : 0.f;
    w = ex / wave_sum(ex);
  } else {
    // softmax over all experts, then renormalised over the selected ones
    const float pj = (lane < k) ? expf(my_s - M) / Z : 0.f;
    w = pj / wave_sum(pj);
  }
  if (lane < k) {
    idx_out[lane] = my_id;
    w_out[lane] = w;
  }
  if (sel_id != nullptr) {
    *sel_id = my_id;
    *sel_w = w;
  }
}

}  // namespace moe
