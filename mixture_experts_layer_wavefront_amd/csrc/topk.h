// Top-k and gate weights of one token's router logits, held by a whole
// wavefront or by a group of 8 or 16 of its lanes, for the router's
// selection kernels.  "Sparsely-Gated MoE 구현 관점에서 살펴보기" (molayo1419.me),
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
  // bitwise, not short-circuit, so it compiles to compares and selects
  const bool take = (ov > bv) | ((ov == bv) & (oe < be));
  bv = take ? ov : bv;
  be = take ? oe : be;
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

// The same selection and gate weights for a token held by a group of G = 8 or
// 16 lanes (aligned inside a 16-lane row, so every DPP move stays inside the
// group): lane g of the group holds experts g + G i, i < NV (-inf beyond E),
// and the wavefront serves 64 / G tokens at once.  The argmax and the maximum
// run over the group with DPP moves only.  Selection is the same (the order
// is total).  The gate weights come out bit for bit as topk_softmax_store's,
// because every floating-point sum here follows that function's order: its
// lane l holds experts l + 64 i', which are this group's lane g = l mod G,
// i = m + (64 / G) i' with m = l / G.  Its per-lane sum and the butterfly
// levels over the high bits of l (m) therefore run inside one lane here, the
// levels over the low bits (g) across the group, in the same sequence; the
// slot sums (slot j in lane j there, zero beyond k) run inside every lane,
// which holds all selected values.  k <= KMAX (a power of two).
template <int G>
__device__ __forceinline__ float group_max_dpp(float v) {
  static_assert(G == 8 || G == 16, "groups of 8 or 16 lanes");
  v = fmaxf(v, __int_as_float(dpp_mov<kDppXor1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_mov<kDppXor2>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_mov<kDppHalfMirror>(__float_as_int(v))));
  if constexpr (G == 16) v = fmaxf(v, __int_as_float(dpp_mov<kDppMirror>(__float_as_int(v))));
  return v;
}
template <int G>
__device__ __forceinline__ void group_argmax(float& bv, int& be) {
  argmax_dpp<kDppXor1>(bv, be);
  argmax_dpp<kDppXor2>(bv, be);
  argmax_dpp<kDppHalfMirror>(bv, be);
  if constexpr (G == 16) argmax_dpp<kDppMirror>(bv, be);
}

template <int G, int NV, int KMAX>
__device__ __forceinline__ void group_topk_softmax_store(float (&v)[NV], int E, int k, int gating,
                                                         int g, bool store,
                                                         int32_t* __restrict__ idx_out,
                                                         float* __restrict__ w_out) {
  constexpr int MV = kWave / G;  // whole-wavefront lanes per group lane
  static_assert((KMAX & (KMAX - 1)) == 0 && KMAX <= kWave, "KMAX: a power of two");
  float M = v[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) M = fmaxf(M, v[i]);
  M = group_max_dpp<G>(M);
  float Z = 0.f;
  if (gating != 0) {
    float zl[MV];
#pragma unroll
    for (int m = 0; m < MV; ++m) zl[m] = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (g + G * i < E) zl[i % MV] += expf(v[i] - M);
#pragma unroll
    for (int h = MV / 2; h >= 1; h >>= 1)
#pragma unroll
      for (int m = 0; m < h; ++m) zl[m] = zl[m] + zl[m + h];
    float z = zl[0];
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) z += __shfl_xor(z, o, kWave);
    Z = z;
  }
  float sv[KMAX];
  int se[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    sv[j] = -INFINITY;
    se[j] = 0;
    if (j < k) {  // k is uniform: the whole wavefront takes the branch
      float bv = v[0];
      int be = g;
#pragma unroll
      for (int i = 1; i < NV; ++i)
        if (v[i] > bv) { bv = v[i]; be = g + G * i; }
      group_argmax<G>(bv, be);
      sv[j] = bv;
      se[j] = be;
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (be == g + G * i) v[i] = -INFINITY;
    }
  }
  float p[KMAX], s[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    p[j] = 0.f;
    if (j < k) p[j] = gating == 0 ? expf(sv[j] - M) : expf(sv[j] - M) / Z;
    s[j] = p[j];
  }
#pragma unroll
  for (int h = KMAX / 2; h >= 1; h >>= 1)
#pragma unroll
    for (int j = 0; j < h; ++j) s[j] = s[j] + s[j + h];
  if (store) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k && g == j) {
        idx_out[j] = se[j];
        w_out[j] = p[j] / s[0];
      }
  }
}

}  // namespace moe
