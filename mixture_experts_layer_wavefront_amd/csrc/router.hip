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
// bf16 layers: the logits run on the matrix cores (exact three-way bf16 split
// of W_r, K split over workgroups), then a selection kernel adds the partial
// logits and the bias and takes the top-k: a group of 8 or 16 lanes per
// token (k <= 8, at least 128 tokens), else one wavefront per token.  fp32
// layers: one fused kernel accumulates a [TT x E] logit tile with fp32 FMAs
// from LDS-staged slices of X and W_r and keeps it in LDS for the top-k.
// The top-k itself: k rounds of an argmax over the lanes holding the
// token's logits (ties to the lower expert id) pick the experts in
// descending-logit order; both layouts give the same bits (topk.h).
#include "common.h"
#include "launch.h"
#include "topk.h"

#include <algorithm>

namespace moe {
namespace {

constexpr int kRouterThreads = 256;
constexpr int kRouterDK = 32;
// Selection with a group of lanes per token: for k up to kGroupSelKMax and at
// least kGroupSelMinT tokens (decode batches keep one wavefront per token,
// which spreads their few tokens over more SIMDs).
constexpr int kGroupSelKMax = 8;
constexpr int kGroupSelMinT = 128;

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

// fp32 layers: one fused kernel.  TX threads across experts (expert
// e = tx + TX*j, j < RE), TY = 256/TX
// threads across tokens (token row = ty + TY*i, i < RT).
// PARTIAL (bf16 layers with few tokens): workgroup (x, s) covers K range
// [s*ks, (s+1)*ks) only and writes its partial logits (no bias) to
// partial[s][t][e] (row stride EP); a select kernel adds the S partials.
template <int TX, int RE, int RT, typename XT, bool PARTIAL>
__global__ __launch_bounds__(kRouterThreads) void router_topk_kernel(
    const XT* __restrict__ X, const float* __restrict__ W_r,
    const float* __restrict__ bias, int T, int d, int E, int k, int gating,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int ks,
    float* __restrict__ partial) {
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

  const int kbeg = PARTIAL ? (int)blockIdx.y * ks : 0;
  const int kend = PARTIAL ? min(d, kbeg + ks) : d;
  // Slices of DK along K go global -> registers -> LDS; the next slice's
  // loads are in flight while the current one is multiplied.
  constexpr int XN = (TT * CPR + kRouterThreads - 1) / kRouterThreads;
  constexpr int WN = (EP * (DK / 4) + kRouterThreads - 1) / kRouterThreads;
  float xr[XN][VE];
  f32x4 wr[WN];
  auto load_slice = [&](int k0) {
#pragma unroll
    for (int n = 0; n < XN; ++n) {
      const int c = tid + n * kRouterThreads;
      const int row = c / CPR, kc = c % CPR;
      const int t = t0 + row, kk = k0 + kc * VE;
      if (c < TT * CPR && t < T && kk < kend) {
        XLoad<XT>::load(X + (int64_t)t * d + kk, xr[n]);
      } else {
#pragma unroll
        for (int i = 0; i < VE; ++i) xr[n][i] = 0.f;
      }
    }
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      const int c = tid + n * kRouterThreads;
      const int e = c / (DK / 4), kc = c % (DK / 4);
      const int kk = k0 + kc * 4;
      wr[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (c < EP * (DK / 4) && e < E && kk < kend)
        wr[n] = *reinterpret_cast<const f32x4*>(W_r + (int64_t)e * d + kk);
    }
  };
  if (kbeg < kend) load_slice(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += DK) {
    // X[t0:t0+TT, k0:k0+DK] and W_r[:, k0:k0+DK], transposed, into LDS
#pragma unroll
    for (int n = 0; n < XN; ++n) {
      const int c = tid + n * kRouterThreads;
      if (c < TT * CPR) {
        const int row = c / CPR, kc = c % CPR;
#pragma unroll
        for (int i = 0; i < VE; ++i) Xs[kc * VE + i][row] = xr[n][i];
      }
    }
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      const int c = tid + n * kRouterThreads;
      if (c < EP * (DK / 4)) {
        const int e = c / (DK / 4), kc = c % (DK / 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) Ws[kc * 4 + i][e] = wr[n][i];
      }
    }
    __syncthreads();
    if (k0 + DK < kend) load_slice(k0 + DK);
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

  if constexpr (PARTIAL) {
    float* out = partial + (int64_t)blockIdx.y * T * EP;
#pragma unroll
    for (int j = 0; j < RE; ++j)
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int t = t0 + ty + TY * i;
        if (t < T) out[(int64_t)t * EP + tx + TX * j] = acc[i][j];
      }
    return;
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
    topk_softmax_store<VPL>(v, E, k, gating, lane, topk_idx + (int64_t)t * k, topk_w + (int64_t)t * k);
  }
}

// ---- bf16 layers: logits on the matrix cores --------------------------------
// X is exactly bf16.  W_r (fp32) is split exactly into three bf16 planes,
// W_r = hi + mid + lo (hi and mid truncate, lo holds the last 8 bits), so
// X W_r^T = X hi^T + X mid^T + X lo^T with every product exact in fp32; the
// v_mfma_f32_16x16x32_bf16 sums are fp32.  The K dimension is split over
// S workgroups per token tile for parallelism; a select kernel adds the S
// partial logits in a fixed order (then the bias) and takes the top-k.

constexpr int kRtTok = 128;  // tokens per logits workgroup (4 waves x 32)
constexpr int kRtK = 32;     // K per stage: one 16x16x32 MFMA k-step
constexpr int kRtZ = 2;  // expert groups of a wide router (EP >= 128)

__device__ __forceinline__ uint32_t rt_swz(uint32_t r) { return ((r >> 1) ^ (r >> 3)) & 3u; }

// W_r [E, d] fp32 -> Wsplit [3][EP][d32] bf16 (zero rows e >= E, zero k >= d)
__global__ __launch_bounds__(256) void router_split_kernel(
    const float* __restrict__ W_r, int E, int d, int EP, int d32,
    uint16_t* __restrict__ Wsplit) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 8 k per thread
  const int per_row = d32 / 8;
  if (i >= (int64_t)EP * per_row) return;
  const int e = (int)(i / per_row), k0 = (int)(i % per_row) * 8;
  uint32_t hw[4] = {0, 0, 0, 0}, mw[4] = {0, 0, 0, 0}, lw[4] = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int kk = k0 + j;
    const float w = (e < E && kk < d) ? W_r[(int64_t)e * d + kk] : 0.f;
    const float hi = __uint_as_float(__float_as_uint(w) & 0xFFFF0000u);
    const float r1 = w - hi;  // exact
    const float mid = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
    const float r2 = r1 - mid;  // exact, <= 8 significant bits: bf16 holds it
    const uint32_t sh = (j & 1) * 16;
    hw[j >> 1] |= (__float_as_uint(hi) >> 16) << sh;
    mw[j >> 1] |= (__float_as_uint(mid) >> 16) << sh;
    lw[j >> 1] |= (uint32_t)f32_to_bf16_bits(r2) << sh;
  }
  const int64_t plane = (int64_t)EP * d32;
  const int64_t o = (int64_t)e * d32 + k0;
  *reinterpret_cast<i32x4*>(Wsplit + o) = i32x4{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3]};
  *reinterpret_cast<i32x4*>(Wsplit + plane + o) = i32x4{(int)mw[0], (int)mw[1], (int)mw[2], (int)mw[3]};
  *reinterpret_cast<i32x4*>(Wsplit + 2 * plane + o) = i32x4{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3]};
}

// Partial logits of 128 tokens x EP experts over K-steps [k-slice of s];
// the experts are [e0, e0 + EP) with e0 = blockIdx.z EP, of the EPtot rows
// of each weight plane (and of each partial row).  Wave w owns tokens
// 32w + [0, 32) (two 16-row tiles) and all NTE expert tiles.  Each K-step's
// three weight planes and 128 token rows are staged in LDS (64-byte rows,
// chunk-swizzled).  The loads run NSR - 1 K-steps ahead (NSR stages): a
// K-step's matrix work is short (3 NTE x 2 MFMAs per wave), so with one step
// ahead every step waited for a whole memory latency.
template <int NTE>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ X, int T, int d, const uint16_t* __restrict__ Wsplit,
    int d32, int S, int EPtot, float* __restrict__ partial) {
  constexpr int EP = 16 * NTE;
  constexpr int ROWS = 3 * EP;           // staged weight rows per K-step
  constexpr int WBYTES = ROWS * 64;      // weight part of a stage
  constexpr int STAGE = WBYTES + kRtTok * 64;  // + the token rows
  constexpr int NINSTR = ROWS / 16;      // 1 KB wave-level weight loads per stage
  constexpr int NSR = NTE >= 8 ? 2 : 4;  // stages (K-steps in flight + 1)
  constexpr int D = NSR - 1;             // K-steps requested ahead
  // vector-memory loads of one K-step issued by the wave with the fewest:
  // its share of the weight loads and its two token-row loads (loads
  // complete in order, so waiting until at most this many per later step
  // are outstanding finishes the step's loads; waves with more wait a
  // little longer)
  constexpr int CMIN = NINSTR / 4 + 2;
  __shared__ __attribute__((aligned(1024))) char smem[NSR * STAGE];

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t0 = blockIdx.x * kRtTok;
  const int s = blockIdx.y;
  const int e0 = blockIdx.z * EP;
  const int nk = d32 / kRtK;
  const int ks0 = (int)((int64_t)s * nk / S), ks1 = (int)((int64_t)(s + 1) * nk / S);
  const int nks = ks1 - ks0;

  // weight-plane loads: instruction q covers staged rows 16q..16q+15; staged
  // row R is row e0 + R % EP of plane R / EP.  Token rows: this wave's 32
  // tokens, 16 rows per load (rows past T read zero, and so do K chunks
  // past d).
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wsplit, (uint32_t)((int64_t)3 * EPtot * d32 * 2));
  const int xt0 = t0 + wave * 32;
  const int xrows = __builtin_amdgcn_readfirstlane(max(0, min(32, T - xt0)));
  const int xbase = __builtin_amdgcn_readfirstlane(min(xt0, max(T - 1, 0)));
  const __amdgpu_buffer_rsrc_t rX =
      make_rsrc(X + (int64_t)xbase * d, (uint32_t)xrows * (uint32_t)d * 2u);
  auto issue = [&](int stage, int kstep) {
    char* st = smem + stage * STAGE;
    for (int q = wave; q < NINSTR; q += 4) {
      const uint32_t R = q * 16 + (lane >> 2);
      const uint32_t c = (lane & 3) ^ rt_swz(R);
      const uint32_t G = (R / EP) * (uint32_t)EPtot + (uint32_t)e0 + R % EP;
      const uint32_t vo = G * (uint32_t)d32 * 2u + (uint32_t)kstep * (kRtK * 2) + c * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, MOE_LDS_PTR(st + q * 1024), 16, vo, 0, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t r = h * 16 + (lane >> 2);  // row within the wave's 32
      const uint32_t R = wave * 32 + r;         // staged token row
      const uint32_t c = (lane & 3) ^ rt_swz(R);
      const int kk = kstep * kRtK + c * 8;
      const uint32_t vo = kk < d ? (r * (uint32_t)d + kk) * 2u : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, MOE_LDS_PTR(st + WBYTES + (wave * 2 + h) * 1024),
                                               16, vo, 0, 0, 0);
    }
  };
  f32x4 acc[2][NTE];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTE; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int u = 0; u < D; ++u)
    if (u < nks) issue(u, ks0 + u);
  // step j consumes stage j % NSR (the loop is unrolled by NSR)
  for (int j0 = 0; j0 < nks; j0 += NSR) {
#pragma unroll
    for (int u = 0; u < NSR; ++u) {
      const int j = j0 + u;
      if (j >= nks) break;
      // step j's loads have landed once at most the later steps' loads are
      // outstanding; every wave is then done with stage (j - 1) % NSR
      if (D > 1 && j + D - 1 < nks)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(CMIN * (D > 1 ? D - 1 : 0)) : "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (j + D < nks) issue((u + D) % NSR, ks0 + j + D);
      const char* st = smem + u * STAGE;
      // A fragments: token (l % 16) of 16-row tile mt of this wave, chunk l / 16
      bf16x8 xa[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const uint32_t R = wave * 32 + mt * 16 + (lane & 15);
        xa[mt] = *reinterpret_cast<const bf16x8*>(st + WBYTES + R * 64 + (((lane >> 4) ^ rt_swz(R)) * 16));
      }
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int nt = 0; nt < NTE; ++nt) {
          // B fragment of expert tile nt, plane p: row p*EP + nt*16 + (l % 16),
          // chunk l / 16
          const uint32_t R = p * EP + nt * 16 + (lane & 15);
          const uint32_t off = R * 64 + (((lane >> 4) ^ rt_swz(R)) * 16);
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(st + off);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mt], b, acc[mt][nt], 0, 0, 0);
        }
    }
  }

  // D[token][expert]: lane holds rows 4*(l/16) + r, column l % 16
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = xt0 + mt * 16 + 4 * (lane >> 4) + r;
      if (t < T) {
        float* dst = partial + ((int64_t)s * T + t) * EPtot + e0 + (lane & 15);
#pragma unroll
        for (int nt = 0; nt < NTE; ++nt) dst[nt * 16] = acc[mt][nt][r];
      }
    }
}

// One wavefront per token: sum the S partials in order, add the bias, top-k.
template <int VPL>
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ partial, const float* __restrict__ bias, int T, int E,
    int EP, int S, int k, int gating, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  // the partials of all of this lane's experts are requested CH at a time per
  // expert before any is added (one memory round trip per chunk instead of
  // one per expert and chunk), then added in the order s = 0, 1, ...
  constexpr int CH = VPL <= 2 ? 32 : 16;
  float acc[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < S; s0 += CH) {
    float pv[VPL][CH];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + kWave * i;
#pragma unroll
      for (int u = 0; u < CH; ++u)
        pv[i][u] = (e < E && s0 + u < S) ? partial[((int64_t)(s0 + u) * T + t) * EP + e] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
      for (int u = 0; u < CH; ++u)
        if (s0 + u < S) acc[i] += pv[i][u];
  }
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    v[i] = (e < E) ? acc[i] + (bias != nullptr ? bias[e] : 0.f) : -INFINITY;
  }
  topk_softmax_store<VPL>(v, E, k, gating, lane, topk_idx + (int64_t)t * k, topk_w + (int64_t)t * k);
}

// The same with a group of G lanes per token (64 / G tokens per wavefront):
// lane g of a group holds experts g + G i, i < NV.  The partials are added in
// the same order (s = 0, 1, ...; SB of them loaded at a time), so the logits,
// the selection and the gate weights equal router_select_kernel's bit for bit.
// Groups past T compute on token T - 1 and store nothing.
template <int G, int NV>
__global__ __launch_bounds__(256) void router_select_group_kernel(
    const float* __restrict__ partial, const float* __restrict__ bias, int T, int E,
    int EP, int S, int k, int gating, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  constexpr int TPW = kWave / G;
  constexpr int SB = NV >= 16 ? 4 : (NV >= 8 ? 8 : 16);
  const int lane = threadIdx.x % kWave;
  const int g = lane % G;
  const int t = (blockIdx.x * (256 / kWave) + threadIdx.x / kWave) * TPW + lane / G;
  const bool valid = t < T;
  const int tl = valid ? t : T - 1;
  float acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < S; s0 += SB) {
    float pv[SB][NV];
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int i = 0; i < NV; ++i)
        pv[u][i] = (s0 + u < S && g + G * i < E)
                       ? partial[((int64_t)(s0 + u) * T + tl) * EP + g + G * i] : 0.f;
#pragma unroll
    for (int u = 0; u < SB; ++u)
      if (s0 + u < S)
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i] += pv[u][i];
  }
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = g + G * i;
    v[i] = e < E ? acc[i] + (bias != nullptr ? bias[e] : 0.f) : -INFINITY;
  }
  group_topk_softmax_store<G, NV, kGroupSelKMax>(v, E, k, gating, g, valid,
                                                 topk_idx + (int64_t)tl * k, topk_w + (int64_t)tl * k);
}

// Few tokens (bf16): K-split FMA partial logits (no W_r split) + select.
constexpr int kSmallT = 64;
constexpr int kSmallKS = 64;  // K per workgroup

// Router statistics (monitoring).  Same selection as router_select_kernel,
// one wavefront per token; each lane also forms, for the experts it holds,
// the gate weight the token gives them (importance), whether the token
// selected them, and their softmax probability over all E logits; lane 0
// the squared log-sum-exp of the logits.  The four wavefronts' values are
// added in order into one row per workgroup:
//   stat_part[block][0:E) importance, [E:2E) probability sums,
//   [2E:3E) selection counts, [3E] sum of squared log-sum-exp.
// Rows are then added in fixed order: 64 at a time by router_stats_rows_kernel
// (when there are more than 64), then by router_stats_reduce_kernel.
constexpr int kStatBlockTok = 4;  // tokens per workgroup
constexpr int kStatRows = 64;     // rows per partial sum

template <int VPL>
__global__ __launch_bounds__(256) void router_select_stats_kernel(
    const float* __restrict__ partial, const float* __restrict__ bias, int T, int E,
    int EP, int S, int k, int gating, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ stat_part) {
  __shared__ float s_acc[4][3 * 256 + 1];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  float imp[VPL], cnt[VPL], prob[VPL], lse2 = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) imp[i] = cnt[i] = prob[i] = 0.f;
  {
    const int t = blockIdx.x * kStatBlockTok + wave;
    if (t < T) {
    float v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E) {
        float acc = 0.f;
        for (int s0 = 0; s0 < S; s0 += 16) {
          float pv[16];
#pragma unroll
          for (int u = 0; u < 16; ++u)
            pv[u] = (s0 + u < S) ? partial[((int64_t)(s0 + u) * T + t) * EP + e] : 0.f;
#pragma unroll
          for (int u = 0; u < 16; ++u)
            if (s0 + u < S) acc += pv[u];
        }
        v[i] = acc + (bias != nullptr ? bias[e] : 0.f);
      } else {
        v[i] = -INFINITY;
      }
    }
    // softmax over all experts and the log-sum-exp, from the untouched logits
    float M = v[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) M = fmaxf(M, v[i]);
    M = wave_max(M);
    float ex[VPL], z = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      ex[i] = (lane + kWave * i < E) ? expf(v[i] - M) : 0.f;
      z += ex[i];
    }
    const float Z = wave_sum(z);
#pragma unroll
    for (int i = 0; i < VPL; ++i) prob[i] += ex[i] / Z;
    const float lse = M + logf(Z);
    lse2 += lse * lse;
    int my_id = 0;
    float my_w = 0.f;
    topk_softmax_store<VPL>(v, E, k, gating, lane, topk_idx + (int64_t)t * k,
                            topk_w + (int64_t)t * k, &my_id, &my_w);
    // slot j's (expert, weight) to the lane that holds that expert
    for (int j = 0; j < k; ++j) {
      const int e = __shfl(my_id, j, kWave);
      const float wj = __shfl(my_w, j, kWave);
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (e == lane + kWave * i) {
          imp[i] += wj;
          cnt[i] += 1.f;
        }
    }
    }
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    if (e < E) {
      s_acc[wave][e] = imp[i];
      s_acc[wave][E + e] = prob[i];
      s_acc[wave][2 * E + e] = cnt[i];
    }
  }
  if (lane == 0) s_acc[wave][3 * E] = lse2;
  __syncthreads();
  for (int c = threadIdx.x; c <= 3 * E; c += 256)
    stat_part[(int64_t)blockIdx.x * (3 * E + 1) + c] =
        ((s_acc[0][c] + s_acc[1][c]) + s_acc[2][c]) + s_acc[3][c];
}

// Rows [64 x, 64 x + 64) of `in` added in order, column by column
// (blockIdx.y picks 256 columns).
__global__ __launch_bounds__(256) void router_stats_rows_kernel(
    const float* __restrict__ in, int nrows, int C, float* __restrict__ out) {
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= C) return;
  const int r0 = blockIdx.x * kStatRows, r1 = min(nrows, r0 + kStatRows);
  float acc = 0.f;
  for (int b0 = r0; b0 < r1; b0 += 16) {
    float pv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      pv[u] = (b0 + u < r1) ? in[(int64_t)(b0 + u) * C + c] : 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (b0 + u < r1) acc += pv[u];
  }
  out[(int64_t)blockIdx.x * C + c] = acc;
}

// One workgroup: add the remaining rows in order (column c by thread c),
// then importance | mean probability | aux loss | z-loss.
__global__ __launch_bounds__(1024) void router_stats_reduce_kernel(
    const float* __restrict__ stat_part, int nblk, int T, int E, int k,
    float* __restrict__ router_stats) {
  __shared__ float s_col[3 * 256 + 1];
  const int C = 3 * E + 1;
  for (int c = threadIdx.x; c < C; c += 1024) {
    float acc = 0.f;
    for (int b0 = 0; b0 < nblk; b0 += 16) {
      float pv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        pv[u] = (b0 + u < nblk) ? stat_part[(int64_t)(b0 + u) * C + c] : 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (b0 + u < nblk) acc += pv[u];
    }
    s_col[c] = acc;
  }
  __syncthreads();
  const float inv_t = 1.f / (float)T;
  for (int e = threadIdx.x; e < E; e += 1024) {
    router_stats[e] = s_col[e];
    router_stats[E + e] = s_col[E + e] * inv_t;
  }
  if (threadIdx.x == 0) {
    float aux = 0.f;
    const float inv_tk = 1.f / ((float)T * (float)k);
    for (int e = 0; e < E; ++e) aux += (s_col[2 * E + e] * inv_tk) * (s_col[E + e] * inv_t);
    router_stats[2 * E] = (float)E * aux;
    router_stats[2 * E + 1] = s_col[3 * E] * inv_t;
  }
}

struct RoutePlan {
  int NTE, EP, d32, S, tiles;
  bool fused;   // fp32 X without statistics: one fused kernel, no scratch
  bool small;   // K-split FMA partial logits (few bf16 tokens, or fp32 X
                // with statistics)
  size_t split_bytes, partial_bytes, stat_bytes;
};

size_t a256r(size_t x) { return (x + 255) & ~size_t(255); }

RoutePlan route_plan(int T, int E, int d, bool x_bf16, bool stats) {
  RoutePlan P{};
  if (stats) {
    const size_t nblk = (size_t)(T + kStatBlockTok - 1) / kStatBlockTok;
    const size_t ngrp = (nblk + kStatRows - 1) / kStatRows;
    P.stat_bytes = a256r(nblk * (3 * E + 1) * 4) + a256r(ngrp * (3 * E + 1) * 4);
  }
  if (!x_bf16 && !stats) {
    P.fused = true;
    return P;
  }
  if (T <= kSmallT || !x_bf16) {
    P.small = true;
    P.EP = E <= 8 ? 8 : E <= 16 ? 16 : E <= 32 ? 32 : E <= 64 ? 64 : E <= 128 ? 128 : 256;
    // fp32 X (statistics requested): one partial over all of K, so the
    // logits equal the fused kernel's bit for bit
    P.S = x_bf16 ? (d + kSmallKS - 1) / kSmallKS : 1;
    P.split_bytes = 0;
    P.partial_bytes = a256r((size_t)P.S * T * P.EP * 4);
    return P;
  }
  int nte = (E + 15) / 16, p2 = 1;
  while (p2 < nte) p2 <<= 1;
  P.NTE = p2;
  P.EP = 16 * p2;
  P.d32 = (d + kRtK - 1) / kRtK * kRtK;
  P.tiles = (T + kRtTok - 1) / kRtTok;
  const int nk = P.d32 / kRtK;
  const int64_t cap = std::max<int64_t>(1, (int64_t(32) << 20) / std::max<int64_t>(1, (int64_t)T * P.EP * 4));
  int S = std::max(1, (256 + std::max(P.tiles, 1) - 1) / std::max(P.tiles, 1));
  S = (int)std::min<int64_t>(std::min<int64_t>(S, nk), cap);
  P.S = std::max(1, S);
  P.split_bytes = a256r((size_t)3 * P.EP * P.d32 * 2);
  P.partial_bytes = a256r((size_t)P.S * T * P.EP * 4);
  return P;
}

template <int TX, int RE, int RT>
hipError_t launch_cfg(const void* X, bool x_bf16, const float* W_r,
                      const float* bias, int T, int d, int E, int k, int gating,
                      int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  constexpr int TT = (kRouterThreads / TX) * RT;
  const dim3 grid((T + TT - 1) / TT);
  if (x_bf16)
    router_topk_kernel<TX, RE, RT, uint16_t, false><<<grid, kRouterThreads, 0, stream>>>(
        static_cast<const uint16_t*>(X), W_r, bias, T, d, E, k, gating, topk_idx, topk_w, 0, nullptr);
  else
    router_topk_kernel<TX, RE, RT, float, false><<<grid, kRouterThreads, 0, stream>>>(
        static_cast<const float*>(X), W_r, bias, T, d, E, k, gating, topk_idx, topk_w, 0, nullptr);
  return hipGetLastError();
}

// K-split partial logits with fp32 FMAs (EP = TX * RE columns)
template <int TX, int RE, int RT, typename XT>
hipError_t launch_partial(const XT* X, const float* W_r, int T, int d, int E,
                          int S, float* partial, hipStream_t stream) {
  constexpr int TT = (kRouterThreads / TX) * RT;
  const dim3 grid((T + TT - 1) / TT, S);
  router_topk_kernel<TX, RE, RT, XT, true><<<grid, kRouterThreads, 0, stream>>>(
      X, W_r, nullptr, T, d, E, 0, 0, nullptr, nullptr, S == 1 ? d : kSmallKS, partial);
  return hipGetLastError();
}

template <typename XT>
hipError_t launch_partial_ep(const XT* X, const float* W_r, int T, int d, int E, int EP,
                             int S, float* partial, hipStream_t stream) {
  switch (EP) {
    case 8: return launch_partial<8, 1, 2>(X, W_r, T, d, E, S, partial, stream);
    case 16: return launch_partial<16, 1, 2>(X, W_r, T, d, E, S, partial, stream);
    case 32: return launch_partial<32, 1, 2>(X, W_r, T, d, E, S, partial, stream);
    case 64: return launch_partial<64, 1, 4>(X, W_r, T, d, E, S, partial, stream);
    case 128: return launch_partial<64, 2, 4>(X, W_r, T, d, E, S, partial, stream);
    default: return launch_partial<64, 4, 4>(X, W_r, T, d, E, S, partial, stream);
  }
}

// Sum of the S partials, bias, top-k and gate weights (and the statistics).
hipError_t launch_select(const float* partial, const float* bias, int T, int E, int EP,
                         int S, int k, int gating, int32_t* topk_idx, float* topk_w,
                         float* stat_part, float* router_stats, hipStream_t stream) {
  if (router_stats == nullptr) {
    if (k <= kGroupSelKMax && T >= kGroupSelMinT && E <= 256) {
      // 4 wavefronts per workgroup, 64 / G tokens per wavefront
      const unsigned g8 = (unsigned)((T + 31) / 32), g16 = (unsigned)((T + 15) / 16);
      if (E <= 8)
        router_select_group_kernel<8, 1><<<g8, 256, 0, stream>>>(partial, bias, T, E, EP, S, k, gating, topk_idx, topk_w);
      else if (E <= 16)
        router_select_group_kernel<8, 2><<<g8, 256, 0, stream>>>(partial, bias, T, E, EP, S, k, gating, topk_idx, topk_w);
      else if (E <= 32)
        router_select_group_kernel<8, 4><<<g8, 256, 0, stream>>>(partial, bias, T, E, EP, S, k, gating, topk_idx, topk_w);
      else if (E <= 64)
        router_select_group_kernel<8, 8><<<g8, 256, 0, stream>>>(partial, bias, T, E, EP, S, k, gating, topk_idx, topk_w);
      else if (E <= 128)
        router_select_group_kernel<16, 8><<<g16, 256, 0, stream>>>(partial, bias, T, E, EP, S, k, gating, topk_idx, topk_w);
      else
        router_select_group_kernel<16, 16><<<g16, 256, 0, stream>>>(partial, bias, T, E, EP, S, k, gating, topk_idx, topk_w);
      return hipGetLastError();
    }
    // one token per wavefront; up to 64 tokens one wavefront per workgroup,
    // so few tokens spread over as many CUs
    const int wpb = T <= 64 ? 1 : 4;
    const unsigned gs = (unsigned)((T + wpb - 1) / wpb);
    const unsigned bs = (unsigned)(wpb * kWave);
    if (E <= 64)
      router_select_kernel<1><<<gs, bs, 0, stream>>>(partial, bias, T, E, EP, S, k, gating, topk_idx, topk_w);
    else if (E <= 128)
      router_select_kernel<2><<<gs, bs, 0, stream>>>(partial, bias, T, E, EP, S, k, gating, topk_idx, topk_w);
    else
      router_select_kernel<4><<<gs, bs, 0, stream>>>(partial, bias, T, E, EP, S, k, gating, topk_idx, topk_w);
    return hipGetLastError();
  }
  const int nblk = (T + kStatBlockTok - 1) / kStatBlockTok;
  if (E <= 64)
    router_select_stats_kernel<1><<<nblk, 256, 0, stream>>>(partial, bias, T, E, EP, S, k, gating, topk_idx, topk_w, stat_part);
  else if (E <= 128)
    router_select_stats_kernel<2><<<nblk, 256, 0, stream>>>(partial, bias, T, E, EP, S, k, gating, topk_idx, topk_w, stat_part);
  else
    router_select_stats_kernel<4><<<nblk, 256, 0, stream>>>(partial, bias, T, E, EP, S, k, gating, topk_idx, topk_w, stat_part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int C = 3 * E + 1;
  const float* rows = stat_part;
  int nrows = nblk;
  if (nblk > kStatRows) {
    float* grp = stat_part + a256r((size_t)nblk * C * 4) / 4;
    const int ngrp = (nblk + kStatRows - 1) / kStatRows;
    router_stats_rows_kernel<<<dim3(ngrp, (C + 255) / 256), 256, 0, stream>>>(stat_part, nblk, C, grp);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    rows = grp;
    nrows = ngrp;
  }
  router_stats_reduce_kernel<<<1, 1024, 0, stream>>>(rows, nrows, T, E, k, router_stats);
  return hipGetLastError();
}

}  // namespace

size_t route_scratch_bytes(int T, int E, int d, bool x_bf16, bool stats) {
  if (T == 0) return 0;
  const RoutePlan P = route_plan(T, E, d, x_bf16, stats);
  return P.split_bytes + P.partial_bytes + P.stat_bytes;
}

hipError_t launch_route(const void* X, bool x_bf16, const float* W_r,
                        const float* bias, int T, int d, int E, int k,
                        int gating, int32_t* topk_idx, float* topk_w,
                        void* scratch, float* router_stats, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const RoutePlan P = route_plan(T, E, d, x_bf16, router_stats != nullptr);
  if (P.fused) {
    if (E <= 8) return launch_cfg<8, 1, 1>(X, x_bf16, W_r, bias, T, d, E, k, gating, topk_idx, topk_w, stream);
    if (E <= 16) return launch_cfg<16, 1, 1>(X, x_bf16, W_r, bias, T, d, E, k, gating, topk_idx, topk_w, stream);
    if (E <= 32) return launch_cfg<32, 1, 2>(X, x_bf16, W_r, bias, T, d, E, k, gating, topk_idx, topk_w, stream);
    if (E <= 64) return launch_cfg<64, 1, 4>(X, x_bf16, W_r, bias, T, d, E, k, gating, topk_idx, topk_w, stream);
    if (E <= 128) return launch_cfg<64, 2, 4>(X, x_bf16, W_r, bias, T, d, E, k, gating, topk_idx, topk_w, stream);
    return launch_cfg<64, 4, 4>(X, x_bf16, W_r, bias, T, d, E, k, gating, topk_idx, topk_w, stream);
  }
  char* sp = static_cast<char*>(scratch);
  uint16_t* Wsplit = reinterpret_cast<uint16_t*>(sp);
  float* partial = reinterpret_cast<float*>(sp + P.split_bytes);
  float* stat_part = reinterpret_cast<float*>(sp + P.split_bytes + P.partial_bytes);
  hipError_t err;
  if (P.small) {
    err = x_bf16 ? launch_partial_ep(static_cast<const uint16_t*>(X), W_r, T, d, E, P.EP, P.S, partial, stream)
                 : launch_partial_ep(static_cast<const float*>(X), W_r, T, d, E, P.EP, P.S, partial, stream);
    if (err != hipSuccess) return err;
    return launch_select(partial, bias, T, E, P.EP, P.S, k, gating, topk_idx, topk_w,
                         stat_part, router_stats, stream);
  }
  const int64_t nthr = (int64_t)P.EP * (P.d32 / 8);
  router_split_kernel<<<(unsigned)((nthr + 255) / 256), 256, 0, stream>>>(W_r, E, d, P.EP, P.d32, Wsplit);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // wide routers: the experts split over Z workgroups (smaller LDS stages,
  // several workgroups per CU)
  const int Z = P.NTE >= 8 ? kRtZ : 1;
  const dim3 g(P.tiles, P.S, Z);
  const uint16_t* Xb = static_cast<const uint16_t*>(X);
  switch (P.NTE / Z) {
    case 1: router_logits_kernel<1><<<g, 256, 0, stream>>>(Xb, T, d, Wsplit, P.d32, P.S, P.EP, partial); break;
    case 2: router_logits_kernel<2><<<g, 256, 0, stream>>>(Xb, T, d, Wsplit, P.d32, P.S, P.EP, partial); break;
    case 4: router_logits_kernel<4><<<g, 256, 0, stream>>>(Xb, T, d, Wsplit, P.d32, P.S, P.EP, partial); break;
    case 8: router_logits_kernel<8><<<g, 256, 0, stream>>>(Xb, T, d, Wsplit, P.d32, P.S, P.EP, partial); break;
    default: router_logits_kernel<16><<<g, 256, 0, stream>>>(Xb, T, d, Wsplit, P.d32, P.S, P.EP, partial); break;
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_select(partial, bias, T, E, P.EP, P.S, k, gating, topk_idx, topk_w,
                       stat_part, router_stats, stream);
}

}  // namespace moe
