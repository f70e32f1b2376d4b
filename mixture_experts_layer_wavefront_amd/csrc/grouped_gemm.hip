// Grouped SwiGLU FFN: for every expert e, over its rows [off[e], off[e+1]) of
// X_perm,
//     H = silu(X_e Wg_e^T) * (X_e Wu_e^T)      (gate/up GEMM, SwiGLU epilogue)
//     Y = H Wd_e^T                             (down GEMM, fp32 out)
// as two launches that each cover every expert ("grouped GEMM").
//
// Method: "5.3 Expert Parallelism" (sungeuns.github.io), section
// "최적화 2: GroupGEMM" (one launch for many GEMMs of different M instead
// of a kernel per expert); "Sparsely-Gated MoE 구현 관점에서 살펴보기"
// (molayo1419.me), forward-pipeline step 4 (each expert's FFN on its batch)
// and the closing remark that production code fuses these steps;
// "MoonEP의 계획 코드를 직접 돌려봤습니다" (thakicloud.com), section
// "설치 및 통합" (one packed weight tensor per projection, cu_seqlens picks
// each expert's active rows, no host sync).
//
// gfx950 design (bf16):
//  * Tiles: BM rows x BN output columns, BK = 64.  A wavefront owns TM x TN
//    32x32 sub-tiles and issues v_mfma_f32_32x32x16_bf16 (fp32 accumulate).
//    For gate/up one wavefront holds the gate AND the up accumulator of the
//    same output columns, so SwiGLU is applied in registers before the
//    single bf16 store of H.
//  * Operands are staged global -> LDS with buffer_load_dwordx4 ... lds (no
//    VGPR round trip), double-buffered.  A buffer resource per operand bounds
//    the tile, so rows past an expert's end, columns past N and the K tail
//    read as zero.  LDS rows are 128 B (64 bf16 of K); the 16-byte chunks of
//    row R are XOR-swizzled by ((R ^ (R >> 3)) & 7) so the ds_read_b128
//    fragment reads hit distinct banks.
//  * Schedule: a one-workgroup kernel turns expert_offsets into a prefix of
//    per-expert M-tile counts.  The grid is a static upper bound; each
//    workgroup finds its (expert, n-tile, m-tile) from the prefix and exits
//    if it has none -- no host round trip.  Tiles are ordered expert-major,
//    then n, then m, and remapped so that the hardware's round-robin of
//    workgroups over the 8 XCDs gives each XCD a contiguous run of tiles:
//    the tiles sharing one expert's weights and rows share one L2.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBK = 64;          // K per stage (bf16): 128-byte LDS rows
constexpr int kRowBytes = kBK * 2;
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t swz(uint32_t R) { return (R ^ (R >> 3)) & 7u; }

__global__ __launch_bounds__(256) void ffn_schedule_kernel(
    const int32_t* __restrict__ offsets, int E, int BM,
    int32_t* __restrict__ mt_prefix) {
  __shared__ int32_t s[256];
  const int e = threadIdx.x;
  const int mt = (e < E) ? (offsets[e + 1] - offsets[e] + BM - 1) / BM : 0;
  s[e] = mt;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int a = (e >= o) ? s[e - o] : 0;
    __syncthreads();
    s[e] += a;
    __syncthreads();
  }
  if (e < E) mt_prefix[e] = s[e] - mt;
  if (e == E - 1) mt_prefix[E] = s[e];
}

template <int MW, int NW, int TM, int TN, bool GATEUP>
struct GemmCfg {
  static constexpr int NWAVES = MW * NW;
  static constexpr int NT = NWAVES * kWave;
  static constexpr int BM = MW * TM * 32;
  static constexpr int BN = NW * TN * 32;            // output columns per tile
  static constexpr int NB = GATEUP ? 2 * TN : TN;    // B sub-tiles per wave
  static constexpr int BROWS = GATEUP ? 2 * BN : BN;  // B rows staged per K step
  static constexpr int ROWS = BM + BROWS;
  static constexpr int STAGE = ROWS * kRowBytes;
  static constexpr int NINSTR = ROWS / 8;            // 1 KB per wave-level load
  static constexpr int IPW = NINSTR / NWAVES;
  static_assert(NINSTR % NWAVES == 0, "loads must split evenly over waves");
  static constexpr int LDS_BYTES = 2 * STAGE + 1040;  // + the tile prefix
};

// A [R, K] bf16 rows; B0/B1 [E, N, K] bf16 (gate/up, or down with B1 unused).
// GATEUP: C = H bf16 [R, N].  Otherwise C = Y fp32 [R, N].
template <int MW, int NW, int TM, int TN, bool GATEUP>
__global__ __launch_bounds__(kWave * MW * NW) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, int N, int K, int E,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ mt_prefix,
    void* __restrict__ Cout) {
  using Cfg = GemmCfg<MW, NW, TM, TN, GATEUP>;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, NB = Cfg::NB, IPW = Cfg::IPW;
  constexpr int NWAVES = Cfg::NWAVES, STAGE = Cfg::STAGE;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int32_t* s_pref = reinterpret_cast<int32_t*>(smem + 2 * STAGE);

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

  for (int i = tid; i <= E; i += Cfg::NT) s_pref[i] = mt_prefix[i];
  __syncthreads();

  // ---- which tile is mine --------------------------------------------------
  const int n_nt = (N + BN - 1) / BN;
  const int total = s_pref[E] * n_nt;
  const int q = (total + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= q) return;
  const int logical = (blockIdx.x % kXcds) * q + slot;
  if (logical >= total) return;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] * n_nt <= logical) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int mt_e = s_pref[e + 1] - s_pref[e];
  const int local = logical - s_pref[e] * n_nt;
  const int n_t = local / mt_e, m_t = local % mt_e;
  const int row_end = offsets[e + 1];
  const int m_start = offsets[e] + m_t * BM;
  const int rows = min(BM, row_end - m_start);
  const int n0 = n_t * BN;
  const int ncols = min(BN, N - n0);

  const uint32_t kbytes = (uint32_t)K * 2u;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(A + (int64_t)m_start * K, (uint32_t)rows * kbytes);
  const int64_t boff = ((int64_t)e * N + n0) * K;
  const __amdgpu_buffer_rsrc_t rB0 = make_rsrc(B0 + boff, (uint32_t)ncols * kbytes);
  const __amdgpu_buffer_rsrc_t rB1 = GATEUP ? make_rsrc(B1 + boff, (uint32_t)ncols * kbytes) : rB0;

  // ---- per-lane load offsets (one 16-byte chunk per wave-level load) -------
  uint32_t voff[IPW];
  int kcol[IPW];
  {
    const uint32_t p = lane & 7;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int qi = wave + NWAVES * i;
      const uint32_t R = qi * 8 + (lane >> 3);
      const uint32_t c = p ^ swz(R);
      uint32_t row;
      if (qi * 8 < BM) row = R;
      else if (!GATEUP || qi * 8 < BM + BN) row = R - BM;
      else row = R - BM - BN;
      voff[i] = row * kbytes + c * 16;
      kcol[i] = c * 8;
    }
  }
  const int nk = (K + kBK - 1) / kBK;
  const bool ktail = (K % kBK) != 0;

  auto issue = [&](int stage, int kt) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int qi = wave + NWAVES * i;
      uint32_t vo = voff[i] + (uint32_t)kt * kRowBytes;
      if (ktail && kt * kBK + kcol[i] >= K) vo = kOob;
      char* dst = smem + stage * STAGE + qi * 1024;
      if (qi * 8 < BM)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, MOE_LDS_PTR(dst), 16, vo, 0, 0, 0);
      else if (!GATEUP || qi * 8 < BM + BN)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB0, MOE_LDS_PTR(dst), 16, vo, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB1, MOE_LDS_PTR(dst), 16, vo, 0, 0, 0);
    }
  };

  // ---- per-lane fragment read offsets within a stage ------------------------
  const int wm = wave % MW, wn = wave / MW;
  uint32_t offA[TM][4], offB[NB][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t c = 2 * ks + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
      const uint32_t R = wm * TM * 32 + mi * 32 + (lane & 31);
      offA[mi][ks] = R * kRowBytes + ((c ^ swz(R)) * 16);
    }
#pragma unroll
    for (int nj = 0; nj < NB; ++nj) {
      uint32_t brow;
      if (GATEUP) brow = (nj < TN) ? wn * TN * 32 + nj * 32 : BN + wn * TN * 32 + (nj - TN) * 32;
      else brow = wn * TN * 32 + nj * 32;
      const uint32_t R = BM + brow + (lane & 31);
      offB[nj][ks] = R * kRowBytes + ((c ^ swz(R)) * 16);
    }
  }

  f32x16 acc[TM][NB];
#pragma unroll
  for (int mi = 0; mi < TM; ++mi)
#pragma unroll
    for (int nj = 0; nj < NB; ++nj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.f;

  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int s = kt & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < nk) issue(s ^ 1, kt + 1);
    const char* st = smem + s * STAGE;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a[TM], b[NB];
#pragma unroll
      for (int mi = 0; mi < TM; ++mi) a[mi] = *reinterpret_cast<const bf16x8*>(st + offA[mi][ks]);
#pragma unroll
      for (int nj = 0; nj < NB; ++nj) b[nj] = *reinterpret_cast<const bf16x8*>(st + offB[nj][ks]);
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int nj = 0; nj < NB; ++nj)
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[nj], acc[mi][nj], 0, 0, 0);
    }
  }

  // ---- epilogue ---------------------------------------------------------------
  // acc[mi][nj][r] is element (row, col) of the tile with
  //   row = wm*TM*32 + mi*32 + 8*(r/4) + 4*(lane/32) + r%4,  col = lane%32 (+ sub-tile base)
  const int col_l = lane & 31;
  const int rbase = wm * TM * 32 + 4 * (lane >> 5);
  if constexpr (GATEUP) {
    uint16_t* H = static_cast<uint16_t*>(Cout);
#pragma unroll
    for (int nj = 0; nj < TN; ++nj) {
      const int col = wn * TN * 32 + nj * 32 + col_l;
      if (col >= ncols) continue;
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + mi * 32 + 8 * (r >> 2) + (r & 3);
          if (row < rows) {
            const float g = acc[mi][nj][r], u = acc[mi][nj + TN][r];
            const float h = g / (1.f + __expf(-g)) * u;
            H[(int64_t)(m_start + row) * N + n0 + col] = f32_to_bf16_bits(h);
          }
        }
    }
  } else {
    float* Y = static_cast<float*>(Cout);
#pragma unroll
    for (int nj = 0; nj < TN; ++nj) {
      const int col = wn * TN * 32 + nj * 32 + col_l;
      if (col >= ncols) continue;
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + mi * 32 + 8 * (r >> 2) + (r & 3);
          if (row < rows) Y[(int64_t)(m_start + row) * N + n0 + col] = acc[mi][nj][r];
        }
    }
  }
}

// ---- fp32 path (plain FMA; for fp32 layers, which are small) ---------------
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E;  // offsets[lo] <= r < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void ffn_f32_gateup_kernel(
    const float* __restrict__ Xp, const float* __restrict__ Wg,
    const float* __restrict__ Wu, const int32_t* __restrict__ offsets, int E,
    int d, int dff, float* __restrict__ H) {
  const int r = blockIdx.y;
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= offsets[E] || n >= dff) return;
  const int e = expert_of_row(offsets, E, r);
  const float* x = Xp + (int64_t)r * d;
  const float* wg = Wg + ((int64_t)e * dff + n) * d;
  const float* wu = Wu + ((int64_t)e * dff + n) * d;
  float g = 0.f, u = 0.f;
  for (int i = 0; i < d; ++i) {
    g = fmaf(x[i], wg[i], g);
    u = fmaf(x[i], wu[i], u);
  }
  H[(int64_t)r * dff + n] = g / (1.f + expf(-g)) * u;
}

__global__ __launch_bounds__(256) void ffn_f32_down_kernel(
    const float* __restrict__ H, const float* __restrict__ Wd,
    const int32_t* __restrict__ offsets, int E, int d, int dff,
    float* __restrict__ Y) {
  const int r = blockIdx.y;
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= offsets[E] || n >= d) return;
  const int e = expert_of_row(offsets, E, r);
  const float* h = H + (int64_t)r * dff;
  const float* w = Wd + ((int64_t)e * d + n) * dff;
  float y = 0.f;
  for (int i = 0; i < dff; ++i) y = fmaf(h[i], w[i], y);
  Y[(int64_t)r * d + n] = y;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

template <int MW, int NW, int TM, int TN, bool GATEUP>
hipError_t launch_gemm(const void* A, const void* B0, const void* B1, int N,
                       int K, int E, int64_t R, const int32_t* offsets,
                       const int32_t* mt_prefix, void* C, hipStream_t stream) {
  using Cfg = GemmCfg<MW, NW, TM, TN, GATEUP>;
  auto kern = grouped_gemm_kernel<MW, NW, TM, TN, GATEUP>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
      Cfg::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  // upper bound on M-tiles: every expert may add one partial tile
  const int64_t mt_max = (R + Cfg::BM - 1) / Cfg::BM + std::min<int64_t>(E, R);
  const int64_t n_nt = (N + Cfg::BN - 1) / Cfg::BN;
  const int64_t tiles = mt_max * n_nt;
  const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::LDS_BYTES, stream,
                     static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B0),
                     static_cast<const uint16_t*>(B1), N, K, E, offsets, mt_prefix, C);
  return hipGetLastError();
}

}  // namespace

size_t ffn_scratch_bytes(int64_t R, int E, int d_ff, bool bf16) {
  return align256((size_t)(E + 1) * 4) + align256((size_t)R * d_ff * (bf16 ? 2 : 4));
}

hipError_t launch_grouped_ffn(const void* X_perm, bool bf16,
                              const int32_t* offsets, const void* W_gate,
                              const void* W_up, const void* W_down, int64_t R,
                              int d, int E, int d_ff, bool small_m,
                              float* Y_perm, void* scratch, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  int32_t* mt_prefix = static_cast<int32_t*>(scratch);
  void* H = static_cast<char*>(scratch) + align256((size_t)(E + 1) * 4);
  if (!bf16) {
    const dim3 g1((d_ff + 255) / 256, (unsigned)R), g2((d + 255) / 256, (unsigned)R);
    ffn_f32_gateup_kernel<<<g1, 256, 0, stream>>>(
        static_cast<const float*>(X_perm), static_cast<const float*>(W_gate),
        static_cast<const float*>(W_up), offsets, E, d, d_ff, static_cast<float*>(H));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ffn_f32_down_kernel<<<g2, 256, 0, stream>>>(static_cast<const float*>(H),
                                                static_cast<const float*>(W_down),
                                                offsets, E, d, d_ff, Y_perm);
    return hipGetLastError();
  }
  hipError_t err;
  if (small_m) {
    // 32-row tiles: few rows per expert, the weights dominate the traffic
    ffn_schedule_kernel<<<1, 256, 0, stream>>>(offsets, E, 32, mt_prefix);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    err = launch_gemm<1, 4, 1, 1, true>(X_perm, W_gate, W_up, d_ff, d, E, R, offsets, mt_prefix, H, stream);
    if (err != hipSuccess) return err;
    return launch_gemm<1, 4, 1, 1, false>(H, W_down, nullptr, d, d_ff, E, R, offsets, mt_prefix, Y_perm, stream);
  }
  ffn_schedule_kernel<<<1, 256, 0, stream>>>(offsets, E, 256, mt_prefix);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  err = launch_gemm<2, 4, 4, 1, true>(X_perm, W_gate, W_up, d_ff, d, E, R, offsets, mt_prefix, H, stream);
  if (err != hipSuccess) return err;
  return launch_gemm<2, 4, 4, 2, false>(H, W_down, nullptr, d, d_ff, E, R, offsets, mt_prefix, Y_perm, stream);
}

}  // namespace moe
