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
//    single bf16 store of H.  256-row tiles use 8 wavefronts (2 x 4) with
//    128 x 64 wave tiles; 160-row tiles (65-160 rows per expert on average)
//    three stages and 8 wavefronts, two per SIMD: for gate/up a SIMD's
//    two waves hold the gate and the up accumulators of one 32-column block
//    (the up wave hands its sums to the gate wave through the LDS for
//    SwiGLU), for the down projection 160 x 32 each; 32-row tiles (few rows
//    per expert) 4.
//    The epilogue writes each 32-row sub-tile into the free LDS stages and
//    stores it with 16-byte stores.
//  * Operands are staged global -> LDS with buffer_load_dwordx4 ... lds (no
//    VGPR round trip), double-buffered, issued by half of the wavefronts so
//    that on every SIMD one wave keeps issuing MFMAs while the other issues
//    loads.  A buffer resource per operand bounds the tile, so rows past an
//    expert's end, columns past N and the K tail read as zero.  LDS rows are
//    128 B (64 bf16 of K); the 16-byte chunks of row R are XOR-swizzled by
//    ((R ^ (R >> 3)) & 7) so the ds_read_b128 fragment reads hit distinct
//    banks (rocprof: no LDS bank conflicts in the K loop).
//  * Ragged tiles (an expert's last rows) run a second instance of the K loop
//    in which each wave only issues the MFMAs of its row sub-tiles that hold
//    rows; the hardware pairs waves w and w + 4 on one SIMD (read from the
//    HW_ID register), and those hold different row halves, so every SIMD
//    keeps working.
//  * Tall tiles: with more than 256 rows per expert on average, an expert's
//    remainder of up to 64 rows joins its last 256-row tile (up to 320 rows,
//    five row sub-tiles per wave) instead of taking a tile of its own, which
//    would stream the whole weight tile again for a few rows.  The tile
//    schedule (m_tiles) and the kernels agree through a tile code.
//  * Two classes: with tall tiles over at least 64 experts, the schedule is
//    written twice, once per class of experts (kept rows up to kClassRows,
//    and more), and the classes run concurrently: 160-row tiles on the
//    library's side stream, tall tiles on the caller's stream.  Every tile
//    kind sums each row in the same K order, so the class split does not
//    change a bit of the result.
//  * Schedule: a one-workgroup kernel turns expert_offsets into a prefix of
//    per-expert M-tile counts.  The grid is a static upper bound; each
//    workgroup finds its (expert, n-tile, m-tile) from the prefix and exits
//    if it has none -- no host round trip.  Tiles are ordered expert-major,
//    an expert's tall tile first (longest first), then in bands of eight
//    M-tiles that walk the N-tiles together, and remapped so that the
//    hardware's round-robin of workgroups over the 8 XCDs gives each XCD a
//    contiguous run of tiles: the tiles sharing one expert's weights and
//    rows share one L2.
//  * Gathered rows (the forward's gate/up GEMM): row r of X_perm is read as
//    row row_token[r] of X itself, so no permuted copy of the input is ever
//    written.  A tile copies its rows' token ids into the LDS (those loads go
//    out before the tile's first weight loads), and each A load of the K
//    loop addresses its source row directly; results are bit-identical to
//    reading X_perm.
//  * fp32 layers run 64 x 64 FMA tiles on the same schedule.
#include "common.h"

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "launch.h"

namespace moe {
namespace {

constexpr int kXcds = 8;
constexpr int kNonTemporal = 2;  // "nt" bit of a buffer load's cache policy

// Tile parameters of the bf16 grouped GEMM (each measured; the record of the
// alternatives is kept with the design notes).
constexpr int kBK = 64;        // 256-row tiles: K per stage
constexpr int kNS = 2;         // 256-row tiles: LDS stages
constexpr int kDTN = 8;        // down GEMM: 32-column sub-tiles per 256-row tile
constexpr int kLW = 4;         // waves that issue the global -> LDS loads
constexpr int kNW = 4;         // waves across N in the 256-row tile (2 x kNW waves)
constexpr int kSNW = 4;        // 32-row tiles: waves across N (one 32-column sub-tile each)
constexpr int kSBK = 64;       // 32-row tiles: K per stage
constexpr int kSNS = 3;        // 32-row tiles: stages
constexpr int kSBAUX = kNonTemporal;  // 32-row tiles: weight loads stream (nt)
constexpr int kWgGroupM = 4;   // weight-gradient tiles: M-tiles per group
constexpr int kGroupM = 8;     // grouped GEMM tiles: M-tiles per band
constexpr int kF8SBK = 128;    // 32-row tiles with FP8 weights: K per stage (128-byte rows)
constexpr int kF8SNS = 2;      // 32-row tiles with FP8 weights: stages
constexpr int kF8SNW = 2;      // 32-row tiles with FP8 weights: 64 output columns (gate/up)
constexpr int kF8DNW = 4;      // 32-row tiles with FP8 weights: 128 columns (down projection)
constexpr int kBntRows = 256;  // 256-row tiles: stream the weights up to this many rows per expert
constexpr int kStreamRows = 160;  // few rows per expert: 160-row tiles, 8 waves, 3 stages
constexpr int kStreamGateNW = 8;  // 160-row gate/up tiles: 8 waves, gate and up of a column block on one SIMD
constexpr int kStreamDownNW = 8;  // 160-row down-projection tiles: 8 waves of 160 x 32 (two per SIMD)
constexpr int kPrefixBytes = 1040;  // LDS copy of the tile prefix (E + 1 <= 257 entries)

// Chunk swizzle of LDS row R (16-byte chunks).  256-byte rows (16 chunks),
// 128-byte rows (8 chunks) and 64-byte rows (4 chunks): 16, 8 or 16
// consecutive rows reading the same logical chunk land on distinct banks under
// both a 32- and a 64-bank LDS.
template <int CPR>
__device__ __forceinline__ uint32_t swz(uint32_t R) {
  if constexpr (CPR == 16) return (R ^ (R >> 2)) & 15u;
  else if constexpr (CPR == 8) return (R ^ (R >> 3)) & 7u;
  else return ((R >> 1) ^ (R >> 3)) & 3u;
}

// Eight FP8 E4M3 codes (little-endian bytes) -> eight bf16 values.  Every
// E4M3 value is exactly representable in bf16: gfx950's scaled conversion
// (v_cvt_scalef32_pk_bf16_fp8, scale 1, so exact) turns two codes into a
// packed bf16 pair in one instruction; the expert's scale is applied to the
// fp32 accumulators instead.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint2 q) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)q.x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)q.x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)q.y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)q.y, 1.0f, true);
  const i32x4 w = {__builtin_bit_cast(int, a), __builtin_bit_cast(int, b),
                   __builtin_bit_cast(int, c), __builtin_bit_cast(int, d)};
  return __builtin_bit_cast(bf16x8, w);
}

// Wait until at most N vector-memory loads of this wave are outstanding,
// and all of its LDS reads have returned, then barrier.  No release fence:
// __syncthreads() would also wait for the loads of the later stages.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  static_assert(N >= 0 && N < 63, "vmcnt holds at most 63 outstanding loads");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Tile schedule(s) from the expert offsets: mt_prefix [E + 1] under
// tile_code and, when tile_code2 != 0, a second one under tile_code2 at
// mt_prefix + E + 1.
__global__ __launch_bounds__(256) void ffn_schedule_kernel(
    const int32_t* __restrict__ offsets, int E, int tile_code,
    int32_t* __restrict__ mt_prefix, int tile_code2 = 0) {
  __shared__ int32_t s[256];
  __shared__ int32_t s2[256];
  const int e = threadIdx.x;
  const int rows = (e < E) ? offsets[e + 1] - offsets[e] : 0;
  const int mt = (e < E) ? m_tiles(rows, tile_code) : 0;
  const int mt2 = (e < E && tile_code2 != 0) ? m_tiles(rows, tile_code2) : 0;
  s[e] = mt;
  s2[e] = mt2;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int a = (e >= o) ? s[e - o] : 0;
    const int b = (e >= o) ? s2[e - o] : 0;
    __syncthreads();
    s[e] += a;
    s2[e] += b;
    __syncthreads();
  }
  if (e < E) mt_prefix[e] = s[e] - mt;
  if (e == E - 1) mt_prefix[E] = s[e];
  if (tile_code2 != 0) {
    int32_t* mt_prefix2 = mt_prefix + E + 1;
    if (e < E) mt_prefix2[e] = s2[e] - mt2;
    if (e == E - 1) mt_prefix2[E] = s2[e];
  }
}

// Operand layouts.  "NT" (row-major along K): A [M][K], B [N][K]; a stage
// holds BM rows of A and BROWS rows of B, each BK elements of K, and the
// fragments are read with ds_read_b128.  "T" (row-major along M or N, i.e.
// K-major: A [K][M], B [K][N]): a stage holds BK rows (one per k) of BM or
// BN elements, and the fragments are read with the gfx950 LDS transpose
// read ds_read_b64_tr_b16 (see lds_frag_tr).  AT / BT select the T layout.
template <int MW, int NW, int TM, int TN, bool GATEUP, int BK, int NS, bool BF8,
          bool AT = false, bool BT = false>
struct GemmCfg {
  static constexpr int NWAVES = MW * NW;
  static constexpr int NT = NWAVES * kWave;
  static constexpr int BM = MW * TM * 32;
  // SPLIT (gate/up, one wave row of 8 waves): waves w < 4 hold the gate
  // accumulators of column block w, waves w + 4 the up accumulators of the
  // same block (the hardware pairs waves w and w + 4 on one SIMD); the up
  // waves hand theirs to the gate waves through the LDS for SwiGLU
  static constexpr bool SPLIT = GATEUP && MW == 1 && NW == 8;
  static constexpr int BN = (SPLIT ? NW / 2 : NW) * TN * 32;  // output columns per tile
  static constexpr int NB = (GATEUP && !SPLIT) ? 2 * TN : TN;  // B sub-tiles per wave
  static constexpr int BROWS = GATEUP ? 2 * BN : BN;  // B rows staged per K step
  // LDS stage: the A region (ROWSA rows of RBA bytes), then the B region
  // (ROWSB rows of RBB bytes; FP8 codes when BF8)
  static constexpr int RBA = AT ? BM * 2 : BK * 2;
  static constexpr int RBB = BT ? BROWS * 2 : (BF8 ? BK : BK * 2);
  static constexpr int ROWSA = AT ? BK : BM;
  static constexpr int ROWSB = BT ? BK : BROWS;
  static constexpr int CPRA = RBA / 16, CPRB = RBB / 16;  // 16-byte chunks per row
  static constexpr int RPIA = 1024 / RBA, RPIB = 1024 / RBB;  // rows per wave-level load
  static constexpr int NIA = ROWSA / RPIA, NIB = ROWSB / RPIB;
  static constexpr int AREG = ROWSA * RBA;
  static constexpr int STAGE = AREG + ROWSB * RBB;
  static constexpr int NINSTR = NIA + NIB;
  // the first LW waves issue the global -> LDS loads (LW <= NWAVES)
  static constexpr int LW = (kLW < NWAVES) ? kLW : NWAVES;
  static constexpr int IPW = NINSTR / LW;
  static_assert(NINSTR % LW == 0, "loads must split evenly over waves");
  static_assert(RBA <= 1024 && RBB <= 1024, "a row must fit one wave-level load");
  static_assert(ROWSA % RPIA == 0 && ROWSB % RPIB == 0 && (BT || BN % RPIB == 0),
                "a load must not straddle operands");
  static_assert((!AT || CPRA >= 16) && (!BT || CPRB >= 16), "T rows: at least 256 bytes");
  static_assert(!(GATEUP && BT) && !(BF8 && BT), "T layout: one bf16 B");
  static constexpr int KSUB = BK / 16;               // MFMA k-steps per stage
  // + the tile prefix, and for gate/up the gathered rows of a tile (mode 6)
  static constexpr int LDS_BYTES = NS * STAGE + kPrefixBytes + (GATEUP ? BM * 4 : 0);
};

// Chunk swizzle of T-layout row R (k index): the four rows a transpose read
// touches at once (R & 3 = 0..3) put their 64 bytes on distinct banks.
__device__ __forceinline__ uint32_t swz_t(uint32_t R) { return (R & 3u) << 2; }

// One 32x32x16 MFMA fragment (8 bf16 of consecutive k for one row m or
// column n per lane) from a T-layout region: LDS row k holds the m (or n)
// values of that k.  ds_read_b64_tr_b16 hands lane l of each 16-lane group
// the element (l % 4) of the 4 elements that lane 4 j + l / 4 addressed, as
// its element j; so lane i of a group addresses row k0 + i / 4 at column
// c0 + 4 (i % 4) and receives k0..k0+3 of column c0 + (its lane) -- the
// second read (rows + 4) completes the 8 values.  p: this lane's address for
// k0 = 0; rb: row bytes.
__device__ __forceinline__ bf16x8 lds_frag_tr(const char* p, uint32_t rb) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 4 * rb));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  const i32x4 w = {(int)a.x, (int)a.y, (int)b.x, (int)b.y};
  return __builtin_bit_cast(bf16x8, w);
}

// This lane's transpose-read address (bytes, k0 = 0) for the 32-wide sub-tile
// starting at column col0 of a T region with rows of rb bytes: lanes 32-63
// take k + 8, lanes 16-31 of each half columns + 16.
__device__ __forceinline__ uint32_t tr_lane_off(int lane, uint32_t col0, uint32_t rb) {
  const uint32_t i = lane & 15;
  const uint32_t row = 8 * (lane >> 5) + (i >> 2);
  const uint32_t col = col0 + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
  return row * rb + (((col >> 3) ^ swz_t(row)) << 4) + (col & 7) * 2;
}

// Kernel arguments.
//   Modes 0-2, 4 (rows grouped by expert): A holds the experts' rows
//   ([R, K] bf16; mode 4: [R, lda]); offsets = row offsets [E + 1];
//   mt_prefix = tile schedule [E + 1].  Modes 0, 1: B0/B1 [E, N, K] bf16 (or
//   FP8 codes).  Mode 2: B0 [E, K, N] (the down projection as stored, read
//   along its rows).  Mode 4: B0, B1 [E, K, N] (gate and up as stored; the
//   two halves of A's K = 2 K), the second half's partial sums go to C1.
//   Mode 5: B0 [E, N, ldb], K = half of A's row (lda = ldb = 2 K), partial
//   sums of the two halves to C and C1.
//   Mode 3 (weight gradient): for expert e, C_e = A_e^T B_e over its rows
//   r in [offsets[e], offsets[e + 1]): A [R, lda] (M = g.M columns used),
//   B0 [R, ldb] (N columns); C rows m < msplit go to C [E, msplit, N], the
//   others to C1 [E, M - msplit, N] (fp32).
struct GemmArgs {
  const uint16_t* A;
  const void* B0;
  const void* B1;
  int N, K, E;
  const int32_t* offsets;
  const int32_t* mt_prefix;
  void* C;
  const float* scales;  // FP8 weights: [E, 3]
  uint16_t* G;          // mode 1: G out; mode 2: G in ([R, N] bf16)
  uint16_t* U;          // mode 1: U out; mode 2: U in
  int M, lda, ldb, msplit;  // mode 3 (lda also modes 4, 5; ldb mode 5)
  void* C1;                 // modes 3-5
  const int32_t* gather;    // mode 6: source row of A for each row r < offsets[E]
  int gather_rows;          // mode 6: rows of A
};

// A [R, K] bf16 rows; B0/B1 [E, N, K] bf16, or FP8 E4M3 codes when BF8
// (gate/up, or down with B1 unused).  GATEUP: C = H bf16 [R, N].  Otherwise
// C = Y fp32 [R, N].  With FP8 weights, scales [E, 3] (gate, up, down) scale
// the fp32 accumulators before the epilogue; the codes are decoded exactly to
// bf16 for the MFMAs.  BAUX: cache-policy
// bits of the weight loads (kNonTemporal when each weight tile is read by
// about one workgroup: the loads then stream past the caches).
// MODE 0: the forward FFN.  MODE 1 (GATEUP, training forward): also stores
// G = A B0^T and U = A B1^T in bf16.  MODE 2 (backward of the down
// projection): dH = A Wd with Wd read along its rows (T layout); the epilogue
// applies the SwiGLU backward with the saved G and U and stores dG | dU as
// bf16 [R, 2N].  MODE 3: weight gradient, both operands in T layout.
// MODE 4: the two halves of dX_perm = dG Wg + dU Wu as separate tiles (B in
// T layout, fp32 out): half 0 writes dG Wg to C, half 1 dU Wu to C1.
// MODE 5: the down projection split in two K halves the same way (A [R, lda],
// B [E, N, ldb] with K = lda / 2 per half): partial sums to C and C1.
// MODE 6: mode 0's gate/up with the A rows gathered: row r of the expert-
// grouped order is row gather[r] of A ([gather_rows, K], the layer's input
// X), so no permuted copy of the input is written or read.
template <int MW, int NW, int TM, int TN, bool GATEUP, int BK, int NS, int BAUX, bool BF8,
          int MODE_>
__global__ __launch_bounds__(kWave * MW * NW) void grouped_gemm_kernel(const GemmArgs g) {
  constexpr bool GATHER = MODE_ == 6;
  constexpr int MODE = GATHER ? 0 : MODE_;
  static_assert(!GATHER || GATEUP, "mode 6 is a gate/up mode");
  constexpr bool AT = MODE == 3;
  constexpr bool BT = MODE >= 2 && MODE <= 4;
  const uint16_t* __restrict__ A = g.A;
  const void* __restrict__ B0 = g.B0;
  const void* __restrict__ B1 = g.B1;
  const int N = g.N, E = g.E;
  const int32_t* __restrict__ offsets = g.offsets;
  const int32_t* __restrict__ mt_prefix = g.mt_prefix;
  void* __restrict__ Cout = g.C;
  const float* __restrict__ scales = g.scales;
  static_assert(MODE != 1 || GATEUP, "mode 1 is a gate/up mode");
  static_assert(MODE < 2 || MODE == 5 || (!GATEUP && !BF8), "modes 2-4: one bf16 B");
  static_assert(MODE != 5 || !GATEUP, "mode 5 is a down-projection mode");
  using Cfg = GemmCfg<MW, NW, TM, TN, GATEUP, BK, NS, BF8, AT, BT>;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, NB = Cfg::NB, IPW = Cfg::IPW;
  constexpr int NWAVES = Cfg::NWAVES, STAGE = Cfg::STAGE, LW = Cfg::LW;
  constexpr int RBA = Cfg::RBA, RBB = Cfg::RBB, CPRA = Cfg::CPRA, CPRB = Cfg::CPRB;
  constexpr int RPIA = Cfg::RPIA, RPIB = Cfg::RPIB, NIA = Cfg::NIA, AREG = Cfg::AREG;
  constexpr int KSUB = Cfg::KSUB;
  // Tall tiles (TM = 5): M-tiles step by 256 rows, and an expert's last tile
  // also takes a remainder of up to 64 rows (the schedule merges it instead
  // of giving it a tile of its own that would stream the whole weight tile
  // for a few rows).
  constexpr bool TALL = TM == 5 && MW == 2;
  static_assert(!TALL || (NS == 2 && !AT), "tall tiles: 2 stages, NT A");
  constexpr int MSTEP = TALL ? 256 : BM;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int32_t* s_pref = reinterpret_cast<int32_t*>(smem + NS * STAGE);
  int32_t* s_rows = reinterpret_cast<int32_t*>(smem + NS * STAGE + kPrefixBytes);  // GATHER

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

  // ---- which tile is mine --------------------------------------------------
  // e, the tile's first row (m_start: of X_perm / H; mode 3: first column
  // of A) and column n0, its row and column counts, K of the tile (per pass),
  // the element offsets of its first A and B elements, and the row strides.
  int e, m_start, rows, n0, ncols, K;
  int half = 0;  // MODE 4: 0 = dG against the gate projection, 1 = dU against up
  int64_t a_off, b_off;
  uint32_t kbytes, kbytesB;  // A and B row strides in bytes
  const int n_nt = (N + BN - 1) / BN;
  if constexpr (MODE == 3) {
    const int n_mt = (g.M + BM - 1) / BM;
    const int per_e = n_mt * n_nt;
    const int total = E * per_e;
    const int q = (total + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    if (slot >= q) return;
    const int logical = (blockIdx.x % kXcds) * q + slot;
    if (logical >= total) return;
    e = logical / per_e;
    const int local = logical - e * per_e;
    // groups of 4 M-tiles walk the N-tiles together: the 32 tiles an XCD
    // runs at once cover about 4 x 8 (M, N) tiles and share their operands
    const int grp = local / (kWgGroupM * n_nt);
    const int first_m = grp * kWgGroupM;
    const int gsize = min(kWgGroupM, n_mt - first_m);
    const int in_grp = local - grp * kWgGroupM * n_nt;
    const int m_t = first_m + in_grp % gsize, n_t = in_grp / gsize;
    m_start = m_t * BM;
    rows = min(BM, g.M - m_start);
    n0 = n_t * BN;
    ncols = min(BN, N - n0);
    const int r0 = offsets[e];
    K = offsets[e + 1] - r0;
    a_off = (int64_t)r0 * g.lda + m_start;
    b_off = (int64_t)r0 * g.ldb + n0;
    kbytes = (uint32_t)g.lda * 2u;
    kbytesB = (uint32_t)g.ldb * 2u;
  } else {
    for (int i = tid; i <= E; i += Cfg::NT) s_pref[i] = mt_prefix[i];
    __syncthreads();
    // MODES 4, 5: each (expert, n, m) tile twice, once per K half (NH = 2)
    constexpr int NH = (MODE == 4 || MODE == 5) ? 2 : 1;
    const int total = s_pref[E] * n_nt * NH;
    const int q = (total + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    if (slot >= q) return;
    const int logical = (blockIdx.x % kXcds) * q + slot;
    if (logical >= total) return;
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] * n_nt * NH <= logical) lo = mid; else hi = mid;
    }
    e = lo;
    const int mt_e = s_pref[e + 1] - s_pref[e];
    int local = logical - s_pref[e] * n_nt * NH;
    half = local / (mt_e * n_nt);
    local -= half * mt_e * n_nt;
    const int row_end = offsets[e + 1];
    // A tall last M-tile (more than MSTEP rows) is the expert's longest:
    // its N-tiles come first, so a round's longest tiles start early and the
    // last tiles to start are short ones (when the tiles fill the CUs only
    // twice, as the Mixtral-shaped down projection's do, a CU drawing two
    // tall tiles would otherwise set the time).  The other M-tiles follow in
    // bands.
    const bool tall_first = TALL && mt_e > 1 && row_end - (offsets[e] + (mt_e - 1) * MSTEP) > MSTEP;
    int m_t, n_t;
    if (tall_first && local < n_nt) {
      m_t = mt_e - 1;
      n_t = local;
    } else {
      // bands of kGroupM M-tiles walk the N-tiles together, so the tiles an
      // XCD runs at once share a few activation panels and weight tiles (an
      // expert of many M-tiles would otherwise re-read all its rows for
      // every N-tile)
      const int lb = tall_first ? local - n_nt : local;  // index among the banded tiles
      const int mt_b = tall_first ? mt_e - 1 : mt_e;
      const int first_m = lb / (kGroupM * n_nt) * kGroupM;
      const int gsize = min(kGroupM, mt_b - first_m);
      const int in_band = lb - first_m * n_nt;
      m_t = first_m + in_band % gsize;
      n_t = in_band / gsize;
    }
    m_start = offsets[e] + m_t * MSTEP;
    rows = (m_t == mt_e - 1) ? row_end - m_start : MSTEP;
    n0 = n_t * BN;
    ncols = min(BN, N - n0);
    K = g.K;
    if constexpr (MODE == 4 || MODE == 5) {
      a_off = (int64_t)m_start * g.lda + (int64_t)half * K;
      kbytes = (uint32_t)g.lda * 2u;
      if (MODE == 4 && half) B0 = B1;
      if (half) Cout = g.C1;
    } else {
      a_off = GATHER ? 0 : (int64_t)m_start * K;
      kbytes = (uint32_t)K * 2u;
    }
    if constexpr (BT) {
      b_off = (int64_t)e * K * N + n0;
      kbytesB = (uint32_t)N * 2u;
    } else if constexpr (MODE == 5) {
      b_off = ((int64_t)e * N + n0) * g.ldb + (int64_t)half * K;
      kbytesB = (uint32_t)g.ldb * (BF8 ? 1u : 2u);
    } else {
      b_off = ((int64_t)e * N + n0) * K;
      kbytesB = (uint32_t)K * (BF8 ? 1u : 2u);
    }
  }

  // Buffer ranges: NT operands span the tile's rows (rows past them read
  // zero).  T operands span K rows of the full row stride, the last one only
  // up to the tile's valid width, so k >= K and the last row's columns past
  // M or N read zero (nothing past the matrix is touched); in earlier rows
  // the columns past M or N read the next row, which only reaches output
  // rows or columns that the epilogue drops.  Widths are multiples of 8
  // elements: no 16-byte chunk straddles a range end.
  // Gathered A: the whole input (its rows are looked up per tile below).
  const uint32_t a_bytes =
      GATHER ? (uint32_t)g.gather_rows * kbytes
      : AT ? (K > 0 ? (uint32_t)(K - 1) * kbytes + (uint32_t)rows * 2u : 0u)
           : (uint32_t)rows * kbytes - (uint32_t)half * (uint32_t)K * 2u;
  const uint32_t b_bytes =
      BT ? (K > 0 ? (uint32_t)(K - 1) * kbytesB + (uint32_t)ncols * 2u : 0u)
         : (uint32_t)ncols * kbytesB - (uint32_t)half * (uint32_t)K * (BF8 ? 1u : 2u);
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(A + a_off, a_bytes);
  const int64_t boff = b_off * (BF8 ? 1 : 2);  // bytes
  const __amdgpu_buffer_rsrc_t rB0 = make_rsrc(static_cast<const char*>(B0) + boff, b_bytes);
  const __amdgpu_buffer_rsrc_t rB1 =
      GATEUP ? make_rsrc(static_cast<const char*>(B1) + boff, b_bytes) : rB0;

  // ---- per-lane load offsets (one 16-byte chunk per wave-level load) -------
  // Loads 0..NIA-1 fill the A region, the rest the B region.  NT: R is the
  // region-local row (B-local for the swizzle), kcol the first K element of
  // the lane's chunk.  T: R is the k row within the stage.  Computed when
  // the load is issued (a few integer operations) rather than held in
  // registers across the K loop.
  auto load_off = [&](int i) __attribute__((always_inline)) -> uint2 {
    const int qi = wave + LW * i;
    uint32_t voff;
    int kcol;
    if (qi < NIA) {
      const uint32_t R = qi * RPIA + lane / CPRA;
      if constexpr (AT) {
        const uint32_t c = (lane % CPRA) ^ swz_t(R);
        voff = R * kbytes + c * 16;
        kcol = 0;
      } else {
        const uint32_t c = (lane % CPRA) ^ swz<CPRA>(R);
        voff = R * kbytes + c * 16;
        kcol = c * 8;
      }
    } else {
      const uint32_t R = (qi - NIA) * RPIB + lane / CPRB;
      if constexpr (BT) {
        const uint32_t c = (lane % CPRB) ^ swz_t(R);
        voff = R * kbytesB + c * 16;
        kcol = 0;
      } else {
        const uint32_t c = (lane % CPRB) ^ swz<CPRB>(R);
        const uint32_t row = (GATEUP && R >= (uint32_t)BN) ? R - BN : R;
        voff = row * kbytesB + c * 16;
        kcol = c * (BF8 ? 16 : 8);
      }
    }
    return uint2{voff, (uint32_t)kcol};
  };
  // Gathered A: the tile's source rows are requested first (before the
  // weight loads of the first stages, so their latency overlaps them), go to
  // the LDS once, and then each of the wave's A loads keeps its byte offset
  // at k = 0 (the source row's, or one past every buffer for rows past the
  // tile, which read zero).
  constexpr int NAW = GATHER ? (NIA + LW - 1) / LW : 1;
  constexpr int RPT = GATHER ? (BM + Cfg::NT - 1) / Cfg::NT : 1;  // rows per thread
  uint32_t a_gat[NAW];
  int32_t rsrc_row[RPT];
  if constexpr (GATHER) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int r = tid + j * Cfg::NT;
      rsrc_row[j] = r < rows ? g.gather[m_start + r] : -1;
    }
    asm volatile("" ::: "memory");  // the row loads go out before the stage loads
  }
  auto gather_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int r = tid + j * Cfg::NT;
      if (r < BM) s_rows[r] = rsrc_row[j];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NAW; ++i) {
      const int qi = wave + LW * i;
      const uint32_t R = qi * RPIA + lane / CPRA;
      const uint32_t c = (lane % CPRA) ^ swz<CPRA>(R);
      const int src = qi < NIA ? s_rows[R] : -1;
      a_gat[i] = src < 0 ? kOob : (uint32_t)src * kbytes + c * 16;
    }
  };
  const int nk = (K + BK - 1) / BK;
  const bool ktail = (K % BK) != 0;
  // bytes a stage advances along K
  const uint32_t stepA = AT ? (uint32_t)BK * kbytes : (uint32_t)RBA;
  const uint32_t stepB = BT ? (uint32_t)BK * kbytesB : (uint32_t)RBB;

  // part 0: the stage's loads; 1: only its A loads; 2: only its B loads
  auto issue = [&](int stage, int kt, int part) __attribute__((always_inline)) {
    if (LW < NWAVES && wave >= LW) return;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int qi = wave + LW * i;
      const bool is_a = qi < NIA;
      if ((part == 1 && !is_a) || (part == 2 && is_a)) continue;
      // A rows past the tile's rows are not loaded when a whole load (8
      // rows) lies past them: their sub-tiles issue no MFMA, or only for
      // rows that are never stored (a partly filled sub-tile reads stale LDS
      // rows there; MFMA rows are independent).  With two stages every wait
      // is for all of a wave's loads, so the count may vary.
      if (NS == 2 && !AT && is_a && qi * RPIA >= rows) continue;
      const uint2 lo = load_off(i);
      const int kc = (int)lo.y;
      uint32_t vo = ((GATHER && is_a) ? a_gat[i < NAW ? i : 0] : lo.x) +
                    (uint32_t)kt * (is_a ? stepA : stepB);
      const bool t_layout = is_a ? AT : BT;
      if (!t_layout && ktail && kt * BK + kc >= K) vo = kOob;
      char* dst = smem + stage * STAGE + qi * 1024;
      if (is_a)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, MOE_LDS_PTR(dst), 16, vo, 0, 0, 0);
      else if (!GATEUP || (qi - NIA) * RPIB < BN)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB0, MOE_LDS_PTR(dst), 16, vo, 0, 0, BAUX);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB1, MOE_LDS_PTR(dst), 16, vo, 0, 0, BAUX);
    }
  };

  // ---- per-lane fragment read offsets within a stage ------------------------
  // wm = wave / NW: the hardware puts waves w and w + 4 on one SIMD, so each
  // SIMD holds waves of different row halves and skipping the empty row
  // sub-tiles of a ragged tile leaves every SIMD with work.
  const int wm = wave / NW, wn = wave % NW;
  // SPLIT: column block and projection (0 gate, 1 up) of this wave; the
  // B-local first row of the wave's sub-tiles
  constexpr bool SPLIT = Cfg::SPLIT;
  static_assert(!SPLIT || MODE == 0, "split gate/up: forward only");
  const int wq = SPLIT ? wn % (NW / 2) : wn;
  const int half_gu = SPLIT ? wn / (NW / 2) : 0;
  // Rows of the wave's sub-tiles: wave row wm covers rows wm * TM * 32 +
  // 32 mi; a tall kernel's tiles of at most 256 rows use 4 sub-tiles per
  // wave row (wm * 128 + 32 mi) so the two wave rows stay balanced, and the
  // fifth is placed past every tile row (never read, never stored).
  const int wrows = (TALL && rows <= 256) ? 128 : TM * 32;
  auto sub_row0 = [&](int mi) { return mi * 32 < wrows ? wm * wrows + mi * 32 : 1 << 16; };
  // row sub-tiles of this wave that hold any of the tile's rows (a prefix
  // of 0..TM-1)
  int tm_active = (rows - wm * wrows + 31) / 32;
  tm_active = tm_active < 0 ? 0 : (tm_active > wrows / 32 ? wrows / 32 : tm_active);
  // NT: per (sub-tile, k-step) offsets.  T: per sub-tile offsets at k = 0
  // (k-step ks adds ks * 16 rows).  NT A with 128-byte rows (ACOMPACT):
  // sub-tile mi's rows are 32 mi past sub-tile 0's, which moves its chunk
  // swizzle by 4 when mi is odd, i.e. turns k-step ks into ks ^ 2; so
  // offA(mi, ks) = abase[ks ^ 2 (mi & 1)] + 4096 mi and only abase is held.
  // The same holds for the B sub-tiles (BCOMPACT): sub-tile nj sits bj(nj)
  // 32-row blocks past the wave's first B row.
  constexpr bool ACOMPACT = !AT && CPRA == 8;
  constexpr bool BCOMPACT = !BT && !BF8 && CPRB == 8;
  uint32_t offA[ACOMPACT ? 1 : TM][AT ? 1 : KSUB], offB[BCOMPACT ? 1 : NB][BT ? 1 : KSUB];
  uint32_t abase[KSUB], bbase[KSUB];
  // B sub-tile nj: 32-row blocks past B-local row wn * TN * 32 (gate/up: the
  // up rows start BN rows on)
  auto bj = [](int nj) { return (GATEUP && nj >= TN) ? nj + (NW - 1) * TN : nj; };  // SPLIT: nj < TN
  if constexpr (AT) {
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) offA[mi][0] = tr_lane_off(lane, sub_row0(mi), RBA);
  }
  if constexpr (BT) {
#pragma unroll
    for (int nj = 0; nj < NB; ++nj)
      offB[nj][0] = AREG + tr_lane_off(lane, wn * TN * 32 + nj * 32, RBB);
  }
#pragma unroll
  for (int ks = 0; ks < KSUB; ++ks) {
    const uint32_t c = 2 * ks + (lane >> 5);
    if constexpr (ACOMPACT) {
      const uint32_t R = sub_row0(0) + (lane & 31);
      abase[ks] = R * RBA + ((c ^ swz<CPRA>(R)) * 16);
    } else if constexpr (!AT) {
#pragma unroll
      for (int mi = 0; mi < TM; ++mi) {
        const uint32_t R = sub_row0(mi) + (lane & 31);
        offA[mi][ks] = R * RBA + ((c ^ swz<CPRA>(R)) * 16);
      }
    }
    if constexpr (BCOMPACT) {
      uint32_t R;
      if constexpr (SPLIT) R = half_gu * BN + wq * TN * 32 + (lane & 31);
      else R = wn * TN * 32 + (lane & 31);
      bbase[ks] = AREG + R * RBB + ((c ^ swz<CPRB>(R)) * 16);
    } else if constexpr (!BT) {
#pragma unroll
      for (int nj = 0; nj < NB; ++nj) {
        uint32_t brow;
        if constexpr (SPLIT) brow = half_gu * BN + wq * TN * 32 + nj * 32;
        else if (GATEUP) brow = (nj < TN) ? wn * TN * 32 + nj * 32 : BN + wn * TN * 32 + (nj - TN) * 32;
        else brow = wn * TN * 32 + nj * 32;
        const uint32_t R = brow + (lane & 31);  // B-local row
        if constexpr (BF8)  // 8 codes: half (lane >> 5) of 16-byte chunk ks
          offB[nj][ks] = AREG + R * RBB + ((ks ^ swz<CPRB>(R)) * 16) + (lane >> 5) * 8;
        else
          offB[nj][ks] = AREG + R * RBB + ((c ^ swz<CPRB>(R)) * 16);
      }
    }
  }

  f32x16 acc[TM][NB];
#pragma unroll
  for (int mi = 0; mi < TM; ++mi)
#pragma unroll
    for (int nj = 0; nj < NB; ++nj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.f;

  // NS-stage pipeline: stage kt+NS-1 is requested while stage kt is consumed.
  // NA = the number of row sub-tiles that hold rows, when known at compile
  // time (full tiles; a tall kernel's 256-row tiles): branch-free loops over
  // them.  NA < 0 (ragged tiles): only the tm_active sub-tiles that hold rows
  // issue MFMAs and read their A fragments.
  auto kloop = [&](auto na) {
    constexpr int NA = decltype(na)::value;
    auto active = [&](int mi) { return NA < 0 ? mi < tm_active : mi < NA; };
    if constexpr (!GATHER) {
#pragma unroll
      for (int s = 0; s < NS - 1; ++s)
        if (s < nk) issue(s, s, 0);
    }
    for (int kt = 0; kt < nk; ++kt) {
      // gathered A: the first stages' A loads went out after all their B
      // loads, so the first wait leaves only later stages' A loads pending
      // (the fewest any loading wave has)
      if (GATHER && NS > 2 && kt == 0 && kt + NS - 2 < nk) stage_barrier<NIA / LW * (NS - 2)>();
      else if (kt + NS - 2 < nk) stage_barrier<IPW * (NS - 2)>();
      else stage_barrier<0>();
      if (kt + NS - 1 < nk) issue((kt + NS - 1) % NS, kt + NS - 1, 0);
      const char* st = smem + (kt % NS) * STAGE;
#pragma unroll
      for (int ks = 0; ks < KSUB; ++ks) {
        bf16x8 a[TM], b[NB];
#pragma unroll
        for (int nj = 0; nj < NB; ++nj) {
          if constexpr (BT) b[nj] = lds_frag_tr(st + offB[nj][0] + ks * 16 * RBB, RBB);
          else if constexpr (BF8) b[nj] = fp8x8_to_bf16x8(*reinterpret_cast<const uint2*>(st + offB[nj][ks]));
          else if constexpr (BCOMPACT)
            b[nj] = *reinterpret_cast<const bf16x8*>(st + bbase[ks ^ (2 * (bj(nj) & 1))] + 4096 * bj(nj));
          else b[nj] = *reinterpret_cast<const bf16x8*>(st + offB[nj][ks]);
        }
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
          if (active(mi)) {
            if constexpr (AT) a[mi] = lds_frag_tr(st + offA[mi][0] + ks * 16 * RBA, RBA);
            else if constexpr (ACOMPACT)
              a[mi] = *reinterpret_cast<const bf16x8*>(st + abase[ks ^ (2 * (mi & 1))] + 4096 * mi);
            else a[mi] = *reinterpret_cast<const bf16x8*>(st + offA[mi][ks]);
          }
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
          if (active(mi)) {
#pragma unroll
            for (int nj = 0; nj < NB; ++nj)
              acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[nj], acc[mi][nj], 0, 0, 0);
          }
        // tall kernels (256 VGPRs): all of the k-step's LDS reads, then its
        // MFMAs; left to itself the scheduler waits on each fragment just
        // before its first MFMA (measured: Mixtral layer 2.91 -> 2.78 ms)
        if constexpr (TALL && NA > 0) {
          // DS reads (a transpose-read fragment takes two)
          __builtin_amdgcn_sched_group_barrier(0x100, NA * (AT ? 2 : 1) + NB * (BT ? 2 : 1), 0);
          __builtin_amdgcn_sched_group_barrier(0x008, NA * NB, 0);  // MFMAs
        }
      }
    }
  };
  // gathered A: the first NS - 1 stages' B loads, then the rows, then their
  // A loads (kloop issues the first stages itself otherwise)
  if constexpr (GATHER) {
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < nk) issue(s, s, 2);
    gather_rows();
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < nk) issue(s, s, 1);
  }
  if (tm_active == TM) kloop(std::integral_constant<int, TM>{});
  else if (TM == 5 && tm_active == 4) kloop(std::integral_constant<int, 4>{});
  else kloop(std::integral_constant<int, -1>{});

  // FP8 weights: the expert's scales multiply the accumulators
  if constexpr (BF8) {
    const float s0 = scales[e * 3 + (GATEUP ? 0 : 2)];
    const float s1 = GATEUP ? scales[e * 3 + 1] : s0;
#pragma unroll
    for (int mi = 0; mi < TM; ++mi)
#pragma unroll
      for (int nj = 0; nj < NB; ++nj)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[mi][nj][r] *= (SPLIT ? half_gu == 1 : (GATEUP && nj >= TN)) ? s1 : s0;
  }

  // ---- epilogue ---------------------------------------------------------------
  // acc[mi][nj][r] is element (row, col) of the tile with
  //   row = wm*TM*32 + mi*32 + 8*(r/4) + 4*(lane/32) + r%4,  col = lane%32 (+ sub-tile base)
  const int col_l = lane & 31;
  const int rlane = 4 * (lane >> 5);
  // SwiGLU: silu(g) u = g u / (1 + e^-g), the quotient by the hardware
  // reciprocal (within 1 ulp of fp32, far below the bf16 rounding of H that
  // follows; for large -g, e^-g = inf gives 0 as the division would).  Two
  // transcendental instructions per element run at a quarter of the VALU
  // rate, so the division's correction steps were a visible part of the
  // epilogue.
  if constexpr (GATEUP && MODE == 0) {
    // H goes out through the LDS, one row sub-tile at a time: the wave writes
    // its 32 x TN*32 block of bf16 row-major (rows padded by 32 bytes, so the
    // two row groups of one LDS write fall on different banks), then stores
    // it with 16 bytes per lane, 16 / TN rows of TN*64 contiguous bytes per
    // instruction -- an eighth of the instructions of 2-byte stores.
    constexpr int RS = TN * 64 + 32;  // staged row stride (bytes)
    constexpr int CPRW = TN * 4;      // 16-byte chunks per staged row
    constexpr int RPI = kWave / CPRW;  // rows per store instruction
    static_assert(NWAVES * 32 * RS <= NS * STAGE, "the staging fits the stages");
    uint16_t* H = static_cast<uint16_t*>(Cout);
    __syncthreads();  // every wave is done with the last stage
    // SPLIT: the up waves' accumulators go to the LDS ([block][mi][r][lane]
    // fp32) and the gate waves read the ones of their block, element for
    // element in their own layout; the up waves are then done
    constexpr int XCH = SPLIT ? (NW / 2) * TM * 16 * kWave * 4 : 0;
    static_assert(XCH + NWAVES * 32 * RS <= NS * STAGE, "exchange and staging fit the stages");
    [[maybe_unused]] const float* xu = reinterpret_cast<const float*>(smem) + wq * TM * 16 * kWave;
    if constexpr (SPLIT) {
      if (half_gu == 1) {
        float* xw = reinterpret_cast<float*>(smem) + wq * TM * 16 * kWave;
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
          if (mi < tm_active)
#pragma unroll
            for (int r = 0; r < 16; ++r) xw[(mi * 16 + r) * kWave + lane] = acc[mi][0][r];
      }
      __syncthreads();
      if (half_gu == 1) return;  // no barrier follows
    }
    char* wreg = SPLIT ? smem + XCH + wave * (32 * RS) : smem + wave * (32 * RS);
    const int rsub = lane / CPRW, ch = lane % CPRW;
    // tile-local first column of the chunk
    const int colc = SPLIT ? wq * TN * 32 + ch * 8 : wn * TN * 32 + ch * 8;
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
      if (mi >= tm_active) continue;  // uniform: no rows of the tile here
#pragma unroll
      for (int nj = 0; nj < TN; ++nj)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float gv = acc[mi][nj][r];
          float u;
          if constexpr (SPLIT) u = xu[(mi * 16 + r) * kWave + lane];  // TN == 1
          else u = acc[mi][nj + TN][r];
          const float h = gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * u;
          const int rl = rlane + 8 * (r >> 2) + (r & 3);
          *reinterpret_cast<uint16_t*>(wreg + rl * RS + (nj * 32 + col_l) * 2) =
              f32_to_bf16_bits(h);
        }
#pragma unroll
      for (int r0 = 0; r0 < 32; r0 += RPI) {
        const int rl = r0 + rsub;
        const int row = sub_row0(mi) + rl;
        const i32x4 v = *reinterpret_cast<const i32x4*>(wreg + rl * RS + ch * 16);
        if (row < rows && colc < ncols)
          *reinterpret_cast<i32x4*>(H + (int64_t)(m_start + row) * N + n0 + colc) = v;
      }
    }
  } else if constexpr (GATEUP) {
    uint16_t* H = static_cast<uint16_t*>(Cout);
#pragma unroll
    for (int nj = 0; nj < TN; ++nj) {
      const int col = wn * TN * 32 + nj * 32 + col_l;
      if (col >= ncols) continue;
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = sub_row0(mi) + rlane + 8 * (r >> 2) + (r & 3);
          if (row < rows) {
            const float gv = acc[mi][nj][r], u = acc[mi][nj + TN][r];
            const float h = gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * u;
            const int64_t o = (int64_t)(m_start + row) * N + n0 + col;
            H[o] = f32_to_bf16_bits(h);
            if constexpr (MODE == 1) {
              g.G[o] = f32_to_bf16_bits(gv);
              g.U[o] = f32_to_bf16_bits(u);
            }
          }
        }
    }
  } else if constexpr (MODE == 2) {
    // SwiGLU backward: dG = dH U silu'(G), dU = dH silu(G) with
    // silu'(z) = s (1 + z (1 - s)), s = 1 / (1 + e^-z).  The saved G and U
    // of each 32x32 sub-tile are staged in LDS with 16-byte loads (a row
    // of 32 values = 4 lanes), then read back in the accumulator layout (4
    // consecutive rows of one column per lane) with the transpose load: lane
    // x of a 16-lane group addresses row x / 4, columns 4 (x % 4)..+3 of its
    // 4x16 block and receives the 4 rows of column (its lane).  Each wave
    // uses its own LDS region (TM sub-tiles x 2 matrices x 2 KB), one column
    // sub-tile at a time.
    // At most four sub-tiles are staged at a time (a tall kernel's fifth
    // is staged after the first four are done): 8 waves x 4 x 4 KB fit the
    // two stages.  Sub-tiles without rows are neither staged nor computed.
    constexpr int CH = TM > 4 ? 4 : TM;
    static_assert(NWAVES * CH * 4096 <= NS * STAGE, "epilogue staging fits the stages");
    uint16_t* dGU = static_cast<uint16_t*>(Cout);
    __syncthreads();  // every wave is done with the last stage
    char* wreg = smem + wave * (CH * 4096);
    const uint32_t gbytes = (uint32_t)rows * (uint32_t)N * 2u;
    const __amdgpu_buffer_rsrc_t rG = make_rsrc(g.G + (int64_t)m_start * N, gbytes);
    const __amdgpu_buffer_rsrc_t rU = make_rsrc(g.U + (int64_t)m_start * N, gbytes);
    const uint32_t i16 = lane & 15;
    // transpose-read address within a 2 KB sub-tile region (k = 8 q added)
    const uint32_t tr_off = (4 * (lane >> 5) + (i16 >> 2)) * 64 + ((lane >> 4) & 1) * 32 +
                            (i16 & 3) * 8;
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
#pragma unroll
    for (int nj = 0; nj < TN; ++nj) {
      const int cb = wn * TN * 32 + nj * 32;  // tile-local first column of the sub-tile
      const int col = cb + col_l;
#pragma unroll
      for (int c0 = 0; c0 < TM; c0 += CH) {
        // the previous chunk's transpose reads are done before its region
        // is written again
        if (nj > 0 || c0 > 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int mi = c0; mi < (c0 + CH < TM ? c0 + CH : TM); ++mi)
          if (mi < tm_active) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t row = sub_row0(mi) + h * 16 + (lane >> 2);
              const uint32_t vo = row * (uint32_t)N * 2u + (uint32_t)(n0 + cb + 8 * (lane & 3)) * 2u;
              char* dg = wreg + (mi - c0) * 4096 + h * 1024;
              __builtin_amdgcn_raw_ptr_buffer_load_lds(rG, MOE_LDS_PTR(dg), 16, vo, 0, 0, 0);
              __builtin_amdgcn_raw_ptr_buffer_load_lds(rU, MOE_LDS_PTR(dg + 2048), 16, vo, 0, 0, 0);
            }
          }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int mi = c0; mi < (c0 + CH < TM ? c0 + CH : TM); ++mi)
          if (mi < tm_active) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const char* pg = wreg + (mi - c0) * 4096 + q * 512 + tr_off;
              const v4s gq = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(pg));
              const v4s uq = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(pg + 2048));
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int r = 4 * q + j;
                const int row = sub_row0(mi) + rlane + 8 * q + j;
                if (row < rows && col < ncols) {
                  const float gv = bf16_bits_to_f32((uint16_t)gq[j]);
                  const float u = bf16_bits_to_f32((uint16_t)uq[j]);
                  const float sg = 1.f / (1.f + __expf(-gv));
                  const float dh = acc[mi][nj][r];
                  const float dgv = dh * u * (sg * (1.f + gv * (1.f - sg)));
                  const float du = dh * (gv * sg);
                  const int64_t o2 = (int64_t)(m_start + row) * (2 * N) + n0 + col;
                  dGU[o2] = f32_to_bf16_bits(dgv);
                  dGU[o2 + N] = f32_to_bf16_bits(du);
                }
              }
            }
          }
      }
    }
  } else {
    // fp32 results through the LDS as for H above: 32 x TN*32 fp32 per row
    // sub-tile (rows padded by 32 bytes), then 16-byte stores, 64 / (TN*8)
    // rows of TN*128 contiguous bytes per instruction.  Mode 3 (weight
    // gradient): C row m of expert e goes to C [E, msplit, N] below msplit,
    // else to C1 [E, M - msplit, N], with non-temporal stores (measured:
    // Mixtral backward 7.16 -> 7.0 ms, DeepSeek-V3 18.3 -> 16.9 ms).
    constexpr int RS = TN * 128 + 32;
    constexpr int CPRW = TN * 8;
    constexpr int RPI = kWave / CPRW;
    static_assert(NWAVES * 32 * RS <= NS * STAGE, "the staging fits the stages");
    float* Y = static_cast<float*>(Cout);
    __syncthreads();  // every wave is done with the last stage
    char* wreg = smem + wave * (32 * RS);
    const int rsub = lane / CPRW, ch = lane % CPRW;
    const int colc = wn * TN * 32 + ch * 4;
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
      if (mi >= tm_active) continue;
#pragma unroll
      for (int nj = 0; nj < TN; ++nj)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = rlane + 8 * (r >> 2) + (r & 3);
          *reinterpret_cast<float*>(wreg + rl * RS + (nj * 32 + col_l) * 4) = acc[mi][nj][r];
        }
#pragma unroll
      for (int r0 = 0; r0 < 32; r0 += RPI) {
        const int rl = r0 + rsub;
        const int row = sub_row0(mi) + rl;
        const f32x4 v = *reinterpret_cast<const f32x4*>(wreg + rl * RS + ch * 16);
        if (row < rows && colc < ncols) {
          float* drow;
          if constexpr (MODE == 3) {
            const int m = m_start + row, ms = g.msplit;
            drow = m < ms ? Y + ((int64_t)e * ms + m) * N
                          : static_cast<float*>(g.C1) + ((int64_t)e * (g.M - ms) + (m - ms)) * N;
          } else {
            drow = Y + (int64_t)(m_start + row) * N;
          }
          if constexpr (MODE == 3)  // weight gradients are written once, not read back here
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(drow + n0 + colc));
          else
            *reinterpret_cast<f32x4*>(drow + n0 + colc) = v;
        }
      }
    }
  }
}

// ---- fp32 path (plain FMA; for fp32 layers, which are small) ---------------
// fp32 layers: the grouped FFN with fp32 FMAs (no fp32 matrix path is worth
// the fixed cost at the sizes fp32 layers run at).  One workgroup per 64 x 64
// output tile of one expert's rows (tile schedule: mt_prefix with 64-row
// tiles), K staged through the LDS 16 at a time; each of the 256 threads
// holds a 4 x 4 block of outputs (gate/up: of both projections, SwiGLU
// applied before the one store of H).  A [R, K] fp32 rows by expert; B0/B1
// [E, N, K] fp32; C [R, N] fp32.  K is a multiple of 4 (rows of 16 bytes).
constexpr int kF32Tile = 64;
template <bool GATEUP>
__global__ __launch_bounds__(256) void ffn_f32_tile_kernel(
    const float* __restrict__ A, const float* __restrict__ B0, const float* __restrict__ B1,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ mt_prefix, int E, int N,
    int K, float* __restrict__ C) {
  constexpr int BM = kF32Tile, BN = kF32Tile, BK = 16, NBM = GATEUP ? 2 : 1;
  __shared__ __attribute__((aligned(16))) float sA[BK][BM + 4];
  __shared__ __attribute__((aligned(16))) float sB[NBM][BK][BN + 4];
  __shared__ int32_t s_pref[257];
  const int tid = threadIdx.x;
  for (int i = tid; i <= E; i += 256) s_pref[i] = mt_prefix[i];
  __syncthreads();
  const int n_nt = (N + BN - 1) / BN;
  const int tile = blockIdx.x;
  if (tile >= s_pref[E] * n_nt) return;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] * n_nt <= tile) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int local = tile - s_pref[e] * n_nt;
  const int m_t = local / n_nt, n_t = local - m_t * n_nt;  // the N-tiles of an M-tile in a row
  const int m_start = offsets[e] + m_t * BM;
  const int rows = min(BM, offsets[e + 1] - m_start);
  const int n0 = n_t * BN;
  const int ncols = min(BN, N - n0);

  // loads: thread -> (row or column tid / 4, four k from (tid % 4) * 4)
  const int lr = tid / 4, lk = (tid % 4) * 4;
  const float* a_row = A + (int64_t)(m_start + lr) * K + lk;
  const float* b_row0 = B0 + ((int64_t)e * N + n0 + lr) * K + lk;
  const float* b_row1 = GATEUP ? B1 + ((int64_t)e * N + n0 + lr) * K + lk : nullptr;
  const int ty = tid / 16, tx = tid % 16;  // outputs rows 4 ty.., columns 4 tx..
  float acc[NBM][4][4];
#pragma unroll
  for (int b = 0; b < NBM; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[b][i][j] = 0.f;
  for (int k0 = 0; k0 < K; k0 += BK) {
    const bool kin = k0 + lk < K;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const f32x4 va = (kin && lr < rows) ? *reinterpret_cast<const f32x4*>(a_row + k0) : z;
    const f32x4 vb0 = (kin && lr < ncols) ? *reinterpret_cast<const f32x4*>(b_row0 + k0) : z;
    f32x4 vb1 = z;
    if constexpr (GATEUP) vb1 = (kin && lr < ncols) ? *reinterpret_cast<const f32x4*>(b_row1 + k0) : z;
    __syncthreads();  // the previous step's reads are done
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sA[lk + i][lr] = va[i];
      sB[0][lk + i][lr] = vb0[i];
      if constexpr (GATEUP) sB[1][lk + i][lr] = vb1[i];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&sA[kk][4 * ty]);
#pragma unroll
      for (int b = 0; b < NBM; ++b) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(&sB[b][kk][4 * tx]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[b][i][j] = fmaf(a[i], w[j], acc[b][i][j]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * ty + i;
    if (r >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 4 * tx + j;
      if (c >= ncols) continue;
      float v = acc[0][i][j];
      if constexpr (GATEUP) v = v / (1.f + expf(-v)) * acc[NBM - 1][i][j];
      C[(int64_t)(m_start + r) * N + n0 + c] = v;
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Modes 0-2: R = rows bound (grid upper bound).  Mode 3: a.M rows of C per
// expert, every (expert, m-tile, n-tile) is a tile.
// mt_cap >= 0: a tighter bound on the schedule's M-tiles than R gives (a
// schedule of one class of experts).
template <int MW, int NW, int TM, int TN, bool GATEUP, int BK, int NS, int BAUX, bool BF8,
          int MODE>
hipError_t launch_gemm_args(const GemmArgs& a, int64_t R, hipStream_t stream,
                            int64_t mt_cap = -1) {
  using Cfg = GemmCfg<MW, NW, TM, TN, GATEUP, BK, NS, BF8>;
  auto kern = grouped_gemm_kernel<MW, NW, TM, TN, GATEUP, BK, NS, BAUX, BF8, MODE>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
      Cfg::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  const int64_t n_nt = (a.N + Cfg::BN - 1) / Cfg::BN;
  int64_t tiles;
  if (MODE == 3) {
    tiles = (int64_t)a.E * ((a.M + Cfg::BM - 1) / Cfg::BM) * n_nt;
  } else {
    // upper bound on M-tiles: every expert may add one partial tile
    constexpr int MSTEP = (TM == 5 && MW == 2) ? 256 : Cfg::BM;  // tall tiles step by 256 rows
    int64_t mt_max = (R + MSTEP - 1) / MSTEP + std::min<int64_t>(a.E, R);
    if (mt_cap >= 0) mt_max = std::min(mt_max, mt_cap);
    tiles = mt_max * n_nt * ((MODE == 4 || MODE == 5) ? 2 : 1);
  }
  const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::LDS_BYTES, stream, a);
  return hipGetLastError();
}

// gather != nullptr (gate/up only): A rows gathered by gather[], A has
// gather_rows rows (mode 6).
template <int MW, int NW, int TM, int TN, bool GATEUP, int BK, int NS, int BAUX, bool BF8 = false>
hipError_t launch_gemm(const void* A, const void* B0, const void* B1, int N,
                       int K, int E, int64_t R, const int32_t* offsets,
                       const int32_t* mt_prefix, void* C, hipStream_t stream,
                       const float* scales = nullptr, const int32_t* gather = nullptr,
                       int gather_rows = 0, int64_t mt_cap = -1) {
  GemmArgs a{};
  a.A = static_cast<const uint16_t*>(A);
  a.B0 = B0;
  a.B1 = B1;
  a.N = N;
  a.K = K;
  a.E = E;
  a.offsets = offsets;
  a.mt_prefix = mt_prefix;
  a.C = C;
  a.scales = scales;
  if constexpr (GATEUP) {
    if (gather != nullptr) {
      a.gather = gather;
      a.gather_rows = gather_rows;
      return launch_gemm_args<MW, NW, TM, TN, GATEUP, BK, NS, BAUX, BF8, 6>(a, R, stream, mt_cap);
    }
  }
  return launch_gemm_args<MW, NW, TM, TN, GATEUP, BK, NS, BAUX, BF8, 0>(a, R, stream, mt_cap);
}

// Y[r] += Y2[r] for the kept rows r < offsets[E] (the two K halves of the
// down projection), 4 values per thread.
__global__ __launch_bounds__(256) void ffn_add_halves_kernel(float* __restrict__ Y,
                                                             const float* __restrict__ Y2,
                                                             const int32_t* __restrict__ offsets,
                                                             int E, int d) {
  const int64_t n4 = (int64_t)offsets[E] * d / 4;
  f32x4* y = reinterpret_cast<f32x4*>(Y);
  const f32x4* y2 = reinterpret_cast<const f32x4*>(Y2);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * 256) {
    const f32x4 a = y[i], b = y2[i];
    y[i] = f32x4{a[0] + b[0], a[1] + b[1], a[2] + b[2], a[3] + b[3]};
  }
}

// The down projection Y = H Wd^T.  Y_half != nullptr: the two K halves run as
// separate tiles (twice as many, so the last round of tiles is fuller), the
// second half's partial sums go to Y_half and are then added into Y.
template <int MW, int NW, int TM, int TN, int BK, int NS, int BAUX, bool BF8>
hipError_t launch_down(const void* H, const void* W_down, int d, int d_ff, int E, int64_t R,
                       const int32_t* offsets, const int32_t* mt_prefix, float* Y_perm,
                       float* Y_half, hipStream_t stream, const float* scales,
                       bool defer = false, int64_t mt_cap = -1) {
  if (Y_half == nullptr)
    return launch_gemm<MW, NW, TM, TN, false, BK, NS, BAUX, BF8>(
        H, W_down, nullptr, d, d_ff, E, R, offsets, mt_prefix, Y_perm, stream, scales, nullptr,
        0, mt_cap);
  GemmArgs a{};
  a.A = static_cast<const uint16_t*>(H);
  a.B0 = W_down;
  a.N = d;
  a.K = d_ff / 2;
  a.E = E;
  a.offsets = offsets;
  a.mt_prefix = mt_prefix;
  a.C = Y_perm;
  a.C1 = Y_half;
  a.scales = scales;
  a.lda = d_ff;
  a.ldb = d_ff;
  hipError_t err = launch_gemm_args<MW, NW, TM, TN, false, BK, NS, BAUX, BF8, 5>(a, R, stream,
                                                                                 mt_cap);
  if (err != hipSuccess || defer) return err;  // defer: the caller adds the halves
  const int64_t n4 = R * d / 4;
  const unsigned grid = (unsigned)std::min<int64_t>((n4 + 255) / 256, 4096);
  ffn_add_halves_kernel<<<grid, 256, 0, stream>>>(Y_perm, Y_half, offsets, E, d);
  return hipGetLastError();
}

size_t prefix_bytes(int E) { return align256((size_t)2 * (E + 1) * 4); }

// The side stream of the two-class grouped FFN and its fork and join events,
// one set per device, made on first use and kept until the process ends.
// g_side_mu also serialises the enqueueing of a fork ... join sequence, so
// calls from several host threads do not interleave their event records.
constexpr int kSideDevices = 64;
constexpr int kTwoClassMinE = 64;  // measured: 128 experts gain, 32 do not
struct SideStream {
  hipStream_t stream;
  hipEvent_t fork, join;
};
std::mutex g_side_mu;
SideStream g_side[kSideDevices];

// The set `side` belongs to (nullptr if it is not one of ours).
const SideStream* side_of(hipStream_t side) {
  for (int i = 0; i < kSideDevices; ++i)
    if (side != nullptr && g_side[i].stream == side) return &g_side[i];
  return nullptr;
}

}  // namespace

bool ffn_split_down(bool bf16, int E, int rows_per_expert, int d, int d_ff) {
  if (!bf16 || rows_per_expert <= 64) return false;
  if (d_ff < 2048 || d_ff % 32 != 0) return false;
  // 256 x 256 tiles of the unsplit GEMM (from the mean rows per expert):
  // split when they fill the 256 CUs fewer than four times and leave the
  // last round at most half full (halves of twice as many tiles then finish
  // sooner; a full last round gains nothing and the halves cost an add)
  const int64_t tiles = (int64_t)E * ((rows_per_expert + 255) / 256) * ((d + 255) / 256);
  const int64_t rem = tiles % 256;
  return tiles < 4 * 256 && rem != 0 && rem <= 128;
}

bool ffn_two_class(bool bf16, bool fp8, int E, int rows_per_expert, int d, int d_ff) {
  // tall tiles (more than 256 rows per expert on average) over enough
  // experts that capacity and routing skew leave many of them with few rows
  return bf16 && !fp8 && E >= kTwoClassMinE && ffn_tile_rows(bf16, rows_per_expert, fp8) == 256 &&
         rows_per_expert > kBntRows && !ffn_split_down(bf16, E, rows_per_expert, d, d_ff);
}

int ffn_tile_code(bool bf16, int rows_per_expert, bool fp8, bool two_class) {
  if (two_class) return kStreamRows | kClassSmall;
  const int bm = ffn_tile_rows(bf16, rows_per_expert, fp8);
  return (bm == 256 && rows_per_expert > kBntRows) ? kTallTileCode : bm;
}

int ffn_tile_code2(bool two_class) { return two_class ? (kTallTileCode | kClassLarge) : 0; }

hipStream_t ffn_side_stream(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kSideDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream& r = g_side[dev];
  if (r.stream == nullptr) {
    // not while `stream` is being captured into a graph (creating a stream
    // is not a capturable call); the next call outside a capture makes it
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
      (void)hipGetLastError();  // not left for a later launch check to find
      return nullptr;
    }
    if (cs != hipStreamCaptureStatusNone) return nullptr;
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) == hipSuccess &&
        hipEventCreateWithFlags(&f, hipEventDisableTiming) == hipSuccess &&
        hipEventCreateWithFlags(&j, hipEventDisableTiming) == hipSuccess) {
      r.stream = s;
      r.fork = f;
      r.join = j;
    } else {
      // one class for this call (e.g. another thread is capturing a graph
      // in a mode that forbids the creation); a later call tries again
      if (j) (void)hipEventDestroy(j);
      if (f) (void)hipEventDestroy(f);
      if (s) (void)hipStreamDestroy(s);
      (void)hipGetLastError();
    }
  }
  return r.stream;
}

int ffn_tile_rows(bool bf16, int rows_per_expert, bool fp8) {
  if (!bf16) return kF32Tile;
  if (rows_per_expert <= 64) return 32;
  if (fp8) return rows_per_expert <= kStreamRows ? kStreamRows : rows_per_expert <= 512 ? 128 : 256;
  return rows_per_expert <= kStreamRows ? kStreamRows : 256;
}

int ffn_train_tile_code(int rows_per_expert) {
  if (rows_per_expert <= 64) return 32;
  return rows_per_expert > kBntRows ? kTallTileCode : 256;
}

float* ffn_half_sums(void* scratch, int64_t R, int E, int d, int d_ff, bool bf16,
                     int rows_per_expert) {
  if (!ffn_split_down(bf16, E, rows_per_expert, d, d_ff)) return nullptr;
  return reinterpret_cast<float*>(static_cast<char*>(scratch) + prefix_bytes(E) +
                                  align256((size_t)R * d_ff * 2));
}

size_t ffn_scratch_bytes(int64_t R, int E, int d, int d_ff, bool bf16, int rows_per_expert) {
  return prefix_bytes(E) + align256((size_t)R * d_ff * (bf16 ? 2 : 4)) +
         (ffn_split_down(bf16, E, rows_per_expert, d, d_ff) ? align256((size_t)R * d * 4) : 0);
}

hipError_t launch_grouped_ffn(const void* X_perm, bool bf16,
                              const int32_t* offsets, const void* W_gate,
                              const void* W_up, const void* W_down, int64_t R,
                              int d, int E, int d_ff, int rows_per_expert,
                              float* Y_perm, void* scratch, bool prefix_ready,
                              hipStream_t stream, const float* w_scales, bool defer,
                              const int32_t* gather, int gather_rows, hipStream_t side) {
  const bool fp8 = w_scales != nullptr;
  const int bm = ffn_tile_rows(bf16, rows_per_expert, fp8);
  const bool small_m = bm == 32;
  if (R == 0) return hipSuccess;
  int32_t* mt_prefix = static_cast<int32_t*>(scratch);
  void* H = static_cast<char*>(scratch) + prefix_bytes(E);
  float* Y_half = ffn_half_sums(scratch, R, E, d, d_ff, bf16, rows_per_expert);
  if (gather != nullptr && (!bf16 || (int64_t)gather_rows * d * 2 > INT32_MAX))
    return hipErrorInvalidValue;  // gathered rows: bf16, one 32-bit buffer range
  if (!bf16) {
    if (!prefix_ready) {
      ffn_schedule_kernel<<<1, 256, 0, stream>>>(offsets, E, kF32Tile, mt_prefix);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    // upper bound on 64-row tiles: every expert may add one partial tile
    const int64_t mt_max = (R + kF32Tile - 1) / kF32Tile + std::min<int64_t>(E, R);
    const int64_t g1 = mt_max * ((d_ff + kF32Tile - 1) / kF32Tile);
    const int64_t g2 = mt_max * ((d + kF32Tile - 1) / kF32Tile);
    if (g1 > 0x7fffffff || g2 > 0x7fffffff) return hipErrorInvalidValue;
    ffn_f32_tile_kernel<true><<<(unsigned)g1, 256, 0, stream>>>(
        static_cast<const float*>(X_perm), static_cast<const float*>(W_gate),
        static_cast<const float*>(W_up), offsets, mt_prefix, E, d_ff, d, static_cast<float*>(H));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ffn_f32_tile_kernel<false><<<(unsigned)g2, 256, 0, stream>>>(
        static_cast<const float*>(H), static_cast<const float*>(W_down), nullptr, offsets,
        mt_prefix, E, d, d_ff, Y_perm);
    return hipGetLastError();
  }
  hipError_t err;
  if (small_m) {
    // 32-row tiles: few rows per expert, the weights dominate the traffic
    if (!prefix_ready) {
      ffn_schedule_kernel<<<1, 256, 0, stream>>>(offsets, E, 32, mt_prefix);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (fp8) {
      err = launch_gemm<1, kF8SNW, 1, 1, true, kF8SBK, kF8SNS, kSBAUX, true>(X_perm, W_gate, W_up, d_ff, d, E, R, offsets, mt_prefix, H, stream, w_scales, gather, gather_rows);
      if (err != hipSuccess) return err;
      // down: 128 columns, so the H rows (bf16, twice the bytes of a code
      // row) are a third of each stage's loads rather than half
      return launch_gemm<1, kF8DNW, 1, 1, false, kF8SBK, kF8SNS, kSBAUX, true>(H, W_down, nullptr, d, d_ff, E, R, offsets, mt_prefix, Y_perm, stream, w_scales);
    }
    err = launch_gemm<1, kSNW, 1, 1, true, kSBK, kSNS, kSBAUX>(X_perm, W_gate, W_up, d_ff, d, E, R, offsets, mt_prefix, H, stream, nullptr, gather, gather_rows);
    if (err != hipSuccess) return err;
    return launch_gemm<1, kSNW, 1, 1, false, kSBK, kSNS, kSBAUX>(H, W_down, nullptr, d, d_ff, E, R, offsets, mt_prefix, Y_perm, stream);
  }
  const bool two = side != nullptr && ffn_two_class(bf16, fp8, E, rows_per_expert, d, d_ff);
  const int code = ffn_tile_code(bf16, rows_per_expert, fp8, two);
  if (!prefix_ready) {
    ffn_schedule_kernel<<<1, 256, 0, stream>>>(offsets, E, code, mt_prefix, ffn_tile_code2(two));
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (two) {
    // Experts of at most kClassRows rows (schedule mt_prefix) on 160-row
    // tiles that stream their weights three stages deep, on the side stream;
    // the others (schedule mt_prefix + E + 1) on tall tiles on `stream`.  The
    // two launches share the CUs, so neither waits for the other's last
    // round.  Each expert's rows take the same K order on either tile, so the
    // results equal the one-class launch's bit for bit.
    const int32_t* pre_big = mt_prefix + E + 1;
    const int64_t cap_small = std::min<int64_t>(E, R);  // at most one 160-row tile each
    std::lock_guard<std::mutex> lock(g_side_mu);
    const SideStream* ss = side_of(side);
    if (ss == nullptr) return hipErrorInvalidValue;
    if ((err = hipEventRecord(ss->fork, stream)) != hipSuccess) return err;
    if ((err = hipStreamWaitEvent(side, ss->fork, 0)) != hipSuccess) return err;
    err = launch_gemm<2, kNW, 5, 4 / kNW, true, kBK, 2, 0>(X_perm, W_gate, W_up, d_ff, d, E, R, offsets, pre_big, H, stream, nullptr, gather, gather_rows);
    if (err != hipSuccess) return err;
    err = launch_gemm<1, kStreamGateNW, 5, 1, true, kBK, 3, kNonTemporal>(X_perm, W_gate, W_up, d_ff, d, E, R, offsets, mt_prefix, H, side, nullptr, gather, gather_rows, cap_small);
    if (err != hipSuccess) return err;
    err = launch_down<2, kNW, 5, kDTN / kNW, kBK, 2, 0, false>(H, W_down, d, d_ff, E, R, offsets, pre_big, Y_perm, nullptr, stream, nullptr);
    if (err != hipSuccess) return err;
    err = launch_down<1, kStreamDownNW, 5, 8 / kStreamDownNW, kBK, 3, kNonTemporal, false>(H, W_down, d, d_ff, E, R, offsets, mt_prefix, Y_perm, nullptr, side, nullptr, false, cap_small);
    if (err != hipSuccess) return err;
    if ((err = hipEventRecord(ss->join, side)) != hipSuccess) return err;
    return hipStreamWaitEvent(stream, ss->join, 0);
  }
  if (fp8 && bm == kStreamRows) {
    // FP8 weights, up to 160 rows per expert on average (one M-tile for most
    // experts): the 8-wave 160-row tiles of the bf16 path with K = 128 per
    // stage (128-byte code rows), two 72 KB stages
    err = launch_gemm<1, kStreamGateNW, 5, 1, true, 128, 2, kNonTemporal, true>(X_perm, W_gate, W_up, d_ff, d, E, R, offsets, mt_prefix, H, stream, w_scales, gather, gather_rows);
    if (err != hipSuccess) return err;
    return launch_down<1, kStreamDownNW, 5, 8 / kStreamDownNW, 128, 2, kNonTemporal, true>(H, W_down, d, d_ff, E, R, offsets, mt_prefix, Y_perm, Y_half, stream, w_scales, defer);
  }
  if (fp8 && bm == 128) {
    // FP8 weights, 160 to 512 rows per expert: 128-row tiles and K = 128 per
    // stage, so each weight row is read 128 bytes (one cache line) at a time;
    // 64 KB stages, two of them
    err = launch_gemm<2, 4, 2, 1, true, 128, 2, 0, true>(X_perm, W_gate, W_up, d_ff, d, E, R, offsets, mt_prefix, H, stream, w_scales, gather, gather_rows);
    if (err != hipSuccess) return err;
    return launch_down<2, 4, 2, 2, 128, 2, 0, true>(H, W_down, d, d_ff, E, R, offsets, mt_prefix, Y_perm, Y_half, stream, w_scales, defer);
  }
  if (fp8) {
    // FP8 weights, many rows per expert: the tall 256-row tiles of the bf16
    // path (the weight tiles are shared by several M-tiles through L2)
    err = launch_gemm<2, kNW, 5, 4 / kNW, true, kBK, 2, 0, true>(X_perm, W_gate, W_up, d_ff, d, E, R, offsets, mt_prefix, H, stream, w_scales, gather, gather_rows);
    if (err != hipSuccess) return err;
    return launch_down<2, kNW, 5, kDTN / kNW, kBK, 2, 0, true>(H, W_down, d, d_ff, E, R, offsets, mt_prefix, Y_perm, Y_half, stream, w_scales, defer);
  }
  if (bm == kStreamRows) {
    // up to 160 rows per expert on average (one M-tile for most experts):
    // the weights stream once, so the bytes in flight per CU set the rate.
    // 160-row tiles of 128 (gate/up) or 256 (down) columns leave room for
    // three 52 KB stages (two in flight while one is multiplied); 128-byte
    // weight-row pieces per stage, read past the caches.  Both GEMMs run 8
    // waves, two per SIMD, so one wave of a SIMD issues MFMAs while the other
    // waits on its loads: the gate/up tile's gate and up accumulators of a
    // column block sit on the two waves of one SIMD (SwiGLU joins them
    // through the LDS), the down projection's 256 columns are 8 blocks of
    // 32.  DeepSeek-V3-shaped FFN 4.66-4.73 -> 4.64-4.68 ms (down) -> 4.51-
    // 4.52 ms (gate/up), the same sums bit for bit
    err = launch_gemm<1, kStreamGateNW, 5, 1, true, kBK, 3, kNonTemporal>(X_perm, W_gate, W_up, d_ff, d, E, R, offsets, mt_prefix, H, stream, nullptr, gather, gather_rows);
    if (err != hipSuccess) return err;
    return launch_down<1, kStreamDownNW, 5, 8 / kStreamDownNW, kBK, 3, kNonTemporal, false>(H, W_down, d, d_ff, E, R, offsets, mt_prefix, Y_perm, Y_half, stream, nullptr, defer);
  }
  if (rows_per_expert <= kBntRows) {
    // about one M-tile per expert: every weight tile is read once
    err = launch_gemm<2, kNW, 4, 4 / kNW, true, kBK, kNS, kNonTemporal>(X_perm, W_gate, W_up, d_ff, d, E, R, offsets, mt_prefix, H, stream, nullptr, gather, gather_rows);
    if (err != hipSuccess) return err;
    return launch_down<2, kNW, 4, kDTN / kNW, kBK, kNS, kNonTemporal, false>(H, W_down, d, d_ff, E, R, offsets, mt_prefix, Y_perm, Y_half, stream, nullptr, defer);
  }
  // several M-tiles per expert: tall tiles (the schedule merges remainders
  // of up to 64 rows into the expert's last tile)
  err = launch_gemm<2, kNW, 5, 4 / kNW, true, kBK, 2, 0>(X_perm, W_gate, W_up, d_ff, d, E, R, offsets, mt_prefix, H, stream, nullptr, gather, gather_rows);
  if (err != hipSuccess) return err;
  return launch_down<2, kNW, 5, kDTN / kNW, kBK, 2, 0, false>(H, W_down, d, d_ff, E, R, offsets, mt_prefix, Y_perm, Y_half, stream, nullptr, defer);
}

}  // namespace moe

// ---- training forward and backward -----------------------------------------
namespace moe {

hipError_t launch_grouped_ffn_train(const void* X_perm, const int32_t* offsets,
                                    const void* W_gate, const void* W_up, const void* W_down,
                                    int64_t R, int d, int E, int d_ff, int rows_per_expert,
                                    int32_t* mt_prefix, bool prefix_ready, void* H, void* G,
                                    void* U, float* Y_perm, hipStream_t stream) {
  const int bm = rows_per_expert <= 64 ? 32 : 256;
  if (R == 0) return hipSuccess;
  hipError_t err;
  if (!prefix_ready) {
    ffn_schedule_kernel<<<1, 256, 0, stream>>>(offsets, E, ffn_train_tile_code(rows_per_expert),
                                               mt_prefix);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  GemmArgs a{};
  a.A = static_cast<const uint16_t*>(X_perm);
  a.B0 = W_gate;
  a.B1 = W_up;
  a.N = d_ff;
  a.K = d;
  a.E = E;
  a.offsets = offsets;
  a.mt_prefix = mt_prefix;
  a.C = H;
  a.G = static_cast<uint16_t*>(G);
  a.U = static_cast<uint16_t*>(U);
  if (bm == 32) {
    err = launch_gemm_args<1, kSNW, 1, 1, true, kSBK, kSNS, kSBAUX, false, 1>(a, R, stream);
    if (err != hipSuccess) return err;
    return launch_gemm<1, kSNW, 1, 1, false, kSBK, kSNS, kSBAUX>(H, W_down, nullptr, d, d_ff, E, R, offsets, mt_prefix, Y_perm, stream);
  }
  // the down projection as in launch_grouped_ffn (same split, same scratch
  // place for the second K half), so the output equals moe_forward's
  float* Y_half = ffn_half_sums(mt_prefix, R, E, d, d_ff, true, rows_per_expert);
  if (rows_per_expert <= kBntRows) {
    err = launch_gemm_args<2, kNW, 4, 4 / kNW, true, kBK, kNS, kNonTemporal, false, 1>(a, R, stream);
    if (err != hipSuccess) return err;
    return launch_down<2, kNW, 4, kDTN / kNW, kBK, kNS, kNonTemporal, false>(H, W_down, d, d_ff, E, R, offsets, mt_prefix, Y_perm, Y_half, stream, nullptr);
  }
  // tall tiles, with the schedule of ffn_train_tile_code
  err = launch_gemm_args<2, kNW, 5, 4 / kNW, true, kBK, 2, 0, false, 1>(a, R, stream);
  if (err != hipSuccess) return err;
  return launch_down<2, kNW, 5, kDTN / kNW, kBK, 2, 0, false>(H, W_down, d, d_ff, E, R, offsets, mt_prefix, Y_perm, Y_half, stream, nullptr);
}

hipError_t launch_ffn_dgrad(const void* dY_perm, const int32_t* offsets, const void* W_gate,
                            const void* W_up, const void* W_down, const void* G, const void* U,
                            int64_t R, int d, int E, int d_ff, int rows_per_expert,
                            int32_t* mt_prefix, void* dGU, float* dX_perm, hipStream_t stream) {
  const int bm = rows_per_expert <= 64 ? 32 : 256;
  if (R == 0) return hipSuccess;
  // dH and dX run on tall tiles where the training forward does
  const int code = ffn_train_tile_code(rows_per_expert);
  const bool tall = code != bm;
  ffn_schedule_kernel<<<1, 256, 0, stream>>>(offsets, E, code, mt_prefix);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // dH = dY_perm Wd (Wd [E, d, d_ff] read along its rows) -> SwiGLU backward
  GemmArgs a{};
  a.A = static_cast<const uint16_t*>(dY_perm);
  a.B0 = W_down;
  a.N = d_ff;
  a.K = d;
  a.E = E;
  a.offsets = offsets;
  a.mt_prefix = mt_prefix;
  a.C = dGU;
  a.G = const_cast<uint16_t*>(static_cast<const uint16_t*>(G));
  a.U = const_cast<uint16_t*>(static_cast<const uint16_t*>(U));
  // dX_perm = dG Wg + dU Wu (Wg, Wu [E, d_ff, d] read along their rows)
  GemmArgs x{};
  x.A = static_cast<const uint16_t*>(dGU);
  x.B0 = W_gate;
  x.B1 = W_up;
  x.N = d;
  x.K = d_ff;
  x.E = E;
  x.offsets = offsets;
  x.mt_prefix = mt_prefix;
  x.C = dX_perm;
  x.C1 = dX_perm + R * d;  // the second K half's partial sums
  x.lda = 2 * d_ff;
  if (bm == 32) {
    err = launch_gemm_args<1, kSNW, 1, 1, false, kSBK, kSNS, kSBAUX, false, 2>(a, R, stream);
    if (err != hipSuccess) return err;
    return launch_gemm_args<1, kSNW, 1, 1, false, kSBK, kSNS, kSBAUX, false, 4>(x, R, stream);
  }
  if (rows_per_expert <= kBntRows) {
    err = launch_gemm_args<2, kNW, 4, kDTN / kNW, false, kBK, kNS, kNonTemporal, false, 2>(a, R, stream);
    if (err != hipSuccess) return err;
    return launch_gemm_args<2, kNW, 4, kDTN / kNW, false, kBK, kNS, kNonTemporal, false, 4>(x, R, stream);
  }
  if (tall) {
    err = launch_gemm_args<2, kNW, 5, kDTN / kNW, false, kBK, 2, 0, false, 2>(a, R, stream);
    if (err != hipSuccess) return err;
    return launch_gemm_args<2, kNW, 5, kDTN / kNW, false, kBK, 2, 0, false, 4>(x, R, stream);
  }
  err = launch_gemm_args<2, kNW, 4, kDTN / kNW, false, kBK, kNS, 0, false, 2>(a, R, stream);
  if (err != hipSuccess) return err;
  return launch_gemm_args<2, kNW, 4, kDTN / kNW, false, kBK, kNS, 0, false, 4>(x, R, stream);
}

hipError_t launch_wgrad(const void* A, int lda, int M, const void* B, int ldb, int N,
                        const int32_t* offsets, int E, int msplit, float* C0, float* C1,
                        hipStream_t stream) {
  GemmArgs a{};
  a.A = static_cast<const uint16_t*>(A);
  a.B0 = B;
  a.N = N;
  a.E = E;
  a.offsets = offsets;
  a.M = M;
  a.lda = lda;
  a.ldb = ldb;
  a.msplit = msplit;
  a.C = C0;
  a.C1 = C1;
  return launch_gemm_args<2, 4, 4, 2, false, 64, 2, 0, false, 3>(a, 0, stream);
}

}  // namespace moe
