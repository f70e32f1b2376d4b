// Permute: per-expert histogram, capacity, exclusive scan (cu_seqlens) and a
// stable counting-sort scatter that writes every kept token copy straight to
// its expert-contiguous row of X_perm.
//
// Method: "Sparsely-Gated MoE 구현 관점에서 살펴보기: Router, Top-k, 부하 분산"
// (molayo1419.me), forward-pipeline steps 2-3 (assign per-expert capacity
// slots, then reorder the tokens in expert order) and section "로드 밸런싱
// 손실과 용량은 별개" (capacity caps one expert's tokens; overflow is
// dropped).  "MoonEP의 계획 코드를 직접 돌려봤습니다" (thakicloud.com),
// sections "이 기술은 무엇인가" (the sender writes each token to its final
// per-expert position -- no separate sort then copy -- and no per-layer host
// round trip for sizes) and "설치 및 통합" (tokens_per_expert, cu_seqlens).
//
// Order: copy (t, j) of expert e ranks after every copy of e from a token
// t' < t (a token never picks one expert twice).  Kept iff rank < C.
//
//   K1 count_rank  256 tokens per workgroup.  Inside a wavefront, the rank
//                  of a copy among the wave's copies of the same expert comes
//                  from ballots over the bits of the expert ids (a lane's
//                  match mask is the AND over bits of the ballot or its
//                  complement), so no atomics decide any order.  Per-wave
//                  counts are combined in LDS into per-block counts.
//   K2 scan        one workgroup: per expert, an exclusive scan over blocks
//                  (in place), the raw count, min(count, C), the exclusive
//                  scan over experts, and the dropped total.
//   K3 scatter     one wavefront per token: destination rows, the inverse
//                  map, then the X row is read once and written to each of
//                  its kept destinations.  Without X_perm (a grouped FFN
//                  that gathers its rows through the inverse map) K3 is
//                  one thread per copy and copies nothing.
//
// Few copies (T*k <= kSmallCopies): one kernel.  Every workgroup ranks all
// copies itself (one copy per lane, 256 per round, token-major), so no
// workgroup waits for another; workgroup 0 publishes counts, offsets, the
// drop count, dest_row and row_token, and each workgroup copies the X rows
// of its own tokens.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kPermThreads = 256;  // tokens per K1 workgroup

template <int KMAX>
__global__ __launch_bounds__(kPermThreads) void count_rank_kernel(
    const int32_t* __restrict__ topk_idx, int T, int E, int k,
    int32_t* __restrict__ local_rank, int32_t* __restrict__ block_counts) {
  __shared__ int32_t wave_cnt[kPermThreads / kWave][256];
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int t = blockIdx.x * kPermThreads + tid;
  const bool valid = t < T;
  for (int i = tid; i < (kPermThreads / kWave) * 256; i += kPermThreads)
    (&wave_cnt[0][0])[i] = 0;

  int e_my[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    e_my[j] = (valid && j < k) ? topk_idx[(int64_t)t * k + j] : -1;

  const int nb = (E <= 1) ? 0 : 32 - __clz(E - 1);  // bits of an expert id
  const uint64_t active = __ballot(valid);
  uint64_t match[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) match[j] = 0;
#pragma unroll
  for (int jo = 0; jo < KMAX; ++jo) {
    if (jo >= k) break;
    uint64_t m[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) m[j] = active;
    for (int b = 0; b < nb; ++b) {
      const uint64_t ones = __ballot(valid && ((e_my[jo] >> b) & 1));
#pragma unroll
      for (int j = 0; j < KMAX; ++j) m[j] &= ((e_my[j] >> b) & 1) ? ones : ~ones;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) match[j] |= m[j];
  }
  __syncthreads();  // wave_cnt zeroed

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank_w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    rank_w[j] = __popcll(match[j] & below);
    if (valid && j < k) {
      const int cnt = __popcll(match[j]);
      if (rank_w[j] == cnt - 1) wave_cnt[wave][e_my[j]] = cnt;  // last lane of e
    }
  }
  __syncthreads();

  // per expert: prefix over the block's waves, block total to global
  for (int e = tid; e < E; e += kPermThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kPermThreads / kWave; ++w) {
      const int c = wave_cnt[w][e];
      wave_cnt[w][e] = run;
      run += c;
    }
    block_counts[(int64_t)blockIdx.x * E + e] = run;
  }
  __syncthreads();
  if (valid) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) local_rank[(int64_t)t * k + j] = wave_cnt[wave][e_my[j]] + rank_w[j];
  }
}

__global__ __launch_bounds__(256) void scan_kernel(
    int32_t* __restrict__ block_counts, int nblk, int E, int C,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ dropped, int32_t* __restrict__ mt_prefix, int tile_code,
    int tile_code2) {
  __shared__ int32_t s_kept[256];
  __shared__ int32_t s_drop[256];
  __shared__ int32_t s_mt[256];
  __shared__ int32_t s_mt2[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    // sixteen blocks' counts are loaded before any is overwritten, so the
    // loads overlap instead of waiting for each other
    for (int b0 = 0; b0 < nblk; b0 += 16) {
      int c[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        c[u] = (b0 + u < nblk) ? block_counts[(int64_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (b0 + u < nblk) block_counts[(int64_t)(b0 + u) * E + e] = run;  // the block's base rank
        run += c[u];
      }
    }
  }
  const int kept = (e < E) ? min(run, C) : 0;
  const int mt = (mt_prefix != nullptr) ? m_tiles(kept, tile_code) : 0;
  const int mt2 = (mt_prefix != nullptr && tile_code2 != 0) ? m_tiles(kept, tile_code2) : 0;
  s_kept[e] = kept;
  s_drop[e] = (e < E) ? run - kept : 0;
  s_mt[e] = mt;
  s_mt2[e] = mt2;
  __syncthreads();
  // inclusive Hillis-Steele scan over 256 entries
  for (int o = 1; o < 256; o <<= 1) {
    const int a = (e >= o) ? s_kept[e - o] : 0;
    const int b = (e >= o) ? s_drop[e - o] : 0;
    const int c = (e >= o) ? s_mt[e - o] : 0;
    const int c2 = (e >= o) ? s_mt2[e - o] : 0;
    __syncthreads();
    s_kept[e] += a;
    s_drop[e] += b;
    s_mt[e] += c;
    s_mt2[e] += c2;
    __syncthreads();
  }
  // the second schedule (tile_code2 != 0) follows the first: mt_prefix + E + 1
  int32_t* mt_prefix2 = (mt_prefix != nullptr && tile_code2 != 0) ? mt_prefix + E + 1 : nullptr;
  if (e < E) {
    counts[e] = run;
    offsets[e] = s_kept[e] - kept;
    if (mt_prefix != nullptr) mt_prefix[e] = s_mt[e] - mt;
    if (mt_prefix2 != nullptr) mt_prefix2[e] = s_mt2[e] - mt2;
    if (e == E - 1) {
      offsets[E] = s_kept[e];
      dropped[0] = s_drop[e];
      if (mt_prefix != nullptr) mt_prefix[E] = s_mt[e];
      if (mt_prefix2 != nullptr) mt_prefix2[E] = s_mt2[e];
    }
  }
}

// One wavefront per token.  VE = elements per 16-byte chunk of a row.
template <int KMAX>
__global__ __launch_bounds__(256) void scatter_kernel(
    const i32x4* __restrict__ X, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ local_rank,
    const int32_t* __restrict__ block_base, const int32_t* __restrict__ offsets,
    int T, int E, int k, int C, int row_chunks, int32_t* __restrict__ dest_row,
    int32_t* __restrict__ row_token, i32x4* __restrict__ X_perm) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  int dest = -1;
  if (lane < k) {
    const int64_t q = (int64_t)t * k + lane;
    const int e = topk_idx[q];
    const int rank = block_base[(int64_t)(t / kPermThreads) * E + e] + local_rank[q];
    if (rank < C) {
      dest = offsets[e] + rank;
      row_token[dest] = t;
    }
    dest_row[q] = dest;
  }
  int dst[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) dst[j] = __shfl(dest, j, kWave);
  const i32x4* src = X + (int64_t)t * row_chunks;
  constexpr int U = 4;
  for (int c0 = 0; c0 < row_chunks; c0 += U * kWave) {
    i32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c < row_chunks) v[u] = src[c];
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k || dst[j] < 0) continue;
      i32x4* out = X_perm + (int64_t)dst[j] * row_chunks;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kWave + lane;
        if (c < row_chunks) out[c] = v[u];
      }
    }
  }
}

// K3 without the row copy: one thread per copy (t, j).
__global__ __launch_bounds__(256) void assign_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ local_rank,
    const int32_t* __restrict__ block_base, const int32_t* __restrict__ offsets, int T,
    int E, int k, int C, int32_t* __restrict__ dest_row, int32_t* __restrict__ row_token) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= (int64_t)T * k) return;
  const int t = (int)(q / k);
  const int e = topk_idx[q];
  const int rank = block_base[(int64_t)(t / kPermThreads) * E + e] + local_rank[q];
  int dest = -1;
  if (rank < C) {
    dest = offsets[e] + rank;
    row_token[dest] = t;
  }
  dest_row[q] = dest;
}

constexpr int kSmallCopies = 2048;

__global__ __launch_bounds__(256) void permute_small_kernel(
    const i32x4* __restrict__ X, const int32_t* __restrict__ topk_idx, int T, int E,
    int k, int C, int row_chunks, int tok_per_block, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ dropped,
    int32_t* __restrict__ dest_row, int32_t* __restrict__ row_token,
    i32x4* __restrict__ X_perm, int32_t* __restrict__ mt_prefix, int tile_code,
    int tile_code2) {
  __shared__ int32_t s_run[256];        // copies of each expert ranked so far
  __shared__ int32_t s_mt[256];         // M-tiles per expert (m_tiles)
  __shared__ int32_t s_mt2[256];        // the same under tile_code2
  __shared__ int32_t s_wcnt[4][256];    // per-wave copies of each expert in a round
  __shared__ int32_t s_off[256];        // kept-row offsets
  __shared__ int32_t s_drop[256];
  __shared__ int32_t s_rank[kSmallCopies];
  __shared__ int32_t s_exp[kSmallCopies];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int n = T * k;
  s_run[tid] = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) s_wcnt[w][tid] = 0;
  __syncthreads();

  const int nb = (E <= 1) ? 0 : 32 - __clz(E - 1);  // bits of an expert id
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < n; c0 += 256) {
    const int q = c0 + tid;
    const bool valid = q < n;
    const int e = valid ? topk_idx[q] : 0;
    // lanes of this wave holding the same expert id: AND over the id's bits
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nb; ++b) {
      const uint64_t ones = __ballot(valid && ((e >> b) & 1));
      m &= ((e >> b) & 1) ? ones : ~ones;
    }
    const int rw = __popcll(m & below), cw = __popcll(m);
    if (valid && rw == cw - 1) s_wcnt[wave][e] = cw;
    __syncthreads();
    if (valid) {
      int r = s_run[e] + rw;
      for (int w = 0; w < wave; ++w) r += s_wcnt[w][e];
      s_rank[q] = r;
      s_exp[q] = e;
    }
    __syncthreads();
    if (tid < E) {
      s_run[tid] += s_wcnt[0][tid] + s_wcnt[1][tid] + s_wcnt[2][tid] + s_wcnt[3][tid];
#pragma unroll
      for (int w = 0; w < 4; ++w) s_wcnt[w][tid] = 0;
    }
    __syncthreads();
  }

  // capacity, exclusive scan of the kept counts, dropped total
  const int cnt = (tid < E) ? s_run[tid] : 0;
  const int kept = min(cnt, C);
  const int mt = (mt_prefix != nullptr) ? m_tiles(kept, tile_code) : 0;
  const int mt2 = (mt_prefix != nullptr && tile_code2 != 0) ? m_tiles(kept, tile_code2) : 0;
  s_off[tid] = kept;
  s_drop[tid] = cnt - kept;
  s_mt[tid] = mt;
  s_mt2[tid] = mt2;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int a = (tid >= o) ? s_off[tid - o] : 0;
    const int b = (tid >= o) ? s_drop[tid - o] : 0;
    const int c = (tid >= o) ? s_mt[tid - o] : 0;
    const int c2 = (tid >= o) ? s_mt2[tid - o] : 0;
    __syncthreads();
    s_off[tid] += a;
    s_drop[tid] += b;
    s_mt[tid] += c;
    s_mt2[tid] += c2;
    __syncthreads();
  }
  int32_t* mt_prefix2 = (mt_prefix != nullptr && tile_code2 != 0) ? mt_prefix + E + 1 : nullptr;
  const int incl = s_off[tid];
  __syncthreads();
  s_off[tid] = incl - kept;  // exclusive
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < E) {
      counts[tid] = cnt;
      offsets[tid] = s_off[tid];
      if (mt_prefix != nullptr) mt_prefix[tid] = s_mt[tid] - mt;
      if (mt_prefix2 != nullptr) mt_prefix2[tid] = s_mt2[tid] - mt2;
    }
    if (tid == E - 1) {
      offsets[E] = incl;
      dropped[0] = s_drop[tid];
      if (mt_prefix != nullptr) mt_prefix[E] = s_mt[tid];
      if (mt_prefix2 != nullptr) mt_prefix2[E] = s_mt2[tid];
    }
    for (int q = tid; q < n; q += 256) {
      const int r = s_rank[q], e = s_exp[q];
      const int dest = (r < C) ? s_off[e] + r : -1;
      dest_row[q] = dest;
      if (dest >= 0) row_token[dest] = q / k;
    }
  }

  // X rows of this workgroup's tokens, one wavefront per (token, slot)
  if (X_perm == nullptr) return;
  const int t0 = blockIdx.x * tok_per_block;
  const int nq = min(tok_per_block, T - t0) * k;
  for (int i = wave; i < nq; i += 4) {
    const int q = t0 * k + i;
    const int r = s_rank[q];
    if (r >= C) continue;
    const int dest = s_off[s_exp[q]] + r;
    const i32x4* src = X + (int64_t)(q / k) * row_chunks;
    i32x4* out = X_perm + (int64_t)dest * row_chunks;
    for (int c = lane; c < row_chunks; c += kWave) out[c] = src[c];
  }
}

template <int KMAX>
hipError_t launch_k(const void* X, bool x_bf16, const int32_t* topk_idx, int T,
                    int d, int E, int k, int C, int32_t* counts,
                    int32_t* offsets, int32_t* dropped, int32_t* dest_row,
                    int32_t* row_token, void* X_perm, int32_t* local_rank,
                    int32_t* block_counts, int32_t* mt_prefix, int tile_code, int tile_code2,
                    hipStream_t stream) {
  const int nblk = (T + kPermThreads - 1) / kPermThreads;
  count_rank_kernel<KMAX><<<nblk, kPermThreads, 0, stream>>>(
      topk_idx, T, E, k, local_rank, block_counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  scan_kernel<<<1, 256, 0, stream>>>(block_counts, nblk, E, C, counts, offsets, dropped,
                                     mt_prefix, tile_code, tile_code2);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (X_perm == nullptr) {
    const int64_t n = (int64_t)T * k;
    assign_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
        topk_idx, local_rank, block_counts, offsets, T, E, k, C, dest_row, row_token);
    return hipGetLastError();
  }
  const int row_chunks = d * (x_bf16 ? 2 : 4) / 16;
  constexpr int kTokPerBlock = 4;
  scatter_kernel<KMAX><<<(T + kTokPerBlock - 1) / kTokPerBlock, kTokPerBlock * kWave, 0, stream>>>(
      static_cast<const i32x4*>(X), topk_idx, local_rank, block_counts, offsets,
      T, E, k, C, row_chunks, dest_row, row_token, static_cast<i32x4*>(X_perm));
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t permute_scratch_bytes(int T, int k, int E) {
  const size_t nblk = (size_t)(T + kPermThreads - 1) / kPermThreads;
  return align256((size_t)T * k * 4) + align256(nblk * E * 4);
}

hipError_t launch_permute(const void* X, bool x_bf16, const int32_t* topk_idx,
                          int T, int d, int E, int k, int C, int32_t* counts,
                          int32_t* offsets, int32_t* dropped, int32_t* dest_row,
                          int32_t* row_token, void* X_perm, void* scratch,
                          int32_t* mt_prefix, int tile_code, hipStream_t stream,
                          int tile_code2) {
  int32_t* local_rank = static_cast<int32_t*>(scratch);
  int32_t* block_counts = reinterpret_cast<int32_t*>(
      static_cast<char*>(scratch) + align256((size_t)T * k * 4));
  if (T == 0) {
    // still publish empty counts/offsets so callers see a consistent state
    scan_kernel<<<1, 256, 0, stream>>>(block_counts, 0, E, C, counts, offsets, dropped,
                                       mt_prefix, tile_code, tile_code2);
    return hipGetLastError();
  }
  if ((int64_t)T * k <= kSmallCopies) {
    const int row_chunks = d * (x_bf16 ? 2 : 4) / 16;
    // tokens per workgroup: at most 256 workgroups; one when no row is copied
    // (workgroup 0 publishes everything else)
    const int tpb = X_perm == nullptr ? T : (T + 255) / 256;
    permute_small_kernel<<<(unsigned)((T + tpb - 1) / tpb), 256, 0, stream>>>(
        static_cast<const i32x4*>(X), topk_idx, T, E, k, C, row_chunks, tpb, counts,
        offsets, dropped, dest_row, row_token, static_cast<i32x4*>(X_perm), mt_prefix, tile_code,
        tile_code2);
    return hipGetLastError();
  }
#define MOE_PERM_CASE(KM)                                                                 \
  if (k <= KM)                                                                            \
    return launch_k<KM>(X, x_bf16, topk_idx, T, d, E, k, C, counts, offsets, dropped,     \
                        dest_row, row_token, X_perm, local_rank, block_counts,       \
                        mt_prefix, tile_code, tile_code2, stream);
  MOE_PERM_CASE(1)
  MOE_PERM_CASE(2)
  MOE_PERM_CASE(4)
  MOE_PERM_CASE(8)
  MOE_PERM_CASE(16)
  MOE_PERM_CASE(32)
#undef MOE_PERM_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
