// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;

#define MOE_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kWave = 64;

// bf16 <-> fp32.  bf16 -> fp32 is exact (the upper half of the fp32 word);
// fp32 -> bf16 rounds to nearest, ties to even (hardware conversion).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

// Buffer resource for raw (unstructured) buffer loads: loads at byte offsets
// >= num_bytes return zero.  Word 3 is the gfx9-family default data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)num_bytes, 0x00020000);
}

// A byte offset that is always outside any buffer resource's range.
constexpr uint32_t kOob = 0x80000000u;

// M-tiles of an expert with `rows` rows under a tile code: tiles of
// (code & 0xFFFF) rows, and a remainder of at most ((code >> 16) & 0xFF) rows
// joins the last full tile instead of taking a tile of its own.  Bits 24-25
// restrict a schedule to one class of experts, so that experts of few and of
// many rows can run on tiles of different heights: kClassSmall keeps the
// experts of at most kClassRows rows, kClassLarge the others; the experts of
// the other class get no tile.
constexpr int kClassRows = 160;
constexpr int kClassSmall = 1 << 24;
constexpr int kClassLarge = 2 << 24;
constexpr int kTallTileCode = 256 | (64 << 16);
__host__ __device__ __forceinline__ int m_tiles(int rows, int code) {
  const int cls = (code >> 24) & 3;
  if ((cls == 1 && rows > kClassRows) || (cls == 2 && rows <= kClassRows)) return 0;
  const int step = code & 0xFFFF, extra = (code >> 16) & 0xFF;
  const int full = rows / step, rem = rows - full * step;
  return (rem == 0 || (full > 0 && rem <= extra)) ? full : full + 1;
}

// Wave-wide reductions (64 lanes) via cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

}  // namespace moe
