// Expert offsets {0, T} for running the grouped FFN as one dense FFN over all
// T rows (the shared expert: one "expert" that owns every row).
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

__global__ void dense_offsets_kernel(int32_t* __restrict__ offsets, int T) {
  if (threadIdx.x < 2) offsets[threadIdx.x] = threadIdx.x == 0 ? 0 : T;
}

}  // namespace

hipError_t launch_dense_offsets(int32_t* offsets, int T, hipStream_t stream) {
  dense_offsets_kernel<<<1, 64, 0, stream>>>(offsets, T);
  return hipGetLastError();
}

}  // namespace moe
