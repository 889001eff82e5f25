// Measured ceilings of the chip, reported by the benchmark beside the
// published peaks (2.5 PFLOP/s dense bf16 matrix, 8 TB/s HBM3E): a loop of
// independent bf16 matrix multiply-accumulates, and a streaming device copy.
// They compute nothing of the convolution.
#include "common.h"

namespace trsc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Each wave keeps four 32x32 fp32 accumulators and issues `iters` rounds of
// four independent v_mfma_f32_32x32x16_bf16 (32*32*16*2 flops each). The sum of
// the accumulators is stored so that the loop is not removed.
__global__ __launch_bounds__(256) void mfma_loop(float* out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(float(threadIdx.x & 7) * 0.125f + float(e));
    b[e] = static_cast<__bf16>(float(e) * 0.5f);
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[int64_t(blockIdx.x) * 256 + threadIdx.x] = s;
}

// 16 bytes per lane, grid-stride over n16 16-byte words.
__global__ __launch_bounds__(256) void stream_copy(const uint4* __restrict__ a, uint4* __restrict__ b, int64_t n16) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride) b[i] = a[i];
}

}  // namespace
}  // namespace trsc

extern "C" {

int64_t tr_sparseconv_ceiling_mfma_flops(int grid, int iters) {
  if (grid <= 0 || iters <= 0) return 0;
  return int64_t(grid) * 4 * int64_t(iters) * 4 * (32 * 32 * 16 * 2);
}

int tr_sparseconv_ceiling_mfma(float* out, int grid, int iters, void* stream) {
  if (out == nullptr || grid <= 0 || iters <= 0) return TR_SC_ERR_INVALID_ARG;
  trsc::mfma_loop<<<unsigned(grid), 256, 0, static_cast<hipStream_t>(stream)>>>(out, iters);
  return hipGetLastError() == hipSuccess ? TR_SC_OK : TR_SC_ERR_HIP;
}

int tr_sparseconv_ceiling_copy(const void* src, void* dst, size_t bytes, int grid, void* stream) {
  if (src == nullptr || dst == nullptr || grid <= 0 || bytes % 16 != 0) return TR_SC_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return TR_SC_ERR_INVALID_ARG;
  trsc::stream_copy<<<unsigned(grid), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(src), static_cast<uint4*>(dst), int64_t(bytes / 16));
  return hipGetLastError() == hipSuccess ? TR_SC_OK : TR_SC_ERR_HIP;
}

}  // extern "C"
