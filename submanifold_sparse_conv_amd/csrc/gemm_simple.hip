// Direct (one output element per lane) form of the gather-GEMM. It is the fp32
// path of the library and the bf16 path for channel counts the matrix-core
// kernel does not tile. y[i, co] = sum over taps k with nbr[i][k] = j >= 0 and
// over ci of w[k, ci, co] * x[j, ci] ("Running TRELLIS.2 on a Mac (1/3)",
// sparse 3D convolution paragraph), fp32 fused multiply-adds in (k, ci) order.
#include "common.h"
#include "launch.h"

namespace trsc {
namespace {

constexpr int kThreads = 256;

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void fwd_simple(const int32_t* __restrict__ nbr, int64_t n,
                                                       const void* __restrict__ xv,
                                                       const void* __restrict__ wv,
                                                       void* __restrict__ yv, int c_in, int c_out) {
  const int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= n * c_out) return;
  const int64_t row = e / c_out;
  const int co = int(e - row * c_out);
  float acc = 0.f;
  for (int k = 0; k < 27; ++k) {
    const int32_t j = nbr[row * 27 + k];
    if (j < 0) continue;
    const int64_t xo = int64_t(j) * c_in;
    const int64_t wo = int64_t(k) * c_in * c_out + co;
    for (int ci = 0; ci < c_in; ++ci) {
      float a, b;
      if constexpr (kBf16) {
        a = bf16_to_f32(static_cast<const uint16_t*>(xv)[xo + ci]);
        b = bf16_to_f32(static_cast<const uint16_t*>(wv)[wo + int64_t(ci) * c_out]);
      } else {
        a = static_cast<const float*>(xv)[xo + ci];
        b = static_cast<const float*>(wv)[wo + int64_t(ci) * c_out];
      }
      acc = fmaf(a, b, acc);
    }
  }
  if constexpr (kBf16)
    static_cast<uint16_t*>(yv)[e] = f32_to_bf16_rne(acc);
  else
    static_cast<float*>(yv)[e] = acc;
}

}  // namespace

hipError_t launch_forward_simple_f32(const ConvArgs& a, hipStream_t st) {
  const int64_t total = a.n * a.c_out;
  if (total > 0)
    fwd_simple<false><<<unsigned((total + kThreads - 1) / kThreads), kThreads, 0, st>>>(
        a.nbr, a.n, a.x, a.w, a.y, a.c_in, a.c_out);
  return hipGetLastError();
}

hipError_t launch_forward_simple_bf16(const ConvArgs& a, hipStream_t st) {
  const int64_t total = a.n * a.c_out;
  if (total > 0)
    fwd_simple<true><<<unsigned((total + kThreads - 1) / kThreads), kThreads, 0, st>>>(
        a.nbr, a.n, a.x, a.w, a.y, a.c_in, a.c_out);
  return hipGetLastError();
}

}  // namespace trsc
