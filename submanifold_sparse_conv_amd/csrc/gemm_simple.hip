// Direct (one output element per lane) form of the gather-GEMM: the fp32 path
// of the library. y[i, co] = sum over taps k with nbr[i][k] = j >= 0 and
// over ci of w[k, ci, co] * x[j, ci] ("Running TRELLIS.2 on a Mac (1/3)",
// sparse 3D convolution paragraph), fp32 fused multiply-adds in (k, ci) order.
#include "common.h"
#include "launch.h"

namespace trsc {
namespace {

constexpr int kThreads = 256;

// fp32 x, w, y; the fused epilogue of the matrix-core path, in fp32:
// y = act(sum + bias) + residual.
__global__ __launch_bounds__(kThreads) void fwd_simple(const int32_t* __restrict__ nbr, int64_t n,
                                                       const float* __restrict__ x,
                                                       const float* __restrict__ w, float* y, int c_in,
                                                       int c_out, const float* __restrict__ bias,
                                                       const float* residual, int act) {
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
    for (int ci = 0; ci < c_in; ++ci) acc = fmaf(x[xo + ci], w[wo + int64_t(ci) * c_out], acc);
  }
  float v = activate(acc + (bias != nullptr ? bias[co] : 0.f), act);
  if (residual != nullptr) v += residual[e];
  y[e] = v;
}

}  // namespace

hipError_t launch_forward_simple_f32(const ConvArgs& a, hipStream_t st) {
  const int64_t total = a.n * a.c_out;
  if (total > 0)
    fwd_simple<<<unsigned((total + kThreads - 1) / kThreads), kThreads, 0, st>>>(
        a.nbr, a.n, static_cast<const float*>(a.x), static_cast<const float*>(a.w),
        static_cast<float*>(a.y), a.c_in, a.c_out, a.epi.bias, static_cast<const float*>(a.epi.residual),
        a.epi.act);
  return hipGetLastError();
}

}  // namespace trsc
