// Weight packing for the gather-GEMM: w [27][C_in][C_out] (the pages' tap-major
// layout, "Porting TRELLIS.2 From Python to Rust and Metal", section V) to
// [27][C_out][C_in] half rows, so that a weight slice of one tap and one
// channel stage is a block of contiguous 64- or 128-byte rows; followed by
// the 256 zero bytes that absent neighbours and channels past C_in read.
#include "common.h"
#include "launch.h"

namespace trsc {
namespace {

constexpr int kThreads = 256;

// wp[k][co][ci] = w[k][ci][co], through 64 x 64 LDS tiles; the first
// workgroup also writes the 256 zero bytes after the packed weights (the copy
// source of absent neighbours and of channels past c_in).
__global__ __launch_bounds__(kThreads) void pack_weights(const uint16_t* __restrict__ w,
                                                         uint16_t* __restrict__ wp, int c_in,
                                                         int c_out, uint16_t* __restrict__ zeros) {
  __shared__ uint16_t t[64][65];
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x < 16)
    reinterpret_cast<uint4*>(zeros)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  const int k = blockIdx.z;
  const int ci0 = blockIdx.y * 64, co0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const uint16_t* src = w + int64_t(k) * c_in * c_out;
  uint16_t* dst = wp + int64_t(k) * c_in * c_out;
  for (int y = ty; y < 64; y += 4) {
    const int ci = ci0 + y, co = co0 + tx;
    t[y][tx] = (ci < c_in && co < c_out) ? src[int64_t(ci) * c_out + co] : uint16_t(0);
  }
  __syncthreads();
  for (int y = ty; y < 64; y += 4) {
    const int co = co0 + y, ci = ci0 + tx;
    if (co < c_out && ci < c_in) dst[int64_t(co) * c_in + ci] = t[tx][y];
  }
}

// The same transpose with 16-byte accesses, for channel counts that are
// multiples of 8 and 16-byte aligned arrays: a thread moves two 8-channel
// pieces in, through a 64 x 66 LDS tile (4-byte words, rows 132 bytes apart so
// that the column reads spread over the banks), and two pieces out.
__device__ __forceinline__ void pack_tile_v8(const uint16_t* __restrict__ w, uint16_t* __restrict__ wp, int c_in,
                                             int c_out, uint16_t* __restrict__ zeros, int bx, int by, int k,
                                             uint32_t* t) {
  if (bx == 0 && by == 0 && k == 0 && threadIdx.x < 16)
    reinterpret_cast<uint4*>(zeros)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  const int ci0 = by * 64, co0 = bx * 64;
  const uint16_t* src = w + int64_t(k) * c_in * c_out;
  uint16_t* dst = wp + int64_t(k) * c_in * c_out;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int q = threadIdx.x + kThreads * m;
    const int r = q >> 3, c8 = q & 7;
    const int ci = ci0 + r, co = co0 + 8 * c8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (ci < c_in && co < c_out) v = *reinterpret_cast<const uint4*>(src + int64_t(ci) * c_out + co);
    uint32_t* row = t + r * 33 + 4 * c8;
    row[0] = v.x, row[1] = v.y, row[2] = v.z, row[3] = v.w;
  }
  __syncthreads();
  const uint16_t* th = reinterpret_cast<const uint16_t*>(t);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int q = threadIdx.x + kThreads * m;
    const int r = q >> 3, c8 = q & 7;
    const int co = co0 + r, ci = ci0 + 8 * c8;
    if (co < c_out && ci < c_in) {
      uint32_t o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        o[u] = uint32_t(th[(8 * c8 + 2 * u) * 66 + r]) | (uint32_t(th[(8 * c8 + 2 * u + 1) * 66 + r]) << 16);
      *reinterpret_cast<uint4*>(dst + int64_t(co) * c_in + ci) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

__global__ __launch_bounds__(kThreads) void pack_weights_v8(const uint16_t* __restrict__ w,
                                                            uint16_t* __restrict__ wp, int c_in,
                                                            int c_out, uint16_t* __restrict__ zeros) {
  __shared__ uint32_t t[64 * 33];
  pack_tile_v8(w, wp, c_in, c_out, zeros, blockIdx.x, blockIdx.y, blockIdx.z, t);
}

// Fragment piece e of the halo kernel's weight copy (one lane of one
// fragment, 8 input channels of one output column) gathered from w
// [27][c_in][c_out]: 8 two-byte loads, consecutive lanes on consecutive columns.
__device__ __forceinline__ uint4 frag_piece_from_w(const uint16_t* __restrict__ w, int c_in, int c_out, int64_t e) {
  const int ncb = c_out / 32;
  const int lane = int(e & 63);
  int64_t f = e >> 6;
  const int cb = int(f % ncb);
  f /= ncb;
  const int s = int(f & 1);
  f >>= 1;
  const int k = int(f % 27);
  const int c = int(f / 27);
  const int col = cb * 32 + (lane & 31);
  const int ci = c * 32 + s * 16 + (lane >> 5) * 8;
  const uint16_t* src = w + (int64_t(k) * c_in + ci) * c_out + col;
  uint32_t o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o[u] = uint32_t(src[(2 * u) * int64_t(c_out)]) | (uint32_t(src[(2 * u + 1) * int64_t(c_out)]) << 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Both layouts of a halo shape in one launch: the first nv8 workgroups pack
// [27][c_out][c_in] tiles as pack_weights_v8, the rest write the fragment
// copy straight from w.
__global__ __launch_bounds__(kThreads) void pack_weights_v8_frag(const uint16_t* __restrict__ w,
                                                                 uint16_t* __restrict__ wp, int c_in, int c_out,
                                                                 uint16_t* __restrict__ zeros, uint4* __restrict__ wf,
                                                                 int nbx, int nby, int nv8, int64_t total) {
  __shared__ uint32_t t[64 * 33];
  const int b = blockIdx.x;
  if (b < nv8) {
    pack_tile_v8(w, wp, c_in, c_out, zeros, b % nbx, (b / nbx) % nby, b / (nbx * nby), t);
    return;
  }
  for (int64_t e = int64_t(b - nv8) * kThreads + threadIdx.x; e < total; e += int64_t(gridDim.x - nv8) * kThreads)
    wf[e] = frag_piece_from_w(w, c_in, c_out, e);
}

// Fragment-order copy: thread = one lane of one fragment, 16 bytes in and out
// (fragment layout in launch.h, next to halo_shape).
__global__ __launch_bounds__(kThreads) void pack_frag(const uint4* __restrict__ wp, uint4* __restrict__ wf, int c_in,
                                                      int c_out, int64_t total) {
  const int ncb = c_out / 32;
  for (int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x; e < total; e += int64_t(gridDim.x) * kThreads) {
    const int lane = int(e & 63);
    int64_t f = e >> 6;
    const int cb = int(f % ncb);
    f /= ncb;
    const int s = int(f & 1);
    f >>= 1;
    const int k = int(f % 27);
    const int c = int(f / 27);
    const int col = cb * 32 + (lane & 31);
    const int ci = c * 32 + s * 16 + (lane >> 5) * 8;
    wf[e] = wp[((int64_t(k) * c_out + col) * c_in + ci) / 8];
  }
}

}  // namespace

hipError_t launch_pack_frag(void* wp, int c_in, int c_out, hipStream_t st) {
  const int64_t total = int64_t(27) * c_in * c_out / 8;  // 16-byte pieces
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  uint16_t* base = static_cast<uint16_t*>(wp);
  pack_frag<<<unsigned(blocks < 4096 ? blocks : 4096), kThreads, 0, st>>>(
      reinterpret_cast<const uint4*>(base), reinterpret_cast<uint4*>(base + frag_weight_offset(c_in, c_out)), c_in,
      c_out, total);
  return hipGetLastError();
}

hipError_t launch_pack_weights(const void* w, void* wp, int c_in, int c_out, hipStream_t st) {
  dim3 grid(unsigned((c_out + 63) / 64), unsigned((c_in + 63) / 64), 27);
  const uint16_t* src = static_cast<const uint16_t*>(w);
  uint16_t* dst = static_cast<uint16_t*>(wp);
  uint16_t* zeros = dst + packed_weight_elems(c_in, c_out);
  const bool v8 = c_in % 8 == 0 && c_out % 8 == 0 && reinterpret_cast<uintptr_t>(w) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(wp) % 16 == 0;
  if (v8 && halo_shape(c_in, c_out)) {
    const int nbx = int(grid.x), nby = int(grid.y), nv8 = nbx * nby * 27;
    const int64_t total = int64_t(27) * c_in * c_out / 8;  // 16-byte fragment pieces
    const int64_t nf = (total + kThreads - 1) / kThreads;
    pack_weights_v8_frag<<<unsigned(nv8 + (nf < 2048 ? nf : 2048)), kThreads, 0, st>>>(
        src, dst, c_in, c_out, zeros, reinterpret_cast<uint4*>(dst + frag_weight_offset(c_in, c_out)), nbx, nby, nv8,
        total);
    return hipGetLastError();
  }
  if (v8)
    pack_weights_v8<<<grid, kThreads, 0, st>>>(src, dst, c_in, c_out, zeros);
  else
    pack_weights<<<grid, kThreads, 0, st>>>(src, dst, c_in, c_out, zeros);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !halo_shape(c_in, c_out)) return e;
  return launch_pack_frag(wp, c_in, c_out, st);
}

}  // namespace trsc
