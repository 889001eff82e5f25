// Backward of the submanifold convolution: the gradients of L = sum_i <y[i], dy[i]>.
//
// Every term w[k, ci, co] * x[j, ci] of the forward sum (j = nbr[i][k], the
// per-tap gather -> matmul -> sum of "Running TRELLIS.2 on a Mac (1/3)", sparse
// 3D convolution paragraph) contributes
//   dx[j, ci]     += w[k, ci, co] * dy[i, co]
//   dw[k, ci, co] += x[j, ci]     * dy[i, co].
//
// Data gradient. Voxel i reads j at tap k exactly when j reads i at the mirrored
// tap 26 - k (p_j = p_i + d_k  <=>  p_i = p_j + d_{26-k}), so dx is the forward
// gather-GEMM over the same kernel map with input dy and weights
// w'[k'][co][ci] = w[26 - k'][ci][co]. In the matrix cores' [tap][out][in]
// packing that is w itself with the taps reversed: pack_dgrad below, then the
// forward kernels with the channel counts swapped.
//
// Weight gradient. dw[k] = X_k^T dY: a reduction over the voxel pairs of tap k.
// Workgroups own (tap, 128 x 128 channel tile, range of Morton positions); each
// compacts the positions of its range that have a neighbour at its tap (bit k
// of the neighbour mask) into an LDS pair list, streams 32 pairs per step --
// gathered x rows and dy rows, copied into LDS with global_load_lds -- and
// multiplies them on the matrix cores. Both operands are needed with the pair
// index along K, while rows are stored channel-contiguous: ds_read_b64_tr_b16
// transposes 4 x 4 blocks of 16-bit values on the way out of LDS. Each
// workgroup writes an fp32 partial tile; a second kernel sums the partials of
// every (tap, ci, co) in range order. No atomics: bit-identical on every run.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace trsc {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Weight packing for the data gradient.
// ---------------------------------------------------------------------------
// Half types: wp[k'] = w[26 - k'] ([27][c_in][c_out] is already the forward
// kernels' [tap][out][in] layout for a c_out -> c_in convolution), 16 bytes per
// lane, then the 256 zero bytes the forward kernels read for absent rows.
__global__ __launch_bounds__(kThreads) void pack_dgrad_half(const uint4* __restrict__ w, uint4* __restrict__ wp,
                                                            int64_t per_tap16, int64_t zero_at16) {
  const int64_t total = 27 * per_tap16;
  for (int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x; e < total; e += int64_t(gridDim.x) * kThreads) {
    const int64_t k = e / per_tap16, r = e - k * per_tap16;
    wp[e] = w[(26 - k) * per_tap16 + r];
  }
  if (blockIdx.x == 0 && threadIdx.x < 16) wp[zero_at16 + threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
}

// fp32: the direct kernel reads [tap][in][out], so wp[k'][co][ci] = w[26-k'][ci][co].
__global__ __launch_bounds__(kThreads) void pack_dgrad_f32(const float* __restrict__ w, float* __restrict__ wp,
                                                           int c_in, int c_out) {
  const int64_t total = int64_t(27) * c_in * c_out;
  for (int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x; e < total; e += int64_t(gridDim.x) * kThreads) {
    const int64_t k = e / (int64_t(c_in) * c_out), r = e - k * c_in * c_out;
    const int co = int(r / c_in), ci = int(r - int64_t(co) * c_in);
    wp[e] = w[(26 - k) * c_in * c_out + int64_t(ci) * c_out + co];
  }
}

// ---------------------------------------------------------------------------
// Weight gradient on the matrix cores.
// ---------------------------------------------------------------------------
template <bool F16>
__device__ __forceinline__ f32x4 mma(i16x8 a, i16x8 b, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ i16x4 read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

struct WgradArgs {
  const int32_t* nbr;    // [n, 27] caller order
  const int32_t* grows;  // [n] caller row at each (grouped Morton) position
  const uint32_t* gmask; // [n] neighbour mask at each position
  int64_t n;
  const uint16_t* x;     // [n, c_in]
  const uint16_t* dy;    // [n, c_out]
  const uint16_t* zeros; // >= 16 zero bytes
  float* out;            // [splits][27][c_in][c_out] partials, or dw when splits == 1
  int c_in, c_out;
  int tiles_i, tiles;    // channel tiles along ci, total channel tiles
  int splits;
  int64_t range;         // positions per split
};

// Staged rows hold TC 16-bit channels: TC / 8 chunks of 16 bytes, in pairs of
// 32 bytes. Pair p of row r sits at p ^ rsw(r): the sixteen rows one transpose
// read touches (r = 8g + {0..3}, g = 0..3, or the next four) land on distinct
// 32-byte bank groups in each half of the wave.
template <int TC>
__device__ __forceinline__ int rsw(int r) {
  constexpr int PAIRS = TC / 16;
  return ((r & 3) | (((r >> 3) & 1) << 2)) & (PAIRS - 1);
}
template <int TC>
__device__ __forceinline__ int chunk_pos(int r, int c) {
  return c ^ (rsw<TC>(r) << 1);
}

template <int TI, int TJ, bool F16>
__global__ __launch_bounds__(kThreads, 2) void wgrad_tiles(const WgradArgs p) {
  constexpr int KS = 32;                     // pairs per step (the MFMA K)
  constexpr int FM = TI / 32, FN = TJ / 32;  // 16-wide blocks per wave (2 x 2 waves)
  constexpr int AROW = TI * 2, BROW = TJ * 2;
  constexpr int LIST = 1024;                 // positions compacted per round
  __shared__ __attribute__((aligned(1024))) unsigned char sa0[KS * AROW];
  __shared__ __attribute__((aligned(1024))) unsigned char sa1[KS * AROW];
  __shared__ __attribute__((aligned(1024))) unsigned char sb0[KS * BROW];
  __shared__ __attribute__((aligned(1024))) unsigned char sb1[KS * BROW];
  __shared__ int32_t li[LIST], lj[LIST];
  __shared__ int32_t wcnt[16];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = logical % p.tiles;
  const int rest = logical / p.tiles;
  const int k = rest % 27, s = rest / 27;
  const int ci0 = (tile % p.tiles_i) * TI, co0 = (tile / p.tiles_i) * TJ;
  const int64_t p0 = int64_t(s) * p.range;
  const int64_t p1 = p0 + p.range < p.n ? p0 + p.range : p.n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int L = lane & 15, g = lane >> 4;
  const int c_in = p.c_in, c_out = p.c_out;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  int total = 0;
  // Copy the rows of step st into LDS: gathered x rows (channels ci0..) into
  // sa, dy rows (channels co0..) into sb. One wave instruction fills 1 KB.
  auto issue = [&](int st, unsigned char* a, unsigned char* b) {
    constexpr int ACPR = TI / 8, BCPR = TJ / 8;  // chunks per row
#pragma unroll
    for (int u = 0; u < ACPR / 8; ++u) {
      const int blk = wave + 4 * u;
      const int r = blk * (64 / ACPR) + lane / ACPR, q = lane % ACPR;
      const int c = chunk_pos<TI>(r, q);
      const int pi = st * KS + r;
      const int32_t j = pi < total ? lj[pi] : -1;
      const int ch = ci0 + c * 8;
      const void* gp = (j >= 0 && ch < c_in) ? static_cast<const void*>(p.x + int64_t(j) * c_in + ch)
                                              : static_cast<const void*>(p.zeros);
      copy16_to_lds(gp, a + blk * 1024);
    }
#pragma unroll
    for (int u = 0; u < BCPR / 8; ++u) {
      const int blk = wave + 4 * u;
      const int r = blk * (64 / BCPR) + lane / BCPR, q = lane % BCPR;
      const int c = chunk_pos<TJ>(r, q);
      const int pi = st * KS + r;
      const int32_t i = pi < total ? li[pi] : -1;
      const int ch = co0 + c * 8;
      const void* gp = (i >= 0 && ch < c_out) ? static_cast<const void*>(p.dy + int64_t(i) * c_out + ch)
                                               : static_cast<const void*>(p.zeros);
      copy16_to_lds(gp, b + blk * 1024);
    }
  };
  // A fragment of a 16-channel block: lane (g, L) receives channel 16*blk + L
  // at pairs 8g .. 8g+7, from two transpose reads of four rows each.
  auto frag = [&](const unsigned char* base, int row_bytes, int blk, auto tc) {
    constexpr int TC = decltype(tc)::value;
    const int c = 2 * blk + ((L & 3) >> 1);
    const int half = (L & 1) * 8;
    const int r0 = 8 * g + (L >> 2), r1 = r0 + 4;
    const i16x4 lo = read_tr(base + r0 * row_bytes + chunk_pos<TC>(r0, c) * 16 + half);
    const i16x4 hi = read_tr(base + r1 * row_bytes + chunk_pos<TC>(r1, c) * 16 + half);
    return i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  auto compute = [&](const unsigned char* a, const unsigned char* b) {
    i16x8 av[FM], bv[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) av[i] = frag(a, AROW, wm * FM + i, std::integral_constant<int, TI>{});
#pragma unroll
    for (int j = 0; j < FN; ++j) bv[j] = frag(b, BROW, wn * FN + j, std::integral_constant<int, TJ>{});
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mma<F16>(av[i], bv[j], acc[i][j]);
  };
  auto step = [&](int st, int nsteps, const unsigned char* aC, const unsigned char* bC, unsigned char* aN,
                  unsigned char* bN) {
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("s_barrier" ::: "memory");
    if (st + 1 < nsteps) issue(st + 1, aN, bN);
    compute(aC, bC);
  };

  for (int64_t base = p0; base < p1; base += LIST) {
    // Compact the positions of this round with bit k set, in position order.
    int32_t ri[4], rj[4], rank[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t pos = base + q * kThreads + tid;
      const bool on = pos < p1 && ((p.gmask[pos] >> k) & 1u);
      ri[q] = on ? p.grows[pos] : -1;
      rj[q] = on ? p.nbr[int64_t(ri[q]) * 27 + k] : -1;
      const uint64_t bal = __ballot(on);
      rank[q] = on ? __popcll(bal & ((uint64_t(1) << lane) - 1)) : -1;
      if (lane == 0) wcnt[q * 4 + wave] = __popcll(bal);
    }
    __syncthreads();
    int before[4];
    total = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = wcnt[e];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (e == q * 4 + wave) before[q] = total;
      total += c;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (rank[q] >= 0) {
        li[before[q] + rank[q]] = ri[q];
        lj[before[q] + rank[q]] = rj[q];
      }
    __syncthreads();

    const int nsteps = (total + KS - 1) / KS;
    if (nsteps > 0) issue(0, sa0, sb0);
    for (int st = 0; st < nsteps; st += 2) {
      step(st, nsteps, sa0, sb0, sa1, sb1);
      if (st + 1 < nsteps) step(st + 1, nsteps, sa1, sb1, sa0, sb0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // the list and the buffers are free for the next round
  }

  // D lane layout: rows (channels ci) 4g + e of the block, column (co) L.
  float* out = p.out + (int64_t(s) * 27 + k) * c_in * c_out;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int co = co0 + (wn * FN + j) * 16 + L;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ci = ci0 + (wm * FM + i) * 16 + 4 * g + e;
        if (ci < c_in && co < c_out) out[int64_t(ci) * c_out + co] = acc[i][j][e];
      }
    }
}

// dw[e] = sum over splits s = 0, 1, ... of part[s][e], in that order.
__global__ __launch_bounds__(kThreads) void wgrad_reduce(const float4* __restrict__ part, float4* __restrict__ dw,
                                                         int64_t n4, int splits) {
  for (int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x; e < n4; e += int64_t(gridDim.x) * kThreads) {
    float4 a = part[e];
    for (int s = 1; s < splits; ++s) {
      const float4 b = part[int64_t(s) * n4 + e];
      a.x += b.x, a.y += b.y, a.z += b.z, a.w += b.w;
    }
    dw[e] = a;
  }
}

__global__ void zero16(uint4* z) {
  if (threadIdx.x < 16) z[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
}

// fp32 weight gradient, one output per lane, voxels in caller order.
__global__ __launch_bounds__(kThreads) void wgrad_f32(const int32_t* __restrict__ nbr, int64_t n,
                                                      const float* __restrict__ x, const float* __restrict__ dy,
                                                      float* __restrict__ dw, int c_in, int c_out) {
  const int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= int64_t(27) * c_in * c_out) return;
  const int k = int(e / (int64_t(c_in) * c_out));
  const int64_t r = e - int64_t(k) * c_in * c_out;
  const int ci = int(r / c_out), co = int(r - int64_t(ci) * c_out);
  float acc = 0.f;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t j = nbr[i * 27 + k];
    if (j >= 0) acc = fmaf(x[int64_t(j) * c_in + ci], dy[i * c_out + co], acc);
  }
  dw[e] = acc;
}

template <int TI, int TJ, bool F16>
hipError_t launch_wgrad_tiles(const WgradArgs& a, hipStream_t st) {
  const int64_t grid = int64_t(a.splits) * 27 * a.tiles;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  wgrad_tiles<TI, TJ, F16><<<unsigned(grid), kThreads, 0, st>>>(a);
  return hipGetLastError();
}

template <bool F16>
hipError_t dispatch_wgrad(const WgradArgs& a, hipStream_t st) {
  if (a.c_in >= 128 && a.c_out >= 128) return launch_wgrad_tiles<128, 128, F16>(a, st);
  if (a.c_in >= 128) return launch_wgrad_tiles<128, 64, F16>(a, st);
  if (a.c_out >= 128) return launch_wgrad_tiles<64, 128, F16>(a, st);
  return launch_wgrad_tiles<64, 64, F16>(a, st);
}

}  // namespace

WgradPlan plan_wgrad(int64_t n, int c_in, int c_out) {
  WgradPlan pl;
  pl.ti = c_in >= 128 ? 128 : 64;
  pl.tj = c_out >= 128 ? 128 : 64;
  pl.tiles_i = (c_in + pl.ti - 1) / pl.ti;
  pl.tiles = pl.tiles_i * ((c_out + pl.tj - 1) / pl.tj);
  // About 1024 workgroups (four per CU), each over at least 4096 positions.
  const int64_t want = (1024 + 27 * pl.tiles - 1) / (27 * pl.tiles);
  const int64_t most = (n + 4095) / 4096;
  pl.splits = int(want < most ? want : most);
  if (pl.splits < 1) pl.splits = 1;
  pl.range = (n + pl.splits - 1) / pl.splits;
  pl.partial_bytes = pl.splits > 1 ? size_t(pl.splits) * 27 * size_t(c_in) * size_t(c_out) * 4 : 0;
  return pl;
}

hipError_t launch_pack_dgrad(const void* w, void* wp, int c_in, int c_out, int dtype, hipStream_t st) {
  const int64_t elems = int64_t(27) * c_in * c_out;
  const int64_t blocks = (elems + 8 * kThreads - 1) / (8 * kThreads);
  const unsigned grid = unsigned(blocks < 4096 ? (blocks > 0 ? blocks : 1) : 4096);
  if (dtype == TR_SC_F32) {
    pack_dgrad_f32<<<grid, kThreads, 0, st>>>(static_cast<const float*>(w), static_cast<float*>(wp), c_in, c_out);
  } else {
    // c_in * c_out is a multiple of 64 (both multiples of 8): whole 16-byte chunks per tap
    pack_dgrad_half<<<grid, kThreads, 0, st>>>(static_cast<const uint4*>(w), static_cast<uint4*>(wp),
                                               int64_t(c_in) * c_out / 8, packed_weight_elems(c_out, c_in) / 8);
    // the data gradient is a c_out -> c_in convolution
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !halo_shape(c_out, c_in)) return e;
    return launch_pack_frag(wp, c_out, c_in, st);
  }
  return hipGetLastError();
}

hipError_t launch_wgrad(const WgradCall& c, hipStream_t st) {
  if (c.dtype == TR_SC_F32) {
    const int64_t total = int64_t(27) * c.c_in * c.c_out;
    wgrad_f32<<<unsigned((total + kThreads - 1) / kThreads), kThreads, 0, st>>>(
        c.nbr, c.n, static_cast<const float*>(c.x), static_cast<const float*>(c.dy), c.dw, c.c_in, c.c_out);
    return hipGetLastError();
  }
  const WgradPlan pl = plan_wgrad(c.n, c.c_in, c.c_out);
  uint16_t* zeros = static_cast<uint16_t*>(c.zeros);
  zero16<<<1, 64, 0, st>>>(static_cast<uint4*>(c.zeros));
  WgradArgs a{c.nbr, c.grows, c.gmask, c.n, static_cast<const uint16_t*>(c.x), static_cast<const uint16_t*>(c.dy),
              zeros, pl.splits > 1 ? c.partials : c.dw, c.c_in, c.c_out, pl.tiles_i, pl.tiles, pl.splits, pl.range};
  hipError_t e = c.dtype == TR_SC_F16 ? dispatch_wgrad<true>(a, st) : dispatch_wgrad<false>(a, st);
  if (e != hipSuccess || pl.splits == 1) return e;
  const int64_t n4 = int64_t(27) * c.c_in * c.c_out / 4;
  const int64_t blocks = (n4 + kThreads - 1) / kThreads;
  wgrad_reduce<<<unsigned(blocks < 8192 ? blocks : 8192), kThreads, 0, st>>>(
      reinterpret_cast<const float4*>(c.partials), reinterpret_cast<float4*>(c.dw), n4, pl.splits);
  return hipGetLastError();
}

}  // namespace trsc
