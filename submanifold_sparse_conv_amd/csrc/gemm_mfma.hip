// Gather-GEMM on the matrix cores (bf16 in, fp32 accumulate, bf16 out): the
// compute half of the sparse convolution -- a gather-GEMM over the neighbour
// table with half-precision inputs and single-precision accumulation
// ("Porting TRELLIS.2 From Python to Rust and Metal", section V), i.e. the
// per-kernel-position gather -> matmul -> sum of "Running TRELLIS.2 on a Mac
// (1/3)" (sparse 3D convolution paragraph).
//
// Output-stationary: a workgroup owns a tile of TM voxels (consecutive in
// Morton order) x TN output channels and keeps it in registers for the whole
// reduction over taps and input channels, then writes every row once at the
// voxel's caller index. No atomics, fixed (tap, channel) order: results are
// the same bit for bit on every run.
//
// K loop: the taps some row of the tile needs (OR of the rows' 27-bit
// neighbour masks), each split into KC-wide channel chunks ("stages"). The
// gather indices of every active tap are read once into LDS. Per stage the TM
// gathered feature rows (zero where the neighbour is absent) and the KC x TN
// weight slice are staged in LDS and four waves run v_mfma_f32_16x16x32_bf16
// over their WM x WN sub-tiles, while the next stage's global loads are
// already in flight into registers.
//
// Weights are first re-laid out to [27][C_out][C_in] (input channels
// contiguous), the operand order of the matrix instruction.
#include "common.h"
#include "launch.h"

namespace trsc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// wp[k][co][ci] = w[k][ci][co], through 64 x 64 LDS tiles.
__global__ __launch_bounds__(kThreads) void pack_weights(const uint16_t* __restrict__ w,
                                                         uint16_t* __restrict__ wp, int c_in,
                                                         int c_out) {
  __shared__ uint16_t t[64][65];
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

// Workgroup index -> tile index so that each XCD (workgroups are dealt to the
// 8 XCDs round-robin) works through one contiguous run of tiles, keeping the
// gathered rows of neighbouring tiles in its own L2.
__device__ inline int xcd_tile(int bid, int grid) {
  const int xcd = bid & 7, local = bid >> 3;
  const int per = grid >> 3, rem = grid & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

template <int TM, int TN, int WM, int WN, int KC>
__global__ __launch_bounds__(kThreads) void fwd_mfma(const int32_t* __restrict__ nbr,
                                                     const int32_t* __restrict__ srows,
                                                     const uint32_t* __restrict__ vmask, int64_t n,
                                                     const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ wp,
                                                     uint16_t* __restrict__ y, int c_in, int c_out,
                                                     int n_tiles_n) {
  constexpr int WAVES_N = TN / WN;
  static_assert((TM / WM) * (TN / WN) == kThreads / 64, "four waves");
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int LDK = KC + 8;                          // padded LDS row (bf16 elements)
  constexpr int CPR = KC / 8;                          // 16-byte chunks per staged row
  constexpr int ACH = (TM * CPR + kThreads - 1) / kThreads;  // A chunks per thread
  constexpr int BCH = (TN * CPR + kThreads - 1) / kThreads;  // B chunks per thread
  constexpr int LDO = TN + 8;                          // padded output staging row
  constexpr int STAGE = (TM + TN) * LDK;
  constexpr int OUTS = TM * LDO;
  constexpr int SMEM = STAGE > OUTS ? STAGE : OUTS;
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM];
  __shared__ int32_t s_row[TM];
  __shared__ int32_t s_src[27 * TM];  // gather source row per (active tap, tile row)
  __shared__ int32_t s_taps[27];
  __shared__ uint32_t s_mask;
  uint16_t* sA = smem;
  uint16_t* sB = smem + TM * LDK;

  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t t0 = int64_t(tile / n_tiles_n) * TM;
  const int n0 = (tile % n_tiles_n) * TN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // Prologue: tile rows, the taps some row needs, and all gather indices.
  if (tid == 0) s_mask = 0;
  uint32_t m = 0;
  for (int r = tid; r < TM; r += kThreads) {
    const int64_t t = t0 + r;
    s_row[r] = t < n ? srows[t] : -1;
    if (t < n) m |= vmask[t];
  }
  for (int o = 32; o > 0; o >>= 1) m |= __shfl_xor(m, o, 64);
  __syncthreads();
  if (lane == 0) atomicOr(&s_mask, m);
  __syncthreads();
  const uint32_t tmask = s_mask;
  const int ntaps = __popc(tmask);
  if (tid < 27) {
    // position of tap tid in the compact list, if active
    if ((tmask >> tid) & 1u) s_taps[__popc(tmask & ((1u << tid) - 1u))] = tid;
  }
  __syncthreads();
  for (int q = tid; q < TM * ntaps; q += kThreads) {
    const int r = q / ntaps, ti = q - r * ntaps;  // consecutive lanes read one row's taps
    const int32_t row = s_row[r];
    s_src[ti * TM + r] = row >= 0 ? nbr[int64_t(row) * 27 + s_taps[ti]] : -1;
  }
  __syncthreads();

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = (c_in + KC - 1) / KC;
  const int nstages = ntaps * nchunks;
  uint4 ra[ACH], rb[BCH];
  // Global -> registers for stage st (tap s_taps[st / nchunks], chunk st % nchunks).
  auto load_stage = [&](int st) {
    const int ti = st / nchunks;
    const int c0 = (st - ti * nchunks) * KC;
    const uint16_t* wk = wp + int64_t(s_taps[ti]) * c_out * c_in;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int q = tid + i * kThreads;
      const int r = q / CPR, cc = q % CPR;
      const int c = c0 + cc * 8;
      ra[i] = make_uint4(0u, 0u, 0u, 0u);
      if (q < TM * CPR) {
        const int32_t src = s_src[ti * TM + r];
        if (src >= 0 && c < c_in) ra[i] = *reinterpret_cast<const uint4*>(x + int64_t(src) * c_in + c);
      }
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int q = tid + i * kThreads;
      const int col = q / CPR, cc = q % CPR;
      const int co = n0 + col, c = c0 + cc * 8;
      rb[i] = make_uint4(0u, 0u, 0u, 0u);
      if (q < TN * CPR && co < c_out && c < c_in)
        rb[i] = *reinterpret_cast<const uint4*>(wk + int64_t(co) * c_in + c);
    }
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int q = tid + i * kThreads;
      if (q < TM * CPR) *reinterpret_cast<uint4*>(sA + (q / CPR) * LDK + (q % CPR) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int q = tid + i * kThreads;
      if (q < TN * CPR) *reinterpret_cast<uint4*>(sB + (q / CPR) * LDK + (q % CPR) * 8) = rb[i];
    }
  };

  if (nstages > 0) load_stage(0);
  for (int st = 0; st < nstages; ++st) {
    store_stage();
    __syncthreads();
    if (st + 1 < nstages) load_stage(st + 1);  // in flight during the matrix work below
#pragma unroll
    for (int kk = 0; kk < KC; kk += 32) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(sA + (wm * WM + i * 16 + (lane & 15)) * LDK + kk +
                                                 (lane >> 4) * 8);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(sB + (wn * WN + j * 16 + (lane & 15)) * LDK + kk +
                                                  (lane >> 4) * 8);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // Epilogue: round to bf16 (nearest-even), stage the tile in LDS, store
  // 16-byte pieces of each row at its caller index.
  uint16_t* sO = smem;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = wm * WM + i * 16 + (lane >> 4) * 4 + e;
        const int c = wn * WN + j * 16 + (lane & 15);
        sO[r * LDO + c] = f32_to_bf16_rne(acc[i][j][e]);
      }
  __syncthreads();
  constexpr int OPR = TN / 8;
  for (int q = tid; q < TM * OPR; q += kThreads) {
    const int r = q / OPR, cc = q % OPR;
    const int32_t row = s_row[r];
    const int co = n0 + cc * 8;
    if (row >= 0 && co < c_out)
      *reinterpret_cast<uint4*>(y + int64_t(row) * c_out + co) =
          *reinterpret_cast<const uint4*>(sO + r * LDO + cc * 8);
  }
}

template <int TM, int TN, int WM, int WN, int KC>
hipError_t launch_tiles(const ConvArgs& a, const uint16_t* wp, hipStream_t st) {
  const int64_t mt = (a.n + TM - 1) / TM;
  const int nt = (a.c_out + TN - 1) / TN;
  const int64_t grid = mt * nt;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  fwd_mfma<TM, TN, WM, WN, KC><<<unsigned(grid), kThreads, 0, st>>>(
      a.nbr, a.srows, a.mask, a.n, static_cast<const uint16_t*>(a.x), wp, static_cast<uint16_t*>(a.y),
      a.c_in, a.c_out, nt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_weights(const void* w, void* wp, int c_in, int c_out, hipStream_t st) {
  dim3 grid(unsigned((c_out + 63) / 64), unsigned((c_in + 63) / 64), 27);
  pack_weights<<<grid, kThreads, 0, st>>>(static_cast<const uint16_t*>(w), static_cast<uint16_t*>(wp),
                                          c_in, c_out);
  return hipGetLastError();
}

hipError_t launch_forward_mfma_bf16(const ConvArgs& a, const void* wp, hipStream_t st) {
  const uint16_t* p = static_cast<const uint16_t*>(wp);
  if (a.c_out >= 128) return launch_tiles<128, 128, 64, 64, 64>(a, p, st);
  if (a.c_out > 32) return launch_tiles<128, 64, 32, 64, 64>(a, p, st);
  if (a.c_out > 16) return launch_tiles<256, 32, 64, 32, 64>(a, p, st);
  return launch_tiles<256, 16, 64, 16, 64>(a, p, st);
}

}  // namespace trsc
