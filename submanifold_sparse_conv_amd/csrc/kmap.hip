// Kernel map: for every active voxel and each of the 27 taps of the 3x3x3
// kernel, the row of the neighbour at that offset or -1. This is the neighbour
// table that is built once per resolution level and then reused by every
// convolution at that level ("Porting TRELLIS.2 From Python to Rust and
// Metal", section V; neighbour maps cached per tensor in "Running TRELLIS.2 on
// a Mac (1/3)", sparse 3D convolution paragraph).
//
// One wave64 per 64 voxels taken in Morton order, so a wave's probes ask for
// keys of one compact block of space and share cache lines of the table.
// Neighbour keys are formed directly on the dilated (interleaved) axis bits,
// without decoding the key. The lookups are latency-bound (dependent loads), so
// each lane keeps nine probes in flight at a time. Each lane also builds its voxel's 27-bit
// neighbour mask (Morton order), which the gather-GEMM uses to skip taps no row
// of a tile needs. The rows of nbr are written back in caller order through
// LDS so that consecutive lanes store consecutive words.
#include "common.h"
#include "launch.h"

namespace trsc {
namespace {

constexpr int kThreads = 256;

// Dilated coordinate of one axis moved by -1, 0, +1; `ok` false when the move
// leaves [0, 65535].
struct AxisMoves {
  uint64_t v[3];
  bool ok[3];
};

__device__ inline AxisMoves axis_moves(uint64_t key, uint64_t axis_mask, uint64_t low_bit) {
  AxisMoves m;
  const uint64_t d = key & axis_mask;
  m.v[1] = d;
  m.ok[1] = true;
  m.ok[0] = d != 0;
  m.v[0] = (d - low_bit) & axis_mask;
  m.ok[2] = d != axis_mask;
  m.v[2] = ((d | ~axis_mask) + low_bit) & axis_mask;
  return m;
}

__global__ __launch_bounds__(kThreads) void kmap_kernel(const uint64_t* __restrict__ skeys,
                                                        const int32_t* __restrict__ srows, int64_t n,
                                                        TableRef t, const HashHeader* __restrict__ hdr,
                                                        int32_t* __restrict__ nbr,
                                                        uint32_t* __restrict__ mask_out) {
  __shared__ int32_t res[kThreads * 27];  // odd stride: conflict-free both ways
  __shared__ int32_t rows[kThreads];
  const int64_t base = int64_t(xcd_remap(blockIdx.x, gridDim.x)) * kThreads;
  const int64_t s = base + threadIdx.x;
  const int32_t special = hdr->special_row;
  if (s < n) {
    const uint64_t key = skeys[s];
    const int32_t me = srows[s];
    const uint64_t bpart = key & ~kMortonMask;
    const AxisMoves mx = axis_moves(key, kMaskX, 4);
    const AxisMoves my = axis_moves(key, kMaskY, 2);
    const AxisMoves mz = axis_moves(key, kMaskZ, 1);
    uint32_t msk = 0;
    // Taps in three batches of nine (one x offset each). A batch first issues
    // the home-slot loads of all its probes, so they are in flight together,
    // and only then resolves them (continuing a probe run where needed).
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      uint64_t q[9];
      uint32_t hs[9];
      uint4 v[9];
      bool ok[9];
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        const int b = j / 3, c = j % 3;
        ok[j] = (a * 9 + j != 13) && mx.ok[a] && my.ok[b] && mz.ok[c];
        q[j] = bpart | mx.v[a] | my.v[b] | mz.v[c];
        hs[j] = home_slot(q[j], t.shift);
        v[j] = ok[j] ? load_slot(t.slots, hs[j]) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        const int k = a * 9 + j;
        int32_t r;
        if (k == 13)
          r = me;
        else if (!ok[j])
          r = -1;
        else if (q[j] == kEmptyKey)
          r = special;
        else
          r = probe_from(t, q[j], hs[j], v[j]);
        res[threadIdx.x * 27 + k] = r;
        msk |= uint32_t(r >= 0) << k;
      }
    }
    rows[threadIdx.x] = me;
    mask_out[s] = msk;
  }
  __syncthreads();
  const int64_t left = n - base;
  const int nvox = left < kThreads ? int(left) : kThreads;
  for (int e = threadIdx.x; e < nvox * 27; e += kThreads) {
    const int v = e / 27;
    const int k = e - v * 27;
    nbr[int64_t(rows[v]) * 27 + k] = res[e];
  }
}

}  // namespace

hipError_t launch_kmap(const uint64_t* skeys, const int32_t* srows, int64_t n, const TableRef& t,
                       const HashHeader* hdr, int32_t* nbr, uint32_t* mask, hipStream_t st) {
  if (n > 0)
    kmap_kernel<<<unsigned((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(skeys, srows, n, t, hdr,
                                                                             nbr, mask);
  return hipGetLastError();
}

}  // namespace trsc
