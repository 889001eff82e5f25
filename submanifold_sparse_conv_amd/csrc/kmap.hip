// Kernel map: for every active voxel and each of the 27 taps of the 3x3x3
// kernel, the row of the neighbour at that offset or -1. This is the neighbour
// table that is built once per resolution level and then reused by every
// convolution at that level ("Porting TRELLIS.2 From Python to Rust and
// Metal", section V; neighbour maps cached per tensor in "Running TRELLIS.2 on
// a Mac (1/3)", sparse 3D convolution paragraph).
//
// One wave64 per 64 voxels taken in Morton order. The 26 neighbours of a
// voxel lie in at most 8 of the 4x4x4 blocks of the table (3.4 on average):
// each lane probes those blocks (all loads in flight together), then finds a
// neighbour by a bit test in its block's occupancy bitmap; its sorted position
// is the block start plus a popcount, and its caller row one more load. Block
// keys of neighbouring blocks are formed on the dilated (interleaved) axis
// bits, without decoding. Each lane also builds its voxel's 27-bit neighbour
// mask, which the gather-GEMM uses to skip taps no row of a tile needs. The
// rows of nbr are written back in caller order through LDS so that
// consecutive lanes store consecutive words.
#include "common.h"
#include "launch.h"

namespace trsc {
namespace {

constexpr int kThreads = 256;

// Block-key moves. A block key is key >> 6: the Morton interleave of the block
// coordinates (x >> 2, y >> 2, z >> 2) with the batch index above bit 42.
constexpr uint64_t kBlockMorton = (uint64_t(1) << 42) - 1;
constexpr uint64_t kBMaskZ = kMaskZ & kBlockMorton;
constexpr uint64_t kBMaskY = kMaskY & kBlockMorton;
constexpr uint64_t kBMaskX = kMaskX & kBlockMorton;

// The block key next to `bkey` along one axis (dir -1 or +1), on the dilated
// bits; `ok` false when the move leaves the coordinate range.
__device__ inline uint64_t block_move(uint64_t bkey, uint64_t amask, uint64_t low, int dir, bool& ok) {
  const uint64_t d = bkey & amask;
  const uint64_t rest = bkey & ~amask;
  if (dir < 0) {
    ok = d != 0;
    return rest | ((d - low) & amask);
  }
  ok = d != amask;
  return rest | (((d | ~amask) + low) & amask);
}

__global__ __launch_bounds__(kThreads) void kmap_kernel(const uint64_t* __restrict__ skeys, int64_t n,
                                                        TableRef t, int32_t* __restrict__ nbr,
                                                        uint32_t* __restrict__ mask_out) {
  __shared__ int32_t res[kThreads * 27];  // odd stride: conflict-free both ways
  __shared__ int32_t rows[kThreads];
  const int64_t base = int64_t(xcd_remap(blockIdx.x, gridDim.x)) * kThreads;
  const int64_t s = base + threadIdx.x;
  const uint32_t tmask = t.hdr->cap_mask, tshift = t.hdr->shift;
  if (s < n) {
    const uint64_t key = skeys[s];
    const int32_t me = t.srows[s];
    const uint64_t bkey = key >> 6;
    // In-block coordinates (0..3) and, per axis, the side on which the 3x3x3
    // neighbourhood leaves the block (0: stays inside).
    const uint32_t cl = uint32_t(key & 63u);
    const int lx = int(((cl >> 2) & 1u) | (((cl >> 5) & 1u) << 1));
    const int ly = int(((cl >> 1) & 1u) | (((cl >> 4) & 1u) << 1));
    const int lz = int((cl & 1u) | (((cl >> 3) & 1u) << 1));
    const int dx = lx == 0 ? -1 : (lx == 3 ? 1 : 0);
    const int dy = ly == 0 ? -1 : (ly == 3 ? 1 : 0);
    const int dz = lz == 0 ? -1 : (lz == 3 ? 1 : 0);
    bool okx = false, oky = false, okz = false;
    const uint64_t kx = dx ? block_move(bkey, kBMaskX, 4, dx, okx) : bkey;
    // Blocks (ix, iy, iz) in {0,1}^3: index 1 on an axis is the next block on
    // that side. Probe the needed ones together (their loads overlap).
    uint64_t bbits[8];
    uint32_t bstart[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ix = (j >> 2) & 1, iy = (j >> 1) & 1, iz = j & 1;
      bool need = (!ix || (dx && okx)) && (!iy || dy) && (!iz || dz);
      uint64_t bk = ix ? kx : bkey;
      if (need && iy) {
        bool ok;
        bk = block_move(bk, kBMaskY, 2, dy, ok);
        need = ok;
      }
      if (need && iz) {
        bool ok;
        bk = block_move(bk, kBMaskZ, 1, dz, ok);
        need = ok;
      }
      bbits[j] = 0;
      bstart[j] = 0;
      if (need) {
        const uint32_t hs = home_slot(bk, tshift) & tmask;
        const uint4 v0 = reinterpret_cast<const uint4*>(t.slots + hs)[0];
        const uint4 v1 = reinterpret_cast<const uint4*>(t.slots + hs)[1];
        block_probe_from(t.slots, tmask, bk, hs, v0, v1, bbits[j], bstart[j]);
      }
    }
    // The 27 neighbours: bit test in the block's bitmap, then the sorted
    // position start + popcount and its caller row.
    uint32_t msk = 0;
    int32_t spos[27];
#pragma unroll
    for (int k = 0; k < 27; ++k) {
      const int ox = k / 9 - 1, oy = (k / 3) % 3 - 1, oz = k % 3 - 1;
      const int nx = lx + ox, ny = ly + oy, nz = lz + oz;
      const int j = ((nx < 0 || nx > 3) ? 4 : 0) | ((ny < 0 || ny > 3) ? 2 : 0) | ((nz < 0 || nz > 3) ? 1 : 0);
      const uint32_t c = cell_of(uint32_t(nx) & 3u, uint32_t(ny) & 3u, uint32_t(nz) & 3u);
      const uint64_t bits = bbits[j];
      spos[k] = ((bits >> c) & 1u) ? int32_t(bstart[j] + __popcll(bits & ((1ull << c) - 1ull))) : -1;
      msk |= uint32_t(spos[k] >= 0) << k;
    }
#pragma unroll
    for (int k = 0; k < 27; ++k) {
      const int32_t r = k == 13 ? me : (spos[k] >= 0 ? t.srows[spos[k]] : -1);
      res[threadIdx.x * 27 + k] = r;
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

// Octant pattern of a neighbour mask: bit (dx>0)*4 + (dy>0)*2 + (dz>0) is set
// when the corner neighbour at (dx, dy, dz), |dx| = |dy| = |dz| = 1, exists.
// It says on which sides of a thin surface the voxel lies.
__device__ inline uint32_t octant_key(uint32_t m) {
  return ((m >> 0) & 1u) | (((m >> 2) & 1u) << 1) | (((m >> 6) & 1u) << 2) | (((m >> 8) & 1u) << 3) |
         (((m >> 18) & 1u) << 4) | (((m >> 20) & 1u) << 5) | (((m >> 24) & 1u) << 6) |
         (((m >> 26) & 1u) << 7);
}

constexpr int kGroupThreads = 1024;

// Row order of the gather-GEMM: inside each window of kGroupWindow Morton-
// consecutive voxels, a stable counting sort by octant pattern. Tiles of
// consecutive rows then hold voxels on the same side of the surface, whose
// neighbour masks overlap more, so fewer taps are multiplied by zero rows.
// (Which tile a voxel lands in does not change its output row.)
__global__ __launch_bounds__(kGroupThreads) void group_rows(const int32_t* __restrict__ srows,
                                                            const uint32_t* __restrict__ mask, int64_t n,
                                                            int32_t* __restrict__ grows,
                                                            uint32_t* __restrict__ gmask) {
  constexpr int WAVES = kGroupThreads / 64;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t base_off[256];
  __shared__ uint32_t wcount[WAVES][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t w0 = int64_t(blockIdx.x) * kGroupWindow;
  const int64_t w1 = w0 + kGroupWindow < n ? w0 + kGroupWindow : n;
  if (tid < 256) hist[tid] = 0;
  __syncthreads();
  for (int64_t t = w0 + tid; t < w1; t += kGroupThreads) atomicAdd(&hist[octant_key(mask[t])], 1u);
  __syncthreads();
  if (tid < 256) {  // exclusive scan of the histogram: four waves, then their totals
    const uint32_t v = hist[tid];
    uint32_t x = v;
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wcount[0][wave] = x;
    base_off[tid] = x - v;
  }
  __syncthreads();
  if (tid < 256) {
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wcount[0][w];
    base_off[tid] += before;
  }
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int64_t r0 = w0; r0 < w1; r0 += kGroupThreads) {
    if (tid < 256)
      for (int w = 0; w < WAVES; ++w) wcount[w][tid] = 0;
    __syncthreads();
    const int64_t t = r0 + tid;
    const bool valid = t < w1;
    uint32_t m = 0, d = 0;
    int32_t row = 0;
    if (valid) {
      m = mask[t];
      row = srows[t];
      d = octant_key(m);
    }
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool bit = (d >> j) & 1u;
      const unsigned long long bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    if (valid && (peers & lt) == 0) wcount[wave][d] = __popcll(peers);
    __syncthreads();
    if (valid) {
      uint32_t pos = base_off[d] + __popcll(peers & lt);
      for (int w = 0; w < wave; ++w) pos += wcount[w][d];
      grows[w0 + pos] = row;
      gmask[w0 + pos] = m;
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t add = 0;
      for (int w = 0; w < WAVES; ++w) add += wcount[w][tid];
      base_off[tid] += add;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_kmap(const uint64_t* skeys, int64_t n, const TableRef& t, int32_t* nbr, uint32_t* mask,
                       int32_t* grows, uint32_t* gmask, hipStream_t st) {
  if (n > 0) {
    kmap_kernel<<<unsigned((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(skeys, n, t, nbr, mask);
    group_rows<<<unsigned((n + kGroupWindow - 1) / kGroupWindow), kGroupThreads, 0, st>>>(t.srows, mask, n,
                                                                                         grows, gmask);
  }
  return hipGetLastError();
}

}  // namespace trsc
