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
#include "halo_plan.h"
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

// Cell bits (of cell_of) contributed by one in-block coordinate on each axis.
__device__ inline uint32_t cell_x(int x) { return (uint32_t(x & 1) << 2) | (uint32_t(x >> 1) << 5); }
__device__ inline uint32_t cell_y(int y) { return (uint32_t(y & 1) << 1) | (uint32_t(y >> 1) << 4); }
__device__ inline uint32_t cell_z(int z) { return uint32_t(z & 1) | (uint32_t(z >> 1) << 3); }

// Each wave works alone until its rows are written (no workgroup barrier): its
// LDS region first holds, for each lane, the {bitmap, start} record of each of
// the 8 blocks around the voxel (record j of lane l at j * 64 + l), which turns
// the per-tap choice of block into one indexed LDS read; the same bytes then
// stage the wave's 64 x 27 output rows and their caller rows for the
// write-back. A workgroup's 256 voxels are one tile of the halo gather-GEMM:
// once every wave is done, the workgroup builds the tile's plan from the
// neighbour rows it holds in registers (halo_plan.h), in the same LDS.
//
// DENSE: the hash was built in a known grid, and the block records come from
// its occupancy bitmap instead of the table: the word of a neighbour block is
// its Morton block index (nearby words for nearby blocks, no probe), its bits
// the block's bitmap, its prefix the block's first sorted position. A block
// outside the grid is absent.
template <bool DENSE>
__global__ __launch_bounds__(kThreads) void kmap_kernel(const uint64_t* __restrict__ skeys, int64_t n,
                                                        TableRef t, DenseRef d, int32_t* __restrict__ nbr,
                                                        uint32_t* __restrict__ mask_out,
                                                        unsigned char* __restrict__ plan,
                                                        uint16_t* __restrict__ costs, int32_t* __restrict__ grows,
                                                        uint32_t* __restrict__ gmask) {
  constexpr int kWaves = kThreads / 64;
  static_assert(kThreads == kPlanThreads, "a workgroup's voxels are one halo tile");
  static_assert(64 * 27 * 4 + 64 * 4 <= 8 * 64 * 16, "staged rows fit in the record region");
  // LDS: the waves' record regions and the bitmap chunk prefixes, then the plan
  constexpr int kMapLds = kWaves * 8 * 64 * 16 + kThreads * 4;
  __shared__ __attribute__((aligned(16))) unsigned char s_u[kMapLds > kPlanLdsBytes ? kMapLds : kPlanLdsBytes];
  uint4 (*const lds)[8 * 64] = reinterpret_cast<uint4 (*)[8 * 64]>(s_u);
  uint32_t* const s_cpre = reinterpret_cast<uint32_t*>(s_u + kWaves * 8 * 64 * 16);  // DENSE: first sorted position of each bitmap chunk
  if constexpr (DENSE) {
    if (int(threadIdx.x) < d.nchunks) s_cpre[threadIdx.x] = d.cpre[threadIdx.x];
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint4* rec = lds[wave];
  int32_t* res = reinterpret_cast<int32_t*>(lds[wave]);  // [64][27]: odd stride, conflict-free
  int32_t* rows = res + 64 * 27;
  const int64_t tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t base = tile * kThreads + wave * 64;
  const int64_t s = base + lane;
  const uint32_t tmask = t.hdr->cap_mask, tshift = t.hdr->shift;
  int32_t got[27];
  uint32_t msk = 0;
  int32_t me = -1;
#pragma unroll
  for (int k = 0; k < 27; ++k) got[k] = -1;
  if (base < n) {
  if (s < n) {
    const uint64_t key = skeys[s];
    me = t.srows[s];
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
    bool okx = false;
    const uint64_t kx = dx ? block_move(bkey, kBMaskX, 4, dx, okx) : bkey;
    // Blocks (ix, iy, iz) in {0,1}^3: index 1 on an axis is the next block on
    // that side (block 0 is the voxel's own). The home slots of all eight are
    // loaded in straight-line code, so that the loads are in flight together
    // (a block the voxel does not need reads its own block's slot, and the
    // result is dropped); the rare probe run that goes past its home slot is
    // finished afterwards.
    uint64_t bk[8];
    bool need[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ix = (j >> 2) & 1, iy = (j >> 1) & 1, iz = j & 1;
      bool nd = (!ix || (dx && okx)) && (!iy || dy) && (!iz || dz);
      uint64_t b = ix ? kx : bkey;
      if (nd && iy) {
        bool ok;
        b = block_move(b, kBMaskY, 2, dy, ok);
        nd = ok;
      }
      if (nd && iz) {
        bool ok;
        b = block_move(b, kBMaskZ, 1, dz, ok);
        nd = ok;
      }
      bk[j] = b;
      need[j] = nd;
    }
    uint64_t bbits[8];
    uint32_t bstart[8];
    if constexpr (DENSE) {
      const int wb = 3 * d.g - 6;  // Morton bits of a block index in the grid
      const uint64_t wlow = (uint64_t(1) << wb) - 1u;
      auto word_of = [&](uint64_t k) { return int64_t(((k >> 42) << wb) | (k & wlow)); };
      const int64_t w_own = word_of(bkey);
      unsigned long long bw[8];
      uint32_t pw[8];
      bool in[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {  // all loads in flight together; a block not needed reads the own word
        in[j] = need[j] && ((bk[j] & kBlockMorton) >> wb) == 0u;
        const int64_t w = in[j] ? word_of(bk[j]) : w_own;
        bw[j] = d.bitmap[w];
        pw[j] = d.wpre[w] + s_cpre[w >> d.lgc];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bbits[j] = in[j] ? bw[j] : 0ull;
        bstart[j] = in[j] ? pw[j] : 0u;
      }
    } else {
      const uint32_t hs0 = home_slot(bkey, tshift) & tmask;
      uint4 v0[8];
      uint32_t st0[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t h = need[j] ? home_slot(bk[j], tshift) & tmask : hs0;
        v0[j] = *reinterpret_cast<const uint4*>(t.slots + h);
        st0[j] = t.slots[h].start;
      }
      uint32_t longer = 0;  // blocks whose home slot holds another key
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint64_t k = uint64_t(v0[j].x) | (uint64_t(v0[j].y) << 32);
        const bool hit = need[j] && k == bk[j];
        bbits[j] = hit ? (uint64_t(v0[j].z) | (uint64_t(v0[j].w) << 32)) : 0ull;
        bstart[j] = hit ? st0[j] : 0u;
        longer |= uint32_t(need[j] && !hit && k != kEmptyKey) << j;
      }
      if (longer) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if ((longer >> j) & 1u) block_find(t.slots, tmask, tshift, bk[j], bbits[j], bstart[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      rec[j * 64 + lane] = uint4{uint32_t(bbits[j]), uint32_t(bbits[j] >> 32), bstart[j], 0u};

    // The 27 neighbours: the record of the tap's block (an offset per axis:
    // the neighbour block on the side the tap leaves by), a bit test in its
    // bitmap, then the sorted position start + popcount.
    const int rxm = dx < 0 ? 4 * 64 : 0, rxp = dx > 0 ? 4 * 64 : 0;
    const int rym = dy < 0 ? 2 * 64 : 0, ryp = dy > 0 ? 2 * 64 : 0;
    const int rzm = dz < 0 ? 64 : 0, rzp = dz > 0 ? 64 : 0;
    const uint32_t cx[3] = {cell_x((lx + 3) & 3), cell_x(lx), cell_x((lx + 1) & 3)};
    const uint32_t cy[3] = {cell_y((ly + 3) & 3), cell_y(ly), cell_y((ly + 1) & 3)};
    const uint32_t cz[3] = {cell_z((lz + 3) & 3), cell_z(lz), cell_z((lz + 1) & 3)};
    msk = 0;
    int32_t spos[27];
#pragma unroll
    for (int k = 0; k < 27; ++k) {
      if (k == 13) continue;
      const int ox = k / 9 - 1, oy = (k / 3) % 3 - 1, oz = k % 3 - 1;
      const int r = (ox < 0 ? rxm : ox > 0 ? rxp : 0) + (oy < 0 ? rym : oy > 0 ? ryp : 0) +
                    (oz < 0 ? rzm : oz > 0 ? rzp : 0);
      const uint4 e = rec[r + lane];
      const uint64_t bits = uint64_t(e.x) | (uint64_t(e.y) << 32);
      const uint32_t c = cx[ox + 1] | cy[oy + 1] | cz[oz + 1];
      const uint32_t hit = uint32_t(bits >> c) & 1u;
      // start + popcount, or -1 for a miss, without a branch
      spos[k] = int32_t(e.z + __popcll(bits & ((1ull << c) - 1ull))) | (int32_t(hit) - 1);
      msk |= hit << k;
    }
    msk |= 1u << 13;
    // Caller rows of the 26 neighbours, loaded together and unconditionally (a
    // missing neighbour reads the voxel's own entry, and its result is
    // dropped); positions are below 2^30, so a 32-bit byte offset from the
    // row array reaches them.
    const char* srow_bytes = reinterpret_cast<const char*>(t.srows);
#pragma unroll
    for (int k = 0; k < 27; ++k) {
      if (k == 13) continue;
      const uint32_t q = spos[k] >= 0 ? uint32_t(spos[k]) : uint32_t(s);
      got[k] = *reinterpret_cast<const int32_t*>(srow_bytes + q * 4u);
    }
#pragma unroll
    for (int k = 0; k < 27; ++k) got[k] = k == 13 ? me : (spos[k] >= 0 ? got[k] : -1);
    mask_out[s] = msk;
    // Every lane of the wave has read its records (LDS executes a wave's
    // instructions in order); the staging below reuses the bytes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int k = 0; k < 27; ++k) res[lane * 27 + k] = got[k];
    rows[lane] = me;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const int64_t left = n - base;
  const int nv = left < 64 ? int(left) : 64;
  for (int e = lane; e < nv * 27; e += 64) {
    const int v = e / 27;
    nbr[int64_t(rows[v]) * 27 + (e - v * 27)] = res[e];
  }
  }
  // the tile's plan, once every wave has read its staged rows
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __syncthreads();
  halo_plan_tile(tile, s < n, msk, me, got, plan, costs, grows, gmask, s_u);
}

}  // namespace

hipError_t launch_kmap(const uint64_t* skeys, int64_t n, const TableRef& t, const DenseRef* dense, int32_t* nbr,
                       uint32_t* mask, int32_t* grows, uint32_t* gmask, unsigned char* plan, uint16_t* costs,
                       int32_t* order, hipStream_t st) {
  if (n > 0) {
    const unsigned grid = unsigned((n + kThreads - 1) / kThreads);
    static_assert(kThreads == kHaloTM, "one workgroup per halo tile");
    if (dense != nullptr)
      kmap_kernel<true><<<grid, kThreads, 0, st>>>(skeys, n, t, *dense, nbr, mask, plan, costs, grows, gmask);
    else
      kmap_kernel<false><<<grid, kThreads, 0, st>>>(skeys, n, t, DenseRef{}, nbr, mask, plan, costs, grows, gmask);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_halo_order(costs, halo_tiles(n), order, st);
  }
  return hipGetLastError();
}

}  // namespace trsc
