// Halo plan of one tile of the gather-GEMM, built inside the kernel-map
// kernel right after the tile's neighbour rows are found (once per resolution
// level, like the neighbour table itself -- "Porting TRELLIS.2 From Python to
// Rust and Metal", section V) and read by every convolution at that level.
//
// A tile is kHaloTM Morton-consecutive voxels. Over a thin surface their
// neighbours are few distinct rows (~1.75 per voxel against ~17.7 (voxel, tap)
// pairs), so the gather-GEMM copies those rows into LDS once and reads every
// tap's operand from there. Per tile the plan holds:
//   - the tile order: the voxels stably regrouped by the octant pattern of
//     their neighbour mask (which corner neighbours exist), so that 32-row
//     blocks hold voxels on the same side of the surface and more blocks can
//     skip a tap none of their rows has;
//   - the halo: the distinct caller rows among the tile's neighbours, found
//     with an LDS hash table (compare-and-swap, linear probing) and numbered
//     by a workgroup scan over the table (slot 0 = absent neighbour);
//   - the slot of every (row, tap) (as its LDS offset in the gather-GEMM's
//     halo), and per tap which 32-row blocks have it.
// The numbering follows the table's layout, which depends on the order of the
// atomics; the products do not (each output row sums its own taps in tap order
// whatever its halo slots), so convolutions are identical run to run.
// A tile with more distinct neighbours than kHaloCap - 1, or whose table
// insertion runs past kHaloProbes probes, is marked nh = -1: the gather-GEMM
// then reads its rows from global memory.
#pragma once
#include "common.h"
#include "launch.h"

namespace trsc {

constexpr int kPlanThreads = kHaloTM;  // thread t takes the tile's t-th Morton item
static_assert(kPlanThreads == 256, "one wave per 64 items, four waves");

// LDS of the plan (bytes, one region of kPlanLdsBytes): the dedup table, the
// slot table, per-(wave, octant pattern) counts, the items' masks in tile
// order, the per-tap block flags and a few words.
constexpr int kPlanTabAt = 0, kPlanTabBytes = kHaloHash * 4;
constexpr int kPlanSlotAt = kPlanTabAt + kPlanTabBytes, kPlanSlotLdsBytes = 27 * kHaloTM * 2;
constexpr int kPlanCntAt = kPlanSlotAt + kPlanSlotLdsBytes;          // uint32 [4][256]
constexpr int kPlanPmaskAt = kPlanCntAt + 4 * 256 * 4;                 // uint32 [kHaloTM]
constexpr int kPlanFmAt = kPlanPmaskAt + kHaloTM * 4;                  // uint8 [27][4]
constexpr int kPlanWordsAt = kPlanFmAt + 112;                          // uint32 wsum[4], tmask, over
constexpr int kPlanLdsBytes = kPlanWordsAt + 8 * 4;

// Position of (tap k, row r) in the slot table, within tap k's kHaloTM entries:
// row half r / 128, then row r % 32 of the half's four 32-row blocks, then the
// block, so that one 64-bit read gives a lane its four rows' offsets.
__device__ inline int slot_index(int r) { return (r >> 7) * 128 + (r & 31) * 4 + ((r >> 5) & 3); }

// The plan of tile `tile` (items tile * kHaloTM + tid): thread tid brings its item's
// validity, 27-bit neighbour mask m, caller row cr and the caller rows of its
// 27 neighbours jv (-1: absent). Every thread of the 256-thread workgroup
// calls it; `lds` is kPlanLdsBytes of LDS no other code uses meanwhile. The
// tile order is also the row order of the row-gather kernels and the weight
// gradient: grows / gmask at the tile's positions.
__device__ __forceinline__ void halo_plan_tile(int64_t tile, bool valid, uint32_t m, int32_t cr,
                                               const int32_t (&jv)[27], unsigned char* __restrict__ plan,
                                               uint16_t* __restrict__ costs, int32_t* __restrict__ grows,
                                               uint32_t* __restrict__ gmask, unsigned char* lds) {
  int32_t* const tab = reinterpret_cast<int32_t*>(lds + kPlanTabAt);
  int16_t* const s_slot = reinterpret_cast<int16_t*>(lds + kPlanSlotAt);
  uint32_t (*const cnt)[256] = reinterpret_cast<uint32_t (*)[256]>(lds + kPlanCntAt);
  uint32_t* const s_pmask = reinterpret_cast<uint32_t*>(lds + kPlanPmaskAt);
  uint8_t (*const s_fm)[4] = reinterpret_cast<uint8_t (*)[4]>(lds + kPlanFmAt);
  uint32_t* const s_wsum = reinterpret_cast<uint32_t*>(lds + kPlanWordsAt);
  uint32_t& s_tmask = s_wsum[4];
  uint32_t& s_over = s_wsum[5];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned char* const rec = plan + tile * int64_t(kPlanBytes);

  for (int q = tid; q < 4 * 256; q += kPlanThreads) (&cnt[0][0])[q] = 0u;
  if (tid == 0) s_tmask = 0u, s_over = 0u;
  __syncthreads();

  // (1) Tile position r: stable counting sort of the valid items by octant
  // pattern (rank among equal patterns of the wave by ballots, then a scan over
  // (pattern, wave)); items past the end keep r = tid (they follow all valid ones).
  const uint32_t d = octant_key(m);
  uint32_t rank = 0;
  {
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1u;
      const unsigned long long bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const unsigned long long lt = (1ull << lane) - 1ull;
    rank = __popcll(peers & lt);
    if (valid && (peers & lt) == 0) cnt[wave][d] = __popcll(peers);
  }
  __syncthreads();
  {
    // thread p owns pattern p: exclusive scan of the pattern totals, then its
    // first position in each wave
    uint32_t tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) tot += cnt[w][tid];
    uint32_t x = tot;
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) s_wsum[wave] = x;
    __syncthreads();
    uint32_t run = x - tot;
    for (int w = 0; w < wave; ++w) run += s_wsum[w];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t v = cnt[w][tid];
      cnt[w][tid] = run;
      run += v;
    }
  }
  __syncthreads();
  const int r = valid ? int(cnt[wave][d] + rank) : tid;
  const int sx = slot_index(r);
  reinterpret_cast<int32_t*>(rec + kPlanCrow)[r] = cr;
  reinterpret_cast<uint32_t*>(rec + kPlanMask)[r] = m;
  if (valid) {  // valid items take the tile's first positions: t0 + r < n
    grows[tile * kHaloTM + r] = cr;
    gmask[tile * kHaloTM + r] = m;
  }
  s_pmask[r] = m;

  // (2) The item's neighbours inserted into the table: every first probe
  // issued together, then the collisions retried (a run longer than
  // kHaloProbes marks the tile as not fitting).
  {
    int hv[27];
    for (int e = tid; e < kHaloHash; e += kPlanThreads) tab[e] = -1;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 27; ++k) hv[k] = jv[k] >= 0 ? int((uint32_t(jv[k]) * 2654435761u) >> (32 - kHaloHashBits)) : -1;
    uint32_t left = 0;  // taps still to place
#pragma unroll
    for (int k = 0; k < 27; ++k) {
      if (hv[k] >= 0) {
        const int32_t old = atomicCAS(&tab[hv[k]], -1, jv[k]);
        if (old != -1 && old != jv[k]) left |= 1u << k;
      }
    }
    bool over = false;
    for (int probe = 1; left != 0u; ++probe) {
      if (probe == kHaloProbes) {
        over = true;
        break;
      }
#pragma unroll
      for (int k = 0; k < 27; ++k) {
        if ((left >> k) & 1u) {
          hv[k] = (hv[k] + 1) & (kHaloHash - 1);
          const int32_t old = atomicCAS(&tab[hv[k]], -1, jv[k]);
          if (old == -1 || old == jv[k]) left &= ~(1u << k);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 27; ++k) s_slot[k * kHaloTM + sx] = int16_t(over ? -1 : hv[k]);
    if (over) s_over = 1u;
  }
  __syncthreads();

  // (3) Block masks in tile order (position tid; a block = 32 positions, two
  // per wave) and the tile's taps.
  {
    const uint32_t pm = s_pmask[tid];
    uint32_t wm = pm;
    for (int o = 32; o > 0; o >>= 1) wm |= __shfl_xor(wm, o, 64);
#pragma unroll 1
    for (int k = 0; k < 27; ++k) {
      const unsigned long long b = __ballot((pm >> k) & 1u);
      if (lane == 0) s_fm[k][wave] = uint8_t(uint32_t((b & 0xFFFFFFFFull) != 0) | (uint32_t((b >> 32) != 0) << 1));
    }
    if (lane == 0) atomicOr(&s_tmask, wm);
  }

  // (4) Number the occupied table entries: thread t owns entries PER t .. PER t + PER - 1.
  int nh;
  {
    constexpr int PER = kHaloHash / kPlanThreads;
    int32_t key[PER];
    int c = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      key[e] = tab[tid * PER + e];
      c += key[e] != -1;
    }
    int incl = c;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    __syncthreads();  // s_wsum is free again
    if (lane == 63) s_wsum[wave] = uint32_t(incl);
    __syncthreads();
    int base = incl - c;
    nh = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int s = int(s_wsum[w]);
      if (w < wave) base += s;
      nh += s;
    }
    int slot = 1 + base;
    int32_t* const rows = reinterpret_cast<int32_t*>(rec + kPlanRows);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (key[e] != -1) {
        if (slot < kHaloCap) rows[slot] = key[e];
        tab[tid * PER + e] = slot;
        ++slot;
      }
    }
  }
  __syncthreads();
  const bool fits = s_over == 0u && nh + 1 <= kHaloCap;

  // (5) Slots of this item's taps, stored as the LDS byte offset of the slot's
  // row in the gather-GEMM's halo (64-byte rows whose 16-byte pieces are
  // rotated by (slot >> 2) & 3: piece q of a row is at offset ^ (q << 4)), then
  // the table written out whole.
  if (fits) {
#pragma unroll 1
    for (int k = 0; k < 27; ++k) {
      const int h = s_slot[k * kHaloTM + sx];
      const int slot = h >= 0 ? tab[h] : 0;
      s_slot[k * kHaloTM + sx] = int16_t(uint16_t(slot * kHaloRowBytes + (((slot >> 2) & 3) << 4)));
    }
  }
  __syncthreads();
  if (fits) {
    const uint4* src = reinterpret_cast<const uint4*>(s_slot);
    uint4* dst = reinterpret_cast<uint4*>(rec + kPlanSlots);
    for (int q = tid; q < kPlanSlotBytes / 16; q += kPlanThreads) dst[q] = src[q];
  }
  HaloHeader* hdr = reinterpret_cast<HaloHeader*>(rec + kPlanHdr);
  if (tid == 0) {
    hdr->nh = fits ? nh : -1;
    hdr->tmask = s_tmask;
  }
  if (tid < 27)
    hdr->fm[tid] = uint16_t(s_fm[tid][0] | (s_fm[tid][1] << 2) | (s_fm[tid][2] << 4) | (s_fm[tid][3] << 6));
  if (tid < 64) {
    // the work estimate: (block, tap) pairs that multiply (a tile gathering
    // from global memory counts three times)
    int pairs = 0;
    if (lane < 27) pairs = __popc(uint32_t(s_fm[lane][0] | (s_fm[lane][1] << 2) | (s_fm[lane][2] << 4) | (s_fm[lane][3] << 6)));
    for (int o = 32; o > 0; o >>= 1) pairs += __shfl_xor(pairs, o, 64);
    if (lane == 0) costs[tile] = uint16_t(fits ? pairs : 3 * pairs);
  }
}

}  // namespace trsc
