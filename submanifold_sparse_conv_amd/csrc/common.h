// Internal definitions shared by the HIP kernels of the library (not part of
// the C ABI). gfx950 only: wave64, 64-bit ballots.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tr_sparseconv.h"

namespace trsc {

// ---------------------------------------------------------------------------
// Keys. A voxel (b, x, y, z), every component in [0, 2^16), becomes the 64-bit
// key  b << 48 | morton48(x, y, z), where morton48 interleaves the bits of
// x, y, z with x the most significant of each triple. Sorting keys gives
// Z-order inside each object, objects in ascending b.
// ---------------------------------------------------------------------------
constexpr uint64_t kMortonMask = 0xFFFFFFFFFFFFull;  // low 48 bits
constexpr uint64_t kMaskZ = 0x249249249249ull;       // bits 0, 3, ..., 45
constexpr uint64_t kMaskY = kMaskZ << 1;
constexpr uint64_t kMaskX = kMaskZ << 2;
constexpr uint64_t kEmptyKey = ~0ull;  // empty table slot: no block key has all 64 bits set

__host__ __device__ inline uint64_t dilate3(uint32_t v) {  // bit i -> bit 3i (16 bits)
  uint64_t x = v & 0xFFFFu;
  x = (x | (x << 16)) & 0x0000FF0000FFull;
  x = (x | (x << 8)) & 0x00F00F00F00Full;
  x = (x | (x << 4)) & 0x0C30C30C30C3ull;
  x = (x | (x << 2)) & 0x249249249249ull;
  return x;
}

__host__ __device__ inline uint32_t compact3(uint64_t x) {  // inverse of dilate3
  x &= 0x249249249249ull;
  x = (x ^ (x >> 2)) & 0x0C30C30C30C3ull;
  x = (x ^ (x >> 4)) & 0x00F00F00F00Full;
  x = (x ^ (x >> 8)) & 0x0000FF0000FFull;
  x = (x ^ (x >> 16)) & 0x00000000FFFFull;
  return uint32_t(x);
}

__host__ __device__ inline uint64_t make_key(uint32_t b, uint32_t x, uint32_t y, uint32_t z) {
  return (uint64_t(b) << 48) | (dilate3(x) << 2) | (dilate3(y) << 1) | dilate3(z);
}

// ---------------------------------------------------------------------------
// Open-addressing table of occupied 4x4x4 blocks. The key of a block is
// key >> 6 (the voxel key without its lowest Morton triple pair), so the 64
// cells of a block are the keys with the same high bits and their cell index
// is key & 63. A slot holds the block key, a 64-bit occupancy bitmap (bit c set
// when cell c is active) and `start`, the Morton-sorted position of the
// block's first active voxel. The sorted position of an active voxel is then
// start + popcount(bitmap & ((1 << c) - 1)), and its caller row is
// sorted_rows[that position]. Block keys have at most 58 bits, so ~0 marks an
// empty slot.
//
// Capacity: a power of two >= 2 * (number of blocks), chosen on the device
// after the sort and kept in the header with the hash shift. Home slot:
// Fibonacci hashing of the block key; collisions probe linearly.
//
// A surface of thickness ~2 fills ~20 of a block's 64 cells, so the table is
// ~20x smaller than one slot per voxel and stays in L2; the 26 neighbours of
// a voxel fall into at most 8 blocks (3.4 on average).
// ---------------------------------------------------------------------------
struct alignas(32) BlockSlot {
  uint64_t bkey;
  uint64_t bits;
  uint32_t start;
  uint32_t pad0;
  uint64_t pad1;
};

constexpr uint32_t kFlagCoordRange = 1u;
constexpr uint32_t kFlagDuplicate = 2u;
constexpr uint32_t kFlagCapacity = 4u;

// One radix digit: key bits pos[0..nbits) (least significant first).
constexpr int kMaxDigitBits = 11;
constexpr int kSortPasses = 4;
struct DigitBits {
  uint8_t pos[12];
  int32_t nbits;
};

struct alignas(256) HashHeader {
  uint32_t flags;
  uint32_t nblocks;             // occupied 4x4x4 blocks
  uint32_t cap_mask;            // table capacity - 1
  uint32_t shift;               // 64 - log2(capacity)
  unsigned long long or_bits;   // OR of all voxel keys
  unsigned long long and_bits;  // AND of all voxel keys
  DigitBits digit[kSortPasses]; // the radix passes over the key bits that vary (empty ones first)
  int32_t rest_n;               // varying bits beyond the passes' digits (sorted by radix_rest)
  uint8_t rest_pos[64];
};

struct TableRef {
  const BlockSlot* slots;
  const HashHeader* hdr;  // capacity and shift live on the device
  const int32_t* srows;   // sorted position -> caller row
};

// The occupancy bitmap of a hash built in a known grid (x, y, z < 2^g): word w
// of block key k is ((k >> 42) << (3g - 6)) | (k & (2^(3g - 6) - 1)); its bits
// are the block's occupancy bitmap, and the block's first sorted position is
// cpre[w >> lgc] + wpre[w] (nchunks <= 256 chunks of 2^lgc words).
struct DenseRef {
  const unsigned long long* bitmap;
  const uint32_t* wpre;
  const uint32_t* cpre;
  int lgc, nchunks, g;
};

__host__ __device__ inline uint32_t home_slot(uint64_t bkey, uint32_t shift) {
  return uint32_t((bkey * 0x9E3779B97F4A7C15ull) >> shift);
}

// Occupancy bitmap and start of block `bkey` (bits = 0 when it is absent),
// continuing a probe run whose first slot s is already loaded: its first 16
// bytes (key, bitmap) in v0 and its start in start0.
__device__ inline void block_probe_from(const BlockSlot* slots, uint32_t mask, uint64_t bkey, uint32_t s,
                                        uint4 v0, uint32_t start0, uint64_t& bits, uint32_t& start) {
  bits = 0;
  start = 0;
  for (uint32_t probe = 0; probe <= mask; ++probe) {
    const uint64_t k = uint64_t(v0.x) | (uint64_t(v0.y) << 32);
    if (k == bkey) {
      bits = uint64_t(v0.z) | (uint64_t(v0.w) << 32);
      start = start0;
      return;
    }
    if (k == kEmptyKey) return;
    s = (s + 1) & mask;
    v0 = *reinterpret_cast<const uint4*>(slots + s);
    start0 = slots[s].start;
  }
}

__device__ inline void block_find(const BlockSlot* slots, uint32_t mask, uint32_t shift, uint64_t bkey,
                                  uint64_t& bits, uint32_t& start) {
  const uint32_t s = home_slot(bkey, shift) & mask;
  block_probe_from(slots, mask, bkey, s, *reinterpret_cast<const uint4*>(slots + s), slots[s].start, bits,
                   start);
}

// Cell index (0..63) of the in-block coordinates (x, y, z in 0..3): the low
// six bits of the Morton key.
__host__ __device__ inline uint32_t cell_of(uint32_t x, uint32_t y, uint32_t z) {
  return (z & 1u) | ((y & 1u) << 1) | ((x & 1u) << 2) | ((z >> 1) << 3) | ((y >> 1) << 4) | ((x >> 1) << 5);
}

// Caller row of the voxel with key `key`, or -1.
__device__ inline int32_t voxel_find(const TableRef& t, uint32_t mask, uint32_t shift, uint64_t key) {
  uint64_t bits;
  uint32_t start;
  block_find(t.slots, mask, shift, key >> 6, bits, start);
  const uint32_t c = uint32_t(key & 63u);
  if (!((bits >> c) & 1u)) return -1;
  return t.srows[start + __popcll(bits & ((1ull << c) - 1ull))];
}

// Workgroup index -> work index such that each XCD (workgroups are dealt to
// the 8 XCDs of the chip round-robin) gets one contiguous run of work items, so
// neighbouring work (Morton-adjacent voxels) shares that XCD's L2.
__device__ inline int xcd_remap(int bid, int grid) {
  const int xcd = bid & 7, local = bid >> 3;
  const int per = grid >> 3, rem = grid & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// Octant pattern of a neighbour mask: bit (dx>0)*4 + (dy>0)*2 + (dz>0) is set
// when the corner neighbour at (dx, dy, dz), |dx| = |dy| = |dz| = 1, exists.
// It says on which sides of a thin surface the voxel lies.
__device__ inline uint32_t octant_key(uint32_t m) {
  return ((m >> 0) & 1u) | (((m >> 2) & 1u) << 1) | (((m >> 6) & 1u) << 2) | (((m >> 8) & 1u) << 3) |
         (((m >> 18) & 1u) << 4) | (((m >> 20) & 1u) << 5) | (((m >> 24) & 1u) << 6) |
         (((m >> 26) & 1u) << 7);
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l of the wave writes lds_base + 16 * l. `lds_base` must be wave-uniform.
__device__ inline void copy16_to_lds(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(g),
                                   (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}

// Staged operand rows are 64 bf16 = 128 bytes = eight 16-byte chunks; chunk c
// of row r sits at chunk position c ^ (r & 7), so eight consecutive rows read
// at one logical chunk hit eight different bank groups.
__device__ inline int swz(int row, int chunk) { return chunk ^ (row & 7); }

// 16-byte store marked non-temporal: outputs written once and not read again by
// the kernel, kept from displacing the gathered rows and weights in the caches.
__device__ __forceinline__ void store_stream(uint4* dst, uint4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(dst));
}

// Epilogue activation in fp32. SiLU(v) = v / (1 + e^-v), with e^-v taken as
// 2^(-v log2 e) on the hardware base-2 exponential and the quotient as a
// product with the hardware reciprocal (each about 1 ulp): a handful of
// instructions per element instead of a library exp and an IEEE divide. At
// v < -88 the reciprocal of the overflowed denominator is 0 and the result is
// -0 (the exact value is below 1e-36 in magnitude).
constexpr int kActNone = TR_SC_ACT_NONE, kActRelu = TR_SC_ACT_RELU, kActSilu = TR_SC_ACT_SILU;
__device__ __forceinline__ float activate(float v, int act) {
  if (act == kActRelu) return v < 0.f ? 0.f : v;
  if (act == kActSilu) return v * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f));
  return v;
}

// Workgroup barrier without the release fence of __syncthreads(): that fence
// waits for every outstanding global_load_lds (they count as LDS stores), even
// ones whose data is not needed yet. Callers wait for the copies they need with
// s_waitcnt before it. The memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ inline void bare_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ inline void stage_barrier() {  // all but this wave's newest copy have landed
  __builtin_amdgcn_s_waitcnt(0x0F71);
  bare_barrier();
}

// ---------------------------------------------------------------------------
// bf16 helpers (bit patterns in uint16_t).
// ---------------------------------------------------------------------------
__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ inline uint16_t f32_to_bf16_rne(float f) {  // finite inputs; NaN kept quiet
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return uint16_t((u >> 16) | 0x40u);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

}  // namespace trsc
