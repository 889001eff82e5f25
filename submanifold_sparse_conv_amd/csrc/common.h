// Internal definitions shared by the HIP kernels of the library (not part of
// the C ABI). gfx950 only: wave64, 64-bit ballots.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

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
constexpr uint64_t kEmptyKey = ~0ull;  // also the key of (65535,65535,65535,65535)

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
// Open-addressing table. 16-byte slots {key, row}; EMPTY key = ~0. The one
// valid key equal to ~0 (every component 65535) lives outside the table in
// HashHeader::special_row. Capacity is a power of two >= 4N (load <= 1/4).
//
// Home slot: Fibonacci (multiplicative) hashing of the whole key, top bits of
// key * 2^64/phi. Collisions are resolved by linear probing. Hashing whole keys
// keeps probe runs short; grouping the 8 voxels of a 2x2x2 brick into one run
// of slots gives better cache-line locality but makes clusters that lengthen
// the probe chains several-fold, and the lookups are latency-bound.
// ---------------------------------------------------------------------------
struct alignas(16) Slot {
  uint64_t key;
  int32_t row;
  int32_t pad;
};

constexpr uint32_t kFlagCoordRange = 1u;
constexpr uint32_t kFlagDuplicate = 2u;
constexpr uint32_t kFlagCapacity = 4u;

struct alignas(256) HashHeader {
  uint32_t flags;
  int32_t special_row;
  uint32_t pad0, pad1;
  unsigned long long or_bits;   // OR of all keys
  unsigned long long and_bits;  // AND of all keys
};

struct TableRef {
  const Slot* slots;
  uint32_t mask;   // capacity - 1 (capacity a power of two >= 16)
  uint32_t shift;  // 64 - log2(capacity)
};

__host__ __device__ inline uint32_t home_slot(uint64_t key, uint32_t shift) {
  return uint32_t((key * 0x9E3779B97F4A7C15ull) >> shift);
}

__device__ inline uint4 load_slot(const Slot* slots, uint32_t s) {
  return *reinterpret_cast<const uint4*>(slots + s);
}

__device__ inline uint64_t slot_key(const uint4& v) { return uint64_t(v.x) | (uint64_t(v.y) << 32); }

// Continues a probe run whose first slot s (already loaded into v) did not
// decide the lookup by itself.
__device__ inline int32_t probe_from(const TableRef& t, uint64_t key, uint32_t s, uint4 v) {
  for (uint32_t probe = 0; probe <= t.mask; ++probe) {
    const uint64_t k = slot_key(v);
    if (k == key) return int32_t(v.z);
    if (k == kEmptyKey) return -1;
    s = (s + 1) & t.mask;
    v = load_slot(t.slots, s);
  }
  return -1;
}

__device__ inline int32_t table_find(const TableRef& t, uint64_t key, int32_t special_row) {
  if (key == kEmptyKey) return special_row;
  const uint32_t s = home_slot(key, t.shift);
  return probe_from(t, key, s, load_slot(t.slots, s));
}

// Workgroup index -> work index such that each XCD (workgroups are dealt to
// the 8 XCDs of the chip round-robin) gets one contiguous run of work items, so
// neighbouring work (Morton-adjacent voxels) shares that XCD's L2.
__device__ inline int xcd_remap(int bid, int grid) {
  const int xcd = bid & 7, local = bid >> 3;
  const int per = grid >> 3, rem = grid & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
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
