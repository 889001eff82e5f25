// Coordinate hash: key packing, Morton radix sort, and the open-addressing
// table of occupied 4x4x4 blocks (occupancy bitmap + first sorted position).
// This is the "spatial hash of the active voxels" of the sparse convolution
// ("Running TRELLIS.2 on a Mac (1/3)", section "Swapping out the CUDA libraries
// one at a time"), built on the device in HBM. The voxels are first sorted along
// the Z-order curve: a block's voxels are then consecutive, and the kernel-map
// pass and the gather-GEMM tiles walk space in compact pieces.
#include "common.h"
#include "launch.h"

namespace trsc {

namespace {

constexpr int kThreads = 256;
constexpr int kItems = 8;
constexpr int kTile = kThreads * kItems;  // keys per sort block
constexpr int kPackBlocks = 1024;         // grid of the key-packing pass

__device__ inline unsigned long long wave_or(unsigned long long v) {
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, 64);
  return v;
}
__device__ inline unsigned long long wave_and(unsigned long long v) {
  for (int o = 32; o > 0; o >>= 1) v &= __shfl_xor(v, o, 64);
  return v;
}

// keys[i] = key of coords[i]; rows[i] = i. Each block leaves the OR and AND of
// its keys in part[2 * block + {0, 1}]; out-of-range coordinates set a flag.
__global__ __launch_bounds__(kThreads) void pack_keys(const int4* __restrict__ coords, int64_t n,
                                                      uint64_t* __restrict__ keys,
                                                      int32_t* __restrict__ rows,
                                                      unsigned long long* __restrict__ part,
                                                      HashHeader* hdr) {
  __shared__ unsigned long long s_or[kThreads / 64], s_and[kThreads / 64];
  unsigned long long k_or = 0, k_and = ~0ull;
  bool bad = false;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * kThreads) {
    const int4 c = coords[i];
    const bool b = (uint32_t(c.x) | uint32_t(c.y) | uint32_t(c.z) | uint32_t(c.w)) > 0xFFFFu;
    bad |= b;
    const uint64_t key = b ? 0ull : make_key(uint32_t(c.x), uint32_t(c.y), uint32_t(c.z), uint32_t(c.w));
    keys[i] = key;
    rows[i] = int32_t(i);
    k_or |= key;
    k_and &= key;
  }
  if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0) atomicOr(&hdr->flags, kFlagCoordRange);
  k_or = wave_or(k_or);
  k_and = wave_and(k_and);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_or[wave] = k_or;
    s_and[wave] = k_and;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w) {
      k_or |= s_or[w];
      k_and &= s_and[w];
    }
    part[2 * blockIdx.x] = k_or;
    part[2 * blockIdx.x + 1] = k_and;
  }
}

__global__ __launch_bounds__(kThreads) void reduce_bits(const unsigned long long* __restrict__ part,
                                                        int nparts, HashHeader* hdr) {
  __shared__ unsigned long long s_or[kThreads / 64], s_and[kThreads / 64];
  unsigned long long k_or = 0, k_and = ~0ull;
  for (int i = threadIdx.x; i < nparts; i += kThreads) {
    k_or |= part[2 * i];
    k_and &= part[2 * i + 1];
  }
  k_or = wave_or(k_or);
  k_and = wave_and(k_and);
  if ((threadIdx.x & 63) == 0) {
    s_or[threadIdx.x >> 6] = k_or;
    s_and[threadIdx.x >> 6] = k_and;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w) {
      k_or |= s_or[w];
      k_and &= s_and[w];
    }
    hdr->or_bits = k_or;
    hdr->and_bits = k_and;
  }
}

__device__ inline uint32_t digit_of(uint64_t key, const DigitSel& sel) {
  uint32_t d = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < sel.nbits) d |= uint32_t((key >> sel.pos[j]) & 1u) << j;
  return d;
}

// counts[d * nblocks + block] = number of keys of this block's tile with digit d.
__global__ __launch_bounds__(kThreads) void radix_hist(const uint64_t* __restrict__ keys, int64_t n,
                                                       DigitSel sel, uint32_t* __restrict__ counts) {
  __shared__ uint32_t h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = int64_t(blockIdx.x) * kTile;
  for (int it = 0; it < kItems; ++it) {
    const int64_t i = base + it * kThreads + threadIdx.x;
    if (i < n) atomicAdd(&h[digit_of(keys[i], sel)], 1u);
  }
  __syncthreads();
  counts[int64_t(threadIdx.x) * gridDim.x + blockIdx.x] = h[threadIdx.x];
}

// Block-wide exclusive scan of one value per thread (256 threads).
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (int w = 0; w < kThreads / 64; ++w) {
    if (w < wave) before += s_tmp[w];
    all += s_tmp[w];
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// One workgroup per digit d: exclusive scan over blocks of counts[d][*] in
// place; totals[d] = number of keys with digit d.
__global__ __launch_bounds__(kThreads) void radix_colscan(uint32_t* __restrict__ counts, int nblocks,
                                                          uint32_t* __restrict__ totals) {
  __shared__ uint32_t s_tmp[kThreads / 64];
  uint32_t* col = counts + int64_t(blockIdx.x) * nblocks;
  uint32_t carry = 0;
  for (int b0 = 0; b0 < nblocks; b0 += kThreads) {
    const int b = b0 + threadIdx.x;
    const uint32_t v = b < nblocks ? col[b] : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan(v, s_tmp, &tot);
    if (b < nblocks) col[b] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = carry;
}

// Stable scatter of one radix pass. Inside a tile, key order is (iteration,
// wave, lane); ranks among equal digits follow that order.
__global__ __launch_bounds__(kThreads) void radix_scatter(const uint64_t* __restrict__ kin,
                                                          const int32_t* __restrict__ vin,
                                                          uint64_t* __restrict__ kout,
                                                          int32_t* __restrict__ vout, int64_t n,
                                                          DigitSel sel,
                                                          const uint32_t* __restrict__ offsets,
                                                          const uint32_t* __restrict__ totals) {
  __shared__ uint32_t base_off[256];
  __shared__ uint32_t wcount[kThreads / 64][256];
  __shared__ uint32_t s_tmp[kThreads / 64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t all;
  const uint32_t digit_base = block_exclusive_scan(totals[threadIdx.x], s_tmp, &all);
  base_off[threadIdx.x] = digit_base + offsets[int64_t(threadIdx.x) * gridDim.x + blockIdx.x];
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int64_t base = int64_t(blockIdx.x) * kTile;
  for (int it = 0; it < kItems; ++it) {
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) wcount[w][threadIdx.x] = 0;
    __syncthreads();
    const int64_t i = base + it * kThreads + threadIdx.x;
    const bool valid = i < n;
    uint64_t key = 0;
    int32_t val = 0;
    uint32_t d = 0;
    if (valid) {
      key = kin[i];
      val = vin[i];
      d = digit_of(key, sel);
    }
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < sel.nbits) {
        const bool bit = (d >> j) & 1u;
        const unsigned long long bal = __ballot(bit);
        peers &= bit ? bal : ~bal;
      }
    }
    const uint32_t rank = __popcll(peers & lt);
    if (valid && (peers & lt) == 0) wcount[wave][d] = __popcll(peers);
    __syncthreads();
    if (valid) {
      uint32_t pos = base_off[d] + rank;
      for (int w = 0; w < wave; ++w) pos += wcount[w][d];
      kout[pos] = key;
      vout[pos] = val;
    }
    __syncthreads();
    uint32_t add = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) add += wcount[w][threadIdx.x];
    base_off[threadIdx.x] += add;
    __syncthreads();
  }
}

// Each workgroup counts the block heads among its sorted keys (first key of
// each 4x4x4 block) into part[block] and flags adjacent equal keys (duplicate
// coordinates: equal keys are adjacent after the sort).
__global__ __launch_bounds__(kThreads) void block_count(const uint64_t* __restrict__ keys, int64_t n,
                                                        uint32_t* __restrict__ part, HashHeader* hdr) {
  __shared__ uint32_t s_cnt[kThreads / 64];
  uint32_t cnt = 0;
  bool dup = false;
  for (int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x; t < n; t += int64_t(gridDim.x) * kThreads) {
    const uint64_t k = keys[t];
    const uint64_t prev = t > 0 ? keys[t - 1] : ~k;
    cnt += (t == 0 || (prev >> 6) != (k >> 6)) ? 1u : 0u;
    dup |= t > 0 && prev == k;
  }
  if (__ballot(dup) != 0 && (threadIdx.x & 63) == 0) atomicOr(&hdr->flags, kFlagDuplicate);
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if ((threadIdx.x & 63) == 0) s_cnt[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t c = 0;
    for (int w = 0; w < kThreads / 64; ++w) c += s_cnt[w];
    part[blockIdx.x] = c;
  }
}

// One workgroup: number of blocks, table capacity (power of two >= 2x blocks,
// at least 16, at most max_cap) and hash shift, into the header.
__global__ __launch_bounds__(kThreads) void block_size(const uint32_t* __restrict__ part, int nparts,
                                                       uint32_t max_cap, HashHeader* hdr) {
  __shared__ uint32_t s_cnt[kThreads / 64];
  uint32_t c = 0;
  for (int i = threadIdx.x; i < nparts; i += kThreads) c += part[i];
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if ((threadIdx.x & 63) == 0) s_cnt[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t nb = 0;
    for (int w = 0; w < kThreads / 64; ++w) nb += s_cnt[w];
    uint32_t cap = 16, lg = 4;
    while (cap < 2u * nb && cap < max_cap) {
      cap <<= 1;
      ++lg;
    }
    hdr->nblocks = nb;
    hdr->cap_mask = cap - 1;
    hdr->shift = 64 - lg;
  }
}

__global__ __launch_bounds__(kThreads) void block_clear(BlockSlot* __restrict__ slots,
                                                        const HashHeader* __restrict__ hdr) {
  const uint32_t cap = hdr->cap_mask + 1u;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < cap; i += gridDim.x * kThreads) {
    uint4* p = reinterpret_cast<uint4*>(slots + i);
    p[0] = make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0u, 0u);
    p[1] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// The thread at each block head builds the block's occupancy bitmap from the
// following sorted keys (at most 64) and inserts {block key, bitmap, start}.
__global__ __launch_bounds__(kThreads) void block_insert(const uint64_t* __restrict__ keys, int64_t n,
                                                         BlockSlot* __restrict__ slots, HashHeader* hdr) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= n) return;
  const uint64_t k = keys[t];
  const uint64_t bkey = k >> 6;
  if (t > 0 && (keys[t - 1] >> 6) == bkey) return;
  uint64_t bits = 0;
  for (int64_t u = t; u < n && u < t + 64; ++u) {
    const uint64_t ku = keys[u];
    if ((ku >> 6) != bkey) break;
    bits |= 1ull << (ku & 63u);
  }
  const uint32_t mask = hdr->cap_mask, shift = hdr->shift;
  uint32_t s = home_slot(bkey, shift) & mask;
  for (uint32_t probe = 0; probe <= mask; ++probe) {
    unsigned long long* kp = reinterpret_cast<unsigned long long*>(&slots[s].bkey);
    const unsigned long long prev = atomicCAS(kp, kEmptyKey, bkey);
    if (prev == kEmptyKey) {
      slots[s].bits = bits;
      slots[s].start = uint32_t(t);
      return;
    }
    s = (s + 1) & mask;
  }
  atomicOr(&hdr->flags, kFlagCapacity);
}

__global__ __launch_bounds__(kThreads) void table_lookup(TableRef t, const int4* __restrict__ q, int64_t nq,
                                                         int32_t* __restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= nq) return;
  const int4 c = q[i];
  if ((uint32_t(c.x) | uint32_t(c.y) | uint32_t(c.z) | uint32_t(c.w)) > 0xFFFFu) {
    out[i] = -1;
    return;
  }
  out[i] = voxel_find(t, t.hdr->cap_mask, t.hdr->shift,
                      make_key(uint32_t(c.x), uint32_t(c.y), uint32_t(c.z), uint32_t(c.w)));
}

__global__ void header_init(HashHeader* hdr) {
  hdr->flags = 0;
  hdr->nblocks = 0;
  hdr->cap_mask = 15;
  hdr->shift = 60;
  hdr->or_bits = 0ull;
  hdr->and_bits = ~0ull;
}

inline unsigned grid_for(int64_t n, int per_block) { return unsigned((n + per_block - 1) / per_block); }

}  // namespace

int64_t sort_blocks(int64_t n) { return (n + kTile - 1) / kTile; }
int64_t pack_partials(int64_t n) {
  const int64_t b = (n + kThreads - 1) / kThreads;
  return b < 1 ? 1 : (b < kPackBlocks ? b : kPackBlocks);
}

hipError_t launch_pack(const int32_t* coords, int64_t n, uint64_t* keys, int32_t* rows,
                       unsigned long long* part, HashHeader* hdr, hipStream_t st) {
  header_init<<<1, 1, 0, st>>>(hdr);
  if (n > 0) {
    const int nb = int(pack_partials(n));
    pack_keys<<<nb, kThreads, 0, st>>>(reinterpret_cast<const int4*>(coords), n, keys, rows, part, hdr);
    reduce_bits<<<1, kThreads, 0, st>>>(part, nb, hdr);
  }
  return hipGetLastError();
}

hipError_t launch_sort_pass(const uint64_t* kin, const int32_t* vin, uint64_t* kout, int32_t* vout,
                            int64_t n, const DigitSel& sel, uint32_t* counts, uint32_t* totals,
                            hipStream_t st) {
  const int64_t nb = sort_blocks(n);
  radix_hist<<<unsigned(nb), kThreads, 0, st>>>(kin, n, sel, counts);
  radix_colscan<<<256, kThreads, 0, st>>>(counts, int(nb), totals);
  radix_scatter<<<unsigned(nb), kThreads, 0, st>>>(kin, vin, kout, vout, n, sel, counts, totals);
  return hipGetLastError();
}

hipError_t launch_blocks(const uint64_t* keys, int64_t n, BlockSlot* slots, uint32_t max_cap,
                         uint32_t* part, HashHeader* hdr, hipStream_t st) {
  const int nb = int(pack_partials(n));
  if (n > 0) block_count<<<nb, kThreads, 0, st>>>(keys, n, part, hdr);
  block_size<<<1, kThreads, 0, st>>>(part, n > 0 ? nb : 0, max_cap, hdr);
  const uint32_t cb = (max_cap + kThreads - 1) / kThreads;
  block_clear<<<cb < 2048u ? cb : 2048u, kThreads, 0, st>>>(slots, hdr);
  if (n > 0) block_insert<<<grid_for(n, kThreads), kThreads, 0, st>>>(keys, n, slots, hdr);
  return hipGetLastError();
}

hipError_t launch_lookup(const TableRef& t, const int32_t* q, int64_t nq, int32_t* out, hipStream_t st) {
  if (nq > 0)
    table_lookup<<<grid_for(nq, kThreads), kThreads, 0, st>>>(t, reinterpret_cast<const int4*>(q), nq, out);
  return hipGetLastError();
}

}  // namespace trsc
