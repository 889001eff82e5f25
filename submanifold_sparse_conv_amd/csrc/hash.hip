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
constexpr int kMaxSortWGs = 768;  // tiles per radix pass: keys per tile grow until n fits
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
// its keys and an out-of-range flag in part[3 * block + {0, 1, 2}].
__global__ __launch_bounds__(kThreads) void pack_keys(const int4* __restrict__ coords, int64_t n,
                                                      uint64_t* __restrict__ keys,
                                                      int32_t* __restrict__ rows,
                                                      unsigned long long* __restrict__ part) {
  __shared__ unsigned long long s_or[kThreads / 64], s_and[kThreads / 64];
  __shared__ int s_bad[kThreads / 64];
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
  k_or = wave_or(k_or);
  k_and = wave_and(k_and);
  const int wave = threadIdx.x >> 6;
  const bool wbad = __ballot(bad) != 0;
  if ((threadIdx.x & 63) == 0) {
    s_or[wave] = k_or;
    s_and[wave] = k_and;
    s_bad[wave] = wbad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int anybad = s_bad[0];
    for (int w = 1; w < kThreads / 64; ++w) {
      k_or |= s_or[w];
      k_and &= s_and[w];
      anybad |= s_bad[w];
    }
    part[3 * blockIdx.x] = k_or;
    part[3 * blockIdx.x + 1] = k_and;
    part[3 * blockIdx.x + 2] = anybad ? 1ull : 0ull;
  }
}

// Initialises the header: flags, an empty-table capacity, the OR / AND of all
// keys, and the radix digits. The key bits that differ between keys (OR ^ AND)
// are split, least significant first, into three digits of equal width (at
// most kMaxDigitBits); any further bits go to the single-workgroup pass. The
// header is assembled in LDS (varying bit b, of rank r among them, is written
// by thread b) and copied out in 4-byte words.
__global__ __launch_bounds__(kThreads) void reduce_bits(const unsigned long long* __restrict__ part,
                                                        int nparts, HashHeader* hdr) {
  static_assert(sizeof(HashHeader) % 4 == 0 && sizeof(HashHeader) / 4 <= kThreads, "header copy");
  constexpr int HW = int(sizeof(HashHeader) / 4);
  __shared__ unsigned long long s_or[kThreads / 64], s_and[kThreads / 64];
  __shared__ unsigned long long s_bad[kThreads / 64];
  __shared__ HashHeader s_h;
  const int tid = threadIdx.x;
  unsigned long long k_or = 0, k_and = ~0ull, bad = 0;
  for (int i = tid; i < nparts; i += kThreads) {
    k_or |= part[3 * i];
    k_and &= part[3 * i + 1];
    bad |= part[3 * i + 2];
  }
  k_or = wave_or(k_or);
  k_and = wave_and(k_and);
  bad = wave_or(bad);
  if ((tid & 63) == 0) {
    s_or[tid >> 6] = k_or;
    s_and[tid >> 6] = k_and;
    s_bad[tid >> 6] = bad;
  }
  if (tid < HW) reinterpret_cast<uint32_t*>(&s_h)[tid] = 0u;
  __syncthreads();
  k_or = s_or[0], k_and = s_and[0], bad = s_bad[0];
  for (int w = 1; w < kThreads / 64; ++w) {
    k_or |= s_or[w];
    k_and &= s_and[w];
    bad |= s_bad[w];
  }
  const unsigned long long vary = nparts > 0 ? (k_or ^ k_and) : 0ull;
  const int nv = __popcll(vary);
  int w = (nv + 2) / 3;
  if (w > kMaxDigitBits) w = kMaxDigitBits;
  if (tid < 64 && ((vary >> tid) & 1ull)) {  // then w >= 1
    const int r = __popcll(vary & ((1ull << tid) - 1ull));
    if (r < 3 * w)
      s_h.digit[r / w].pos[r % w] = uint8_t(tid);
    else
      s_h.rest_pos[r - 3 * w] = uint8_t(tid);
  }
  if (tid == 0) {
    s_h.flags = bad ? kFlagCoordRange : 0u;
    s_h.nblocks = 0;
    s_h.cap_mask = 15;
    s_h.shift = 60;
    s_h.or_bits = k_or;
    s_h.and_bits = k_and;
    for (int d = 0; d < 3; ++d) {
      const int left = nv - d * w;
      s_h.digit[d].nbits = left < 0 ? 0 : (left > w ? w : left);
    }
    s_h.rest_n = nv > 3 * w ? nv - 3 * w : 0;
  }
  __syncthreads();
  if (tid < HW) reinterpret_cast<uint32_t*>(hdr)[tid] = reinterpret_cast<const uint32_t*>(&s_h)[tid];
}

__device__ inline uint32_t digit_of(uint64_t key, const uint8_t* pos, int nbits) {
  uint32_t d = 0;
  for (int j = 0; j < nbits; ++j) d |= uint32_t((key >> pos[j]) & 1u) << j;
  return d;
}

constexpr int kMaxBuckets = 1 << kMaxDigitBits;
constexpr int kColscanWGs = 1024;  // radix_colscan workgroups (each scans digits g, g + 1024, ...)

// counts[d * nblocks + block] = number of keys of this block's tile with digit d
// (d below 2^nbits of the pass's digit).
template <int ITEMS>
__global__ __launch_bounds__(kThreads) void radix_hist(const uint64_t* __restrict__ keys, int64_t n,
                                                       const HashHeader* __restrict__ hdr, int pass,
                                                       uint32_t* __restrict__ counts) {
  __shared__ uint32_t h[kMaxBuckets];
  __shared__ uint8_t s_pos[12];
  const int nbits = hdr->digit[pass].nbits;
  const int nb = 1 << nbits;
  if (threadIdx.x < 12) s_pos[threadIdx.x] = hdr->digit[pass].pos[threadIdx.x];
  for (int d = threadIdx.x; d < nb; d += kThreads) h[d] = 0;
  __syncthreads();
  const int64_t base = int64_t(blockIdx.x) * (kThreads * ITEMS);
  uint64_t kv[ITEMS];  // the tile's keys, loaded before any is counted
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int64_t i = base + it * kThreads + threadIdx.x;
    kv[it] = i < n ? keys[i] : 0ull;
  }
#pragma unroll
  for (int it = 0; it < ITEMS; ++it)
    if (base + it * kThreads + threadIdx.x < n) atomicAdd(&h[digit_of(kv[it], s_pos, nbits)], 1u);
  __syncthreads();
  for (int d = threadIdx.x; d < nb; d += kThreads) counts[int64_t(d) * gridDim.x + blockIdx.x] = h[d];
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

// Workgroup g scans digits g, g + gridDim.x, ...: exclusive scan over blocks
// of counts[d][*] in place; totals[d] = number of keys with digit d (0 for
// digits the pass lacks).
__global__ __launch_bounds__(kThreads) void radix_colscan(uint32_t* __restrict__ counts, int nblocks,
                                                          const HashHeader* __restrict__ hdr, int pass,
                                                          uint32_t* __restrict__ totals) {
  __shared__ uint32_t s_tmp[kThreads / 64];
  const int nb = 1 << hdr->digit[pass].nbits;
  for (int d = blockIdx.x; d < kMaxBuckets; d += gridDim.x) {
    if (d >= nb) {
      if (threadIdx.x == 0) totals[d] = 0;
      continue;
    }
    uint32_t* col = counts + int64_t(d) * nblocks;
    uint32_t carry = 0;
    // CPT consecutive entries per thread: one scan covers a whole pass of up to
    // kMaxSortWGs tiles, its loads all in flight together.
    constexpr int CPT = (kMaxSortWGs + kThreads - 1) / kThreads;
    for (int b0 = 0; b0 < nblocks; b0 += kThreads * CPT) {
      uint32_t v[CPT], sum = 0;
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int b = b0 + threadIdx.x * CPT + q;
        v[q] = b < nblocks ? col[b] : 0u;
        sum += v[q];
      }
      uint32_t tot;
      uint32_t ex = carry + block_exclusive_scan(sum, s_tmp, &tot);
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int b = b0 + threadIdx.x * CPT + q;
        if (b < nblocks) col[b] = ex;
        ex += v[q];
      }
      carry += tot;
    }
    if (threadIdx.x == 0) totals[d] = carry;
  }
}

// Stable scatter of one radix pass. Inside a tile, key order is (iteration,
// wave, lane); ranks among equal digits follow that order.
template <int ITEMS>
__global__ __launch_bounds__(kThreads) void radix_scatter(const uint64_t* __restrict__ kin,
                                                          const int32_t* __restrict__ vin,
                                                          uint64_t* __restrict__ kout,
                                                          int32_t* __restrict__ vout, int64_t n,
                                                          const HashHeader* __restrict__ hdr, int pass,
                                                          const uint32_t* __restrict__ offsets,
                                                          const uint32_t* __restrict__ totals) {
  constexpr int PER = kMaxBuckets / kThreads;  // digits per thread in the digit scan
  __shared__ uint32_t base_off[kMaxBuckets];
  __shared__ uint32_t wcount[kThreads / 64][kMaxBuckets];
  __shared__ uint32_t s_tmp[kThreads / 64];
  __shared__ uint8_t s_pos[12];
  const int nbits = hdr->digit[pass].nbits;
  const int nb = 1 << nbits;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (threadIdx.x < 12) s_pos[threadIdx.x] = hdr->digit[pass].pos[threadIdx.x];
  // exclusive scan of the digit totals: thread t owns digits t*PER .. t*PER+PER-1
  uint32_t loc[PER], sum = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    loc[q] = totals[threadIdx.x * PER + q];
    sum += loc[q];
  }
  uint32_t all;
  uint32_t run = block_exclusive_scan(sum, s_tmp, &all);
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int d = threadIdx.x * PER + q;
    if (d < nb) base_off[d] = run + offsets[int64_t(d) * gridDim.x + blockIdx.x];
    run += loc[q];
  }
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int64_t base = int64_t(blockIdx.x) * (kThreads * ITEMS);
  uint64_t kv[ITEMS];  // the tile's keys and rows, loaded before the first is ranked
  int32_t vv[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int64_t i = base + it * kThreads + threadIdx.x;
    kv[it] = i < n ? kin[i] : 0ull;
    vv[it] = i < n ? vin[i] : 0;
  }
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    for (int d = threadIdx.x; d < nb; d += kThreads)
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) wcount[w][d] = 0;
    __syncthreads();
    const int64_t i = base + it * kThreads + threadIdx.x;
    const bool valid = i < n;
    const uint64_t key = kv[it];
    const int32_t val = vv[it];
    const uint32_t d = valid ? digit_of(key, s_pos, nbits) : 0u;
    unsigned long long peers = __ballot(valid);
    for (int j = 0; j < nbits; ++j) {
      const bool bit = (d >> j) & 1u;
      const unsigned long long bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
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
    for (int dd = threadIdx.x; dd < nb; dd += kThreads) {
      uint32_t add = 0;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) add += wcount[w][dd];
      base_off[dd] += add;
    }
    __syncthreads();
  }
}

// The key bits beyond the three digits (only when more than 3 * kMaxDigitBits
// bits vary): one workgroup sorts keys[0..n) stably by them, 8 bits per pass,
// using tmp as the other buffer, and leaves the result in keys / rows.
__global__ __launch_bounds__(kThreads) void radix_rest(uint64_t* __restrict__ keys, int32_t* __restrict__ rows,
                                                       uint64_t* __restrict__ tkeys, int32_t* __restrict__ trows,
                                                       int64_t n, const HashHeader* __restrict__ hdr) {
  __shared__ uint32_t hist[256], base_off[256];
  __shared__ uint32_t wcount[kThreads / 64][256];
  __shared__ uint32_t s_tmp[kThreads / 64];
  __shared__ uint8_t s_pos[8];
  const int rest = hdr->rest_n;
  if (rest == 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long lt = (1ull << lane) - 1ull;
  uint64_t* ka = keys;
  int32_t* ra = rows;
  uint64_t* kb = tkeys;
  int32_t* rb = trows;
  for (int p0 = 0; p0 < rest; p0 += 8) {
    const int nbits = rest - p0 < 8 ? rest - p0 : 8;
    if (threadIdx.x < 8) s_pos[threadIdx.x] = threadIdx.x < nbits ? hdr->rest_pos[p0 + threadIdx.x] : 0;
    hist[threadIdx.x] = 0;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += kThreads) atomicAdd(&hist[digit_of(ka[i], s_pos, nbits)], 1u);
    __syncthreads();
    uint32_t all;
    base_off[threadIdx.x] = block_exclusive_scan(hist[threadIdx.x], s_tmp, &all);
    for (int64_t t0 = 0; t0 < n; t0 += kThreads) {
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) wcount[w][threadIdx.x] = 0;
      __syncthreads();
      const int64_t i = t0 + threadIdx.x;
      const bool valid = i < n;
      uint64_t key = valid ? ka[i] : 0ull;
      const int32_t val = valid ? ra[i] : 0;
      const uint32_t d = digit_of(key, s_pos, nbits);
      unsigned long long peers = __ballot(valid);
      for (int j = 0; j < nbits; ++j) {
        const bool bit = (d >> j) & 1u;
        const unsigned long long bal = __ballot(bit);
        peers &= bit ? bal : ~bal;
      }
      if (valid && (peers & lt) == 0) wcount[wave][d] = __popcll(peers);
      __syncthreads();
      if (valid) {
        uint32_t pos = base_off[d] + __popcll(peers & lt);
        for (int w = 0; w < wave; ++w) pos += wcount[w][d];
        kb[pos] = key;
        rb[pos] = val;
      }
      __syncthreads();
      uint32_t add = 0;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) add += wcount[w][threadIdx.x];
      base_off[threadIdx.x] += add;
      __syncthreads();
    }
    uint64_t* kt = ka;
    ka = kb;
    kb = kt;
    int32_t* rt = ra;
    ra = rb;
    rb = rt;
  }
  if (ka != keys) {  // an odd number of passes: copy back
    for (int64_t i = threadIdx.x; i < n; i += kThreads) {
      keys[i] = ka[i];
      rows[i] = ra[i];
    }
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

// The lane at each block head inserts {block key, occupancy bitmap, start}.
// The bitmap is a segmented OR over the lanes of the wave that hold the same
// block (sorted keys make a block one run of lanes); only a block that runs
// past the wave's last lane is finished by its head with a short serial loop.
__global__ __launch_bounds__(kThreads) void block_insert(const uint64_t* __restrict__ keys, int64_t n,
                                                         BlockSlot* __restrict__ slots, HashHeader* hdr) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const bool valid = t < n;
  const uint64_t k = valid ? keys[t] : ~0ull;
  const uint64_t bkey = k >> 6;
  const bool head = valid && (t == 0 || (keys[t - 1] >> 6) != bkey);
  uint64_t bits = valid ? (1ull << (k & 63u)) : 0ull;
  for (int o = 1; o < 64; o <<= 1) {  // bits of lanes [lane, lane + 2o) of the same block
    const uint64_t ob = __shfl_down(bits, o, 64);
    const uint64_t okey = __shfl_down(bkey, o, 64);
    if (lane + o < 64 && okey == bkey) bits |= ob;
  }
  const uint64_t last_key = __shfl(bkey, 63, 64);
  if (!head) return;
  if (last_key == bkey) {  // the block may continue in the next wave
    for (int64_t u = t - lane + 64; u < n && u < t + 64; ++u) {
      const uint64_t ku = keys[u];
      if ((ku >> 6) != bkey) break;
      bits |= 1ull << (ku & 63u);
    }
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


inline unsigned grid_for(int64_t n, int per_block) { return unsigned((n + per_block - 1) / per_block); }

}  // namespace

// Keys per radix tile: kThreads times the smallest power of two (<= 32) that
// keeps a pass at no more than kMaxSortWGs workgroups.
int sort_items(int64_t n) {
  int it = 1;
  while (it < 32 && (n + int64_t(kThreads) * it - 1) / (int64_t(kThreads) * it) > kMaxSortWGs) it *= 2;
  return it;
}
int64_t sort_blocks(int64_t n) {
  const int64_t tile = int64_t(kThreads) * sort_items(n);
  return (n + tile - 1) / tile;
}
int64_t pack_partials(int64_t n) {
  const int64_t b = (n + kThreads - 1) / kThreads;
  return b < 1 ? 1 : (b < kPackBlocks ? b : kPackBlocks);
}

hipError_t launch_pack(const int32_t* coords, int64_t n, uint64_t* keys, int32_t* rows,
                       unsigned long long* part, HashHeader* hdr, hipStream_t st) {
  const int nb = n > 0 ? int(pack_partials(n)) : 0;
  if (n > 0)
    pack_keys<<<nb, kThreads, 0, st>>>(reinterpret_cast<const int4*>(coords), n, keys, rows, part);
  reduce_bits<<<1, kThreads, 0, st>>>(part, nb, hdr);
  return hipGetLastError();
}

hipError_t launch_sort(uint64_t* keys0, int32_t* rows0, uint64_t* keys1, int32_t* rows1, int64_t n,
                       const HashHeader* hdr, uint32_t* counts, uint32_t* totals, hipStream_t st) {
  const int64_t nb = sort_blocks(n);
  uint64_t* k[2] = {keys0, keys1};
  int32_t* r[2] = {rows0, rows1};
  const int items = sort_items(n);
  for (int pass = 0; pass < 3; ++pass) {
    const int a = pass & 1;  // 0 -> 1 -> 0 -> 1
    switch (items) {
#define TRSC_RADIX_PASS(IT)                                                                                   \
  case IT:                                                                                                    \
    radix_hist<IT><<<unsigned(nb), kThreads, 0, st>>>(k[a], n, hdr, pass, counts);                            \
    radix_colscan<<<kColscanWGs, kThreads, 0, st>>>(counts, int(nb), hdr, pass, totals);                      \
    radix_scatter<IT><<<unsigned(nb), kThreads, 0, st>>>(k[a], r[a], k[a ^ 1], r[a ^ 1], n, hdr, pass, counts, \
                                                         totals);                                             \
    break;
      TRSC_RADIX_PASS(1)
      TRSC_RADIX_PASS(2)
      TRSC_RADIX_PASS(4)
      TRSC_RADIX_PASS(8)
      TRSC_RADIX_PASS(16)
      TRSC_RADIX_PASS(32)
#undef TRSC_RADIX_PASS
      default:
        return hipErrorInvalidValue;
    }
  }
  radix_rest<<<1, kThreads, 0, st>>>(keys1, rows1, keys0, rows0, n, hdr);
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
