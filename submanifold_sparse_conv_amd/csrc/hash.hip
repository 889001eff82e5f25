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
constexpr int kSmallDigitBits = 8;  // digits up to this width are ranked in one sweep per tile
constexpr int kMaxSortWGs = 768;  // tiles per radix pass: keys per tile grow until n fits
constexpr int kPackBlocks = 256;          // grid of the key-packing pass (its partials are read by
                                          // every workgroup of the first histogram pass)

__device__ inline unsigned long long wave_or(unsigned long long v) {
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, 64);
  return v;
}
__device__ inline unsigned long long wave_and(unsigned long long v) {
  for (int o = 32; o > 0; o >>= 1) v &= __shfl_xor(v, o, 64);
  return v;
}

// keys[i] = keys2[i] = key of coords[i]; rows[i] = rows2[i] = i (the first
// radix pass that has bits reads whichever of the two buffers its parity
// gives). Each block leaves the OR and AND of its keys and an out-of-range
// flag (a spatial component >= lim or an object index >= blim) in
// part[3 * block + {0, 1, 2}].
__global__ __launch_bounds__(kThreads) void pack_keys(const int4* __restrict__ coords, int64_t n,
                                                      uint32_t lim, uint32_t blim, uint64_t* __restrict__ keys,
                                                      int32_t* __restrict__ rows,
                                                      uint64_t* __restrict__ keys2,
                                                      int32_t* __restrict__ rows2,
                                                      unsigned long long* __restrict__ part) {
  __shared__ unsigned long long s_or[kThreads / 64], s_and[kThreads / 64];
  __shared__ int s_bad[kThreads / 64];
  unsigned long long k_or = 0, k_and = ~0ull;
  bool bad = false;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * kThreads) {
    const int4 c = coords[i];
    const bool b = uint32_t(c.x) >= blim || uint32_t(c.y) >= lim || uint32_t(c.z) >= lim || uint32_t(c.w) >= lim;
    bad |= b;
    const uint64_t key = b ? 0ull : make_key(uint32_t(c.x), uint32_t(c.y), uint32_t(c.z), uint32_t(c.w));
    keys[i] = key;
    rows[i] = int32_t(i);
    keys2[i] = key;
    rows2[i] = int32_t(i);
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

// The header: flags, an empty-table capacity, the OR / AND of all keys, and the
// radix digits, from the packing pass's partials; built by a whole workgroup
// in LDS (s_h). The nv key bits that differ between keys (OR ^ AND) are split,
// least significant first, into P digits, the last one the rest: P =
// ceil(nv / 8) digits of at most 8 bits while that is at most kSortPasses (the
// scatter then ranks a tile in one sweep), else P = ceil(nv / kMaxDigitBits)
// digits of ceil(nv / P) bits (at most kSortPasses). They go to the last P
// passes, so that the last pass that moves data is always the last pass (its
// output buffer is the result); the passes before them have no bits and return
// at once. Bits beyond kSortPasses * kMaxDigitBits go to the single-workgroup
// pass. Varying bit b, of rank r among them, is written by thread b.
__device__ void build_header(const unsigned long long* __restrict__ part, int nparts, HashHeader& s_h) {
  constexpr int HW = int(sizeof(HashHeader) / 4);
  __shared__ unsigned long long s_or[kThreads / 64], s_and[kThreads / 64];
  __shared__ unsigned long long s_bad[kThreads / 64];
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
  int np = (nv + kSmallDigitBits - 1) / kSmallDigitBits;  // passes with bits
  if (np > kSortPasses) np = (nv + kMaxDigitBits - 1) / kMaxDigitBits;
  if (np > kSortPasses) np = kSortPasses;
  int w = np > 0 ? (nv + np - 1) / np : 0;
  if (w > kMaxDigitBits) w = kMaxDigitBits;  // more bits than the passes hold: the rest pass
  const int first = kSortPasses - np;        // the first pass with bits
  if (tid < 64 && ((vary >> tid) & 1ull)) {  // then w >= 1
    const int r = __popcll(vary & ((1ull << tid) - 1ull));
    if (r < np * w)
      s_h.digit[first + r / w].pos[r % w] = uint8_t(tid);
    else
      s_h.rest_pos[r - np * w] = uint8_t(tid);
  }
  if (tid == 0) {
    s_h.flags = bad ? kFlagCoordRange : 0u;
    s_h.nblocks = 0;
    s_h.cap_mask = 15;
    s_h.shift = 60;
    s_h.or_bits = k_or;
    s_h.and_bits = k_and;
    for (int d = 0; d < kSortPasses; ++d) {
      const int left = d < first ? 0 : nv - (d - first) * w;
      s_h.digit[d].nbits = left < 0 ? 0 : (left > w ? w : left);
    }
    s_h.rest_n = nv > np * w ? nv - np * w : 0;
  }
  __syncthreads();
}

__device__ inline void store_header(const HashHeader& s_h, HashHeader* hdr) {
  static_assert(sizeof(HashHeader) % 4 == 0 && sizeof(HashHeader) / 4 <= kThreads, "header copy");
  constexpr int HW = int(sizeof(HashHeader) / 4);
  if (threadIdx.x < HW)
    reinterpret_cast<uint32_t*>(hdr)[threadIdx.x] = reinterpret_cast<const uint32_t*>(&s_h)[threadIdx.x];
}

// The header of an empty voxel set (no histogram pass runs then).
__global__ __launch_bounds__(kThreads) void reduce_bits(const unsigned long long* __restrict__ part,
                                                        int nparts, HashHeader* hdr) {
  __shared__ HashHeader s_h;
  build_header(part, nparts, s_h);
  store_header(s_h, hdr);
}

__device__ inline uint32_t digit_of(uint64_t key, const uint8_t* pos, int nbits) {
  uint32_t d = 0;
  for (int j = 0; j < nbits; ++j) d |= uint32_t((key >> pos[j]) & 1u) << j;
  return d;
}

constexpr int kMaxBuckets = 1 << kMaxDigitBits;
constexpr int kColscanWGs = 1024;  // radix_colscan workgroups (each scans digits g, g + 1024, ...)

// counts[d * nblocks + block] = number of keys of this block's tile with digit d
// (d below 2^nbits of the pass's digit). The histogram of pass 0, the first one
// launched, also builds the header from the packing pass's partials: every
// workgroup derives the digits itself, and workgroup 0 stores the header for
// the kernels that follow.
template <int ITEMS>
__global__ __launch_bounds__(kThreads) void radix_hist(const uint64_t* __restrict__ keys, int64_t n,
                                                       HashHeader* hdr, int pass, uint32_t* __restrict__ counts,
                                                       const unsigned long long* __restrict__ part, int nparts) {
  __shared__ uint32_t h[kMaxBuckets];
  __shared__ uint8_t s_pos[12];
  __shared__ HashHeader s_h;
  int nbits;
  if (pass == 0) {
    build_header(part, nparts, s_h);
    if (blockIdx.x == 0) store_header(s_h, hdr);
    nbits = s_h.digit[0].nbits;
    if (threadIdx.x < 12) s_pos[threadIdx.x] = s_h.digit[0].pos[threadIdx.x];
  } else {
    nbits = hdr->digit[pass].nbits;
    if (threadIdx.x < 12) s_pos[threadIdx.x] = hdr->digit[pass].pos[threadIdx.x];
  }
  nbits = min(nbits, kMaxDigitBits);  // never more buckets than the LDS holds
  if (nbits == 0) return;  // a pass without bits moves nothing
  const int nb = 1 << nbits;
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
  const int nbits = min(hdr->digit[pass].nbits, kMaxDigitBits);
  if (nbits == 0) return;
  const int nb = 1 << nbits;
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
// wave, lane); ranks among equal digits follow that order. Each thread first
// holds the base offsets of its digits: the digits below them over all tiles
// (scan of the totals) plus this digit in the tiles before this one (colscan).
//
// Digits of at most kSmallDigitBits bits: a wave ranks each of its keys among
// the equal digits of the same (iteration, wave) with ballots, the first lane
// of each digit stores the digit's count for that (iteration, wave), and the
// thread that owns the digit turns its counts into positions in (iteration,
// wave) order, items kChunk at a time: four barriers per chunk.
// Wider digits (up to kMaxDigitBits, 2048 buckets, whose counts per (iteration,
// wave) would not fit the LDS): the same ranking one iteration at a time, with
// per-wave counts.
template <int ITEMS>
__global__ __launch_bounds__(kThreads) void radix_scatter(const uint64_t* __restrict__ kin,
                                                          const int32_t* __restrict__ vin,
                                                          uint64_t* __restrict__ kout,
                                                          int32_t* __restrict__ vout, int64_t n,
                                                          const HashHeader* __restrict__ hdr, int pass,
                                                          const uint32_t* __restrict__ offsets,
                                                          const uint32_t* __restrict__ totals) {
  constexpr int PER = kMaxBuckets / kThreads;  // digits per thread in the digit scan (wide digits)
  constexpr int kSmall = 1 << kSmallDigitBits;
  static_assert(kSmall == kThreads, "one small digit per thread");
  constexpr int kChunk = ITEMS < 8 ? ITEMS : 8;  // items ranked per sweep (small digits)
  constexpr int kWaves = kThreads / 64;
  constexpr int kWideWords = kMaxBuckets * (1 + kWaves);
  constexpr int kSmallWords = kChunk * kWaves * kSmall;
  __shared__ uint32_t lds[kWideWords > kSmallWords ? kWideWords : kSmallWords];
  __shared__ uint32_t s_tmp[kWaves];
  __shared__ uint8_t s_pos[12];
  const int nbits = min(hdr->digit[pass].nbits, kMaxDigitBits);  // never more buckets than the LDS holds
  if (nbits == 0) return;
  const int nb = 1 << nbits;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (threadIdx.x < 12) s_pos[threadIdx.x] = hdr->digit[pass].pos[threadIdx.x];
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
  if (nbits <= kSmallDigitBits) {
    // thread d owns digit d: run = its next position
    const int d_own = threadIdx.x;
    const uint32_t tot = d_own < nb ? totals[d_own] : 0u;
    uint32_t all;
    uint32_t run = block_exclusive_scan(tot, s_tmp, &all);  // also makes s_pos visible
    if (d_own < nb) run += offsets[int64_t(d_own) * gridDim.x + blockIdx.x];
    uint32_t(*cnt)[kWaves][kSmall] = reinterpret_cast<uint32_t(*)[kWaves][kSmall]>(lds);
#pragma unroll
    for (int c0 = 0; c0 < ITEMS; c0 += kChunk) {
      for (int q = threadIdx.x; q < kSmallWords; q += kThreads) lds[q] = 0u;
      __syncthreads();
      uint32_t dg[kChunk], rank[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        const int it = c0 + c;
        const bool valid = base + it * kThreads + threadIdx.x < n;
        const uint32_t d = valid ? digit_of(kv[it], s_pos, nbits) : 0u;
        unsigned long long peers = __ballot(valid);
        for (int j = 0; j < nbits; ++j) {
          const bool bit = (d >> j) & 1u;
          const unsigned long long bal = __ballot(bit);
          peers &= bit ? bal : ~bal;
        }
        dg[c] = d;
        rank[c] = valid ? __popcll(peers & lt) : ~0u;
        if (valid && (peers & lt) == 0) cnt[c][wave][d] = __popcll(peers);
      }
      __syncthreads();
      if (d_own < nb) {
#pragma unroll
        for (int c = 0; c < kChunk; ++c)
#pragma unroll
          for (int w = 0; w < kWaves; ++w) {
            const uint32_t v = cnt[c][w][d_own];
            cnt[c][w][d_own] = run;
            run += v;
          }
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        if (rank[c] != ~0u) {
          const uint32_t pos = cnt[c][wave][dg[c]] + rank[c];
          kout[pos] = kv[c0 + c];
          vout[pos] = vv[c0 + c];
        }
      }
      __syncthreads();  // the next chunk clears the counts
    }
    return;
  }
  uint32_t* base_off = lds;
  uint32_t(*wcount)[kMaxBuckets] = reinterpret_cast<uint32_t(*)[kMaxBuckets]>(lds + kMaxBuckets);
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
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    for (int d = threadIdx.x; d < nb; d += kThreads)
#pragma unroll
      for (int w = 0; w < kWaves; ++w) wcount[w][d] = 0;
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
      for (int w = 0; w < kWaves; ++w) add += wcount[w][dd];
      base_off[dd] += add;
    }
    __syncthreads();
  }
}

// The key bits beyond the passes' digits (only when more than kSortPasses *
// kMaxDigitBits bits vary): one workgroup sorts keys[0..n) stably by them, 8
// bits per pass, using tmp as the other buffer, and leaves the result in keys /
// rows.
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
// each 4x4x4 block) into part[workgroup] and flags adjacent equal keys
// (duplicate coordinates: equal keys are adjacent after the sort).
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

// Every workgroup adds up the block counts (nparts partials, from L2), derives
// the table capacity (power of two >= 2x the blocks, at least 16, at most
// max_cap) and hash shift, and clears its share of the slots; the first one
// records them in the header. (One atomic counter for the blocks, or a
// separate single-workgroup sizing kernel, each cost more at 0.4M voxels.)
__global__ __launch_bounds__(kThreads) void block_clear(BlockSlot* __restrict__ slots, uint32_t max_cap,
                                                        const uint32_t* __restrict__ part, int nparts,
                                                        HashHeader* hdr) {
  __shared__ uint32_t s_cnt[kThreads / 64];
  uint32_t c = 0;
  for (int i = threadIdx.x; i < nparts; i += kThreads) c += part[i];
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if ((threadIdx.x & 63) == 0) s_cnt[threadIdx.x >> 6] = c;
  __syncthreads();
  uint32_t nb = 0;
  for (int w = 0; w < kThreads / 64; ++w) nb += s_cnt[w];
  uint32_t cap = 16, lg = 4;
  while (cap < 2u * nb && cap < max_cap) {
    cap <<= 1;
    ++lg;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    hdr->nblocks = nb;
    hdr->cap_mask = cap - 1;
    hdr->shift = 64 - lg;
  }
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < cap; i += gridDim.x * kThreads) {
    uint4* p = reinterpret_cast<uint4*>(slots + i);
    p[0] = make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0u, 0u);
    p[1] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// The lane at each block head inserts {block key, occupancy bitmap, start}.
// The bitmap is a segmented OR over the lanes of the wave that hold the same
// block (sorted keys make a block one run of lanes). A block that runs past the
// wave's last lane continues in at most the next 63 keys: the wave loads those
// 64 keys in one coalesced load and ORs in the bits of the leading ones that
// belong to the same block.
__global__ __launch_bounds__(kThreads) void block_insert(const uint64_t* __restrict__ keys, int64_t n,
                                                         BlockSlot* __restrict__ slots, HashHeader* hdr) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = t - lane;
  if (wave0 >= n) return;  // whole wave past the end
  const bool valid = t < n;
  const uint64_t k = valid ? keys[t] : ~0ull;
  const uint64_t bkey = k >> 6;
  uint64_t prev = __shfl_up(k, 1, 64);
  if (lane == 0) prev = t > 0 ? keys[t - 1] : ~k;
  const bool head = valid && (t == 0 || (prev >> 6) != bkey);
  uint64_t bits = valid ? (1ull << (k & 63u)) : 0ull;
  for (int o = 1; o < 64; o <<= 1) {  // bits of lanes [lane, lane + 2o) of the same block
    const uint64_t ob = __shfl_down(bits, o, 64);
    const uint64_t okey = __shfl_down(bkey, o, 64);
    if (lane + o < 64 && okey == bkey) bits |= ob;
  }
  const uint64_t last_key = __shfl(bkey, 63, 64);
  uint64_t tail = 0;  // bits of the last lane's block in the next wave's keys
  if (wave0 + 64 < n) {  // wave-uniform: lane 63 is valid and keys follow
    const int64_t u = wave0 + 64 + lane;
    const bool uv = u < n;
    const uint64_t ku = uv ? keys[u] : 0ull;
    const unsigned long long other = __ballot(!uv || (ku >> 6) != last_key);
    const int run = other ? __ffsll(static_cast<long long>(other)) - 1 : 64;
    tail = wave_or(lane < run ? (1ull << (ku & 63u)) : 0ull);
  }
  if (!head) return;
  if (last_key == bkey) bits |= tail;
  const uint32_t mask = hdr->cap_mask, shift = hdr->shift;
  uint32_t s = home_slot(bkey, shift) & mask;
  for (uint32_t probe = 0; probe <= mask; ++probe) {
    unsigned long long* kp = reinterpret_cast<unsigned long long*>(&slots[s].bkey);
    const unsigned long long prev_key = atomicCAS(kp, kEmptyKey, bkey);
    if (prev_key == kEmptyKey) {
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


// ---------------------------------------------------------------------------
// Morton order from an occupancy bitmap, for voxels in a known grid (x, y, z <
// 2^g, object b < B). Cell c = (b << 3g) | the low 3g bits of the Morton key
// orders the cells as the keys do, so the sorted position of a voxel is the
// number of occupied cells before its own: a counting sort over the bitmap,
// with no radix passes. An aligned 64-cell word of the bitmap is one 4x4x4
// block (its six low Morton bits are the in-block cell), so the words are also
// the block table's occupancy bitmaps and the nonzero words its blocks.
// ---------------------------------------------------------------------------
// The bitmap is scanned in at most kThreads chunks of 2^lgc words (lgc >= 10:
// at least four words per thread), so that every workgroup of the two kernels
// after the scan can take the exclusive scan of the chunk totals itself, one
// value per thread.
constexpr int kDenseMinLgChunk = 10;

// Clears the bitmap and initialises the header (flags 0, empty-table capacity).
__global__ __launch_bounds__(kThreads) void dense_clear(uint4* __restrict__ bitmap16, int64_t n16, HashHeader* hdr) {
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n16; i += int64_t(gridDim.x) * kThreads)
    bitmap16[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    hdr->flags = 0u;
    hdr->nblocks = 0u;
    hdr->cap_mask = 15u;
    hdr->shift = 60u;
  }
}

// Sets each voxel's cell bit (a coordinate outside the grid sets the range flag
// and no bit). Lanes of a wave whose cells share a bitmap word -- runs of
// consecutive lanes, common when the rows come in raster or Morton order -- are
// merged first, and the first lane of each run sets the run's bits with one
// atomic that returns nothing. Duplicates are found from the count of set bits
// (dense_scatter): each voxel in the grid sets one bit, so the bitmap holds
// fewer bits than voxels exactly when two voxels share a cell.
__global__ __launch_bounds__(kThreads) void dense_mark(const int4* __restrict__ coords, int64_t n, int g,
                                                       uint32_t batch, unsigned long long* __restrict__ bitmap,
                                                       HashHeader* hdr) {
  const uint32_t lim = 1u << g;
  const uint64_t low = (uint64_t(1) << (3 * g)) - 1u;
  const int lane = threadIdx.x & 63;
  bool bad = false;
  for (int64_t i0 = int64_t(blockIdx.x) * kThreads; i0 < n; i0 += int64_t(gridDim.x) * kThreads) {
    const int64_t i = i0 + threadIdx.x;
    int64_t word = -1 - lane;  // distinct from every other lane's when the lane sets nothing
    unsigned long long bit = 0ull;
    if (i < n) {
      const int4 c = coords[i];
      if (uint32_t(c.x) >= batch || uint32_t(c.y) >= lim || uint32_t(c.z) >= lim || uint32_t(c.w) >= lim) {
        bad = true;
      } else {
        const uint64_t key = make_key(uint32_t(c.x), uint32_t(c.y), uint32_t(c.z), uint32_t(c.w));
        const uint64_t cell = (uint64_t(uint32_t(c.x)) << (3 * g)) | (key & low);
        word = int64_t(cell >> 6);
        bit = 1ull << (cell & 63u);
      }
    }
    for (int o = 1; o < 64; o <<= 1) {  // bits of lanes [lane, lane + 2o) with the same word
      const unsigned long long ob = __shfl_down(bit, o, 64);
      const int64_t ow = __shfl_down(word, o, 64);
      if (lane + o < 64 && ow == word) bit |= ob;
    }
    const int64_t prev = __shfl_up(word, 1, 64);
    if (word >= 0 && (lane == 0 || prev != word))
      __hip_atomic_fetch_or(&bitmap[word], bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0) atomicOr(&hdr->flags, kFlagCoordRange);
}

// Per chunk of 2^lgc words: each word's occupied cells before it within the
// chunk (wpre), the chunk's occupied cells (ctot) and nonzero words (cblk).
// Thread t takes 2^lgc / kThreads consecutive words.
__global__ __launch_bounds__(kThreads) void dense_scan(const unsigned long long* __restrict__ bitmap, int lgc,
                                                       uint32_t* __restrict__ wpre, uint32_t* __restrict__ ctot,
                                                       uint32_t* __restrict__ cblk) {
  __shared__ uint32_t s_tmp[kThreads / 64];
  const int per = (1 << lgc) / kThreads;  // a multiple of 4
  const int64_t w0 = (int64_t(blockIdx.x) << lgc) + int64_t(threadIdx.x) * per;
  uint32_t sum = 0, nz = 0;
  for (int q = 0; q < per; q += 2) {
    const ulonglong2 a = *reinterpret_cast<const ulonglong2*>(bitmap + w0 + q);
    sum += __popcll(a.x) + __popcll(a.y);
    nz += uint32_t(a.x != 0ull) + uint32_t(a.y != 0ull);
  }
  uint32_t tot, nzt;
  uint32_t ex = block_exclusive_scan(sum, s_tmp, &tot);
  block_exclusive_scan(nz, s_tmp, &nzt);
  for (int q = 0; q < per; q += 4) {
    const ulonglong2 a = *reinterpret_cast<const ulonglong2*>(bitmap + w0 + q);
    const ulonglong2 b = *reinterpret_cast<const ulonglong2*>(bitmap + w0 + q + 2);
    const uint32_t p0 = __popcll(a.x), p1 = __popcll(a.y), p2 = __popcll(b.x), p3 = __popcll(b.y);
    *reinterpret_cast<uint4*>(wpre + w0 + q) = make_uint4(ex, ex + p0, ex + p0 + p1, ex + p0 + p1 + p2);
    ex += p0 + p1 + p2 + p3;
  }
  if (threadIdx.x == 0) {
    ctot[blockIdx.x] = tot;
    cblk[blockIdx.x] = nzt;
  }
}

// Exclusive scan of the chunk totals into s_pre (nchunks <= kThreads) and the
// number of nonzero words; every workgroup of the next two kernels does it.
__device__ uint32_t dense_chunk_prefix(const uint32_t* __restrict__ ctot, const uint32_t* __restrict__ cblk,
                                       int nchunks, uint32_t* s_pre, uint32_t* s_tmp, uint32_t* bits_set = nullptr) {
  const int c = threadIdx.x;
  const uint32_t v = c < nchunks ? ctot[c] : 0u, nz = c < nchunks ? cblk[c] : 0u;
  uint32_t tot, nzt;
  s_pre[c] = block_exclusive_scan(v, s_tmp, &tot);
  block_exclusive_scan(nz, s_tmp, &nzt);
  __syncthreads();
  if (bits_set != nullptr) *bits_set = tot;
  return nzt;
}

// Sorted keys and rows: voxel i goes to the occupied cells before its own.
// The same workgroups also size the block table from the nonzero words
// (capacity: power of two >= 2x the blocks, at least 16, at most max_cap) and
// clear it; the first one records the capacity.
__global__ __launch_bounds__(kThreads) void dense_scatter(const int4* __restrict__ coords, int64_t n, int g,
                                                          uint32_t batch, const unsigned long long* __restrict__ bitmap,
                                                          int lgc, const uint32_t* __restrict__ wpre,
                                                          const uint32_t* __restrict__ ctot,
                                                          const uint32_t* __restrict__ cblk, int nchunks,
                                                          uint32_t* __restrict__ cpre, uint64_t* __restrict__ skeys,
                                                          int32_t* __restrict__ srows, BlockSlot* __restrict__ slots,
                                                          uint32_t max_cap, HashHeader* hdr) {
  __shared__ uint32_t s_pre[kThreads];
  __shared__ uint32_t s_tmp[kThreads / 64];
  uint32_t nset;
  const uint32_t nb = dense_chunk_prefix(ctot, cblk, nchunks, s_pre, s_tmp, &nset);
  uint32_t cap = 16, lg = 4;
  while (cap < 2u * nb && cap < max_cap) {
    cap <<= 1;
    ++lg;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    hdr->nblocks = nb;
    hdr->cap_mask = cap - 1;
    hdr->shift = 64 - lg;
    // fewer bits than voxels: two voxels share a cell (or some voxel lies
    // outside the grid, which the range flag reports first)
    if (int64_t(nset) != n) atomicOr(&hdr->flags, kFlagDuplicate);
  }
  if (blockIdx.x == 0 && int(threadIdx.x) < nchunks) cpre[threadIdx.x] = s_pre[threadIdx.x];
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < cap; i += gridDim.x * kThreads) {
    uint4* q = reinterpret_cast<uint4*>(slots + i);
    q[0] = make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0u, 0u);
    q[1] = make_uint4(0u, 0u, 0u, 0u);
  }
  const uint32_t lim = 1u << g;
  const uint64_t low = (uint64_t(1) << (3 * g)) - 1u;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n; i += int64_t(gridDim.x) * kThreads) {
    const int4 c = coords[i];
    if (uint32_t(c.x) >= batch || uint32_t(c.y) >= lim || uint32_t(c.z) >= lim || uint32_t(c.w) >= lim)
      continue;  // outside the grid: flagged by dense_mark
    const uint64_t key = make_key(uint32_t(c.x), uint32_t(c.y), uint32_t(c.z), uint32_t(c.w));
    const uint64_t cell = (uint64_t(uint32_t(c.x)) << (3 * g)) | (key & low);
    const int64_t w = int64_t(cell >> 6);
    const uint32_t below = __popcll(bitmap[w] & ((1ull << (cell & 63u)) - 1ull));
    const uint32_t pos = s_pre[w >> lgc] + wpre[w] + below;
    skeys[pos] = key;
    srows[pos] = int32_t(i);
  }
}

// One thread per bitmap word: a nonzero word is a block; insert {block key,
// bitmap, first sorted position}. Block key = key >> 6 = (b << 42) | (the
// word's Morton bits).
__global__ __launch_bounds__(kThreads) void dense_insert(const unsigned long long* __restrict__ bitmap, int lgc,
                                                         const uint32_t* __restrict__ wpre,
                                                         const uint32_t* __restrict__ ctot,
                                                         const uint32_t* __restrict__ cblk, int nchunks, int g,
                                                         BlockSlot* __restrict__ slots, HashHeader* hdr) {
  __shared__ uint32_t s_pre[kThreads];
  __shared__ uint32_t s_tmp[kThreads / 64];
  dense_chunk_prefix(ctot, cblk, nchunks, s_pre, s_tmp);
  const uint32_t mask = hdr->cap_mask, shift = hdr->shift;
  const int wb = 3 * g - 6;  // Morton bits of a block index
  const int64_t nwords = int64_t(nchunks) << lgc;
  for (int64_t w = int64_t(blockIdx.x) * kThreads + threadIdx.x; w < nwords; w += int64_t(gridDim.x) * kThreads) {
    const unsigned long long bits = bitmap[w];
    if (bits == 0ull) continue;
    const uint64_t bkey = (uint64_t(w >> wb) << 42) | uint64_t(w & ((int64_t(1) << wb) - 1));
    const uint32_t start = s_pre[w >> lgc] + wpre[w];
    uint32_t s = home_slot(bkey, shift) & mask;
    bool placed = false;
    for (uint32_t probe = 0; probe <= mask; ++probe) {
      unsigned long long* kp = reinterpret_cast<unsigned long long*>(&slots[s].bkey);
      if (atomicCAS(kp, kEmptyKey, bkey) == kEmptyKey) {
        slots[s].bits = bits;
        slots[s].start = start;
        placed = true;
        break;
      }
      s = (s + 1) & mask;
    }
    if (!placed) atomicOr(&hdr->flags, kFlagCapacity);
  }
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

hipError_t launch_pack(const int32_t* coords, int64_t n, uint32_t lim, uint32_t blim, uint64_t* keys, int32_t* rows,
                       uint64_t* keys2, int32_t* rows2, unsigned long long* part, HashHeader* hdr, hipStream_t st) {
  if (n > 0)  // the first histogram pass of the sort builds the header
    pack_keys<<<int(pack_partials(n)), kThreads, 0, st>>>(reinterpret_cast<const int4*>(coords), n, lim, blim, keys,
                                                          rows, keys2, rows2, part);
  else
    reduce_bits<<<1, kThreads, 0, st>>>(part, 0, hdr);
  return hipGetLastError();
}

hipError_t launch_sort(uint64_t* keys0, int32_t* rows0, uint64_t* keys1, int32_t* rows1, int64_t n,
                       HashHeader* hdr, const unsigned long long* part, uint32_t* counts, uint32_t* totals,
                       hipStream_t st) {
  const int nparts = int(pack_partials(n));
  const int64_t nb = sort_blocks(n);
  uint64_t* k[2] = {keys0, keys1};
  int32_t* r[2] = {rows0, rows1};
  const int items = sort_items(n);
  for (int pass = 0; pass < kSortPasses; ++pass) {
    const int a = (pass + 1) & 1;  // 1 -> 0 -> 1 -> 0 -> 1: the last pass writes keys1
    switch (items) {
#define TRSC_RADIX_PASS(IT)                                                                                   \
  case IT:                                                                                                    \
    radix_hist<IT><<<unsigned(nb), kThreads, 0, st>>>(k[a], n, hdr, pass, counts, part, nparts);              \
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
  const int nb = n > 0 ? int(pack_partials(n)) : 0;
  if (n > 0) block_count<<<nb, kThreads, 0, st>>>(keys, n, part, hdr);
  const uint32_t cb = (max_cap + kThreads - 1) / kThreads;
  block_clear<<<cb < 2048u ? cb : 2048u, kThreads, 0, st>>>(slots, max_cap, part, nb, hdr);
  if (n > 0) block_insert<<<grid_for(n, kThreads), kThreads, 0, st>>>(keys, n, slots, hdr);
  return hipGetLastError();
}

int dense_max_chunks() { return kThreads; }
int dense_chunk_log2(int64_t words) {
  int lgc = kDenseMinLgChunk;
  while ((words + (int64_t(1) << lgc) - 1) >> lgc > kThreads) ++lgc;
  return lgc;
}

hipError_t launch_dense_hash(const int32_t* coords, int64_t n, int g, int batch, unsigned long long* bitmap,
                             int lgc, int nchunks, uint32_t* wpre, uint32_t* ctot, uint32_t* cblk, uint32_t* cpre,
                             uint64_t* skeys, int32_t* srows, BlockSlot* slots, uint32_t max_cap, HashHeader* hdr,
                             hipStream_t st) {
  const int64_t words = int64_t(nchunks) << lgc;
  const int64_t n16 = words / 2;
  const int64_t cb = (n16 + kThreads - 1) / kThreads;
  dense_clear<<<unsigned(cb < 4096 ? cb : 4096), kThreads, 0, st>>>(reinterpret_cast<uint4*>(bitmap), n16, hdr);
  const int64_t vb = (n + kThreads - 1) / kThreads;
  const unsigned vgrid = unsigned(vb < 4096 ? (vb > 0 ? vb : 1) : 4096);
  const auto* c4 = reinterpret_cast<const int4*>(coords);
  dense_mark<<<vgrid, kThreads, 0, st>>>(c4, n, g, uint32_t(batch), bitmap, hdr);
  dense_scan<<<unsigned(nchunks), kThreads, 0, st>>>(bitmap, lgc, wpre, ctot, cblk);
  const int64_t sb = (int64_t(max_cap) + kThreads - 1) / kThreads;
  const unsigned sgrid = unsigned(vb > sb ? (vb < 2048 ? vb : 2048) : (sb < 2048 ? sb : 2048));
  dense_scatter<<<sgrid, kThreads, 0, st>>>(c4, n, g, uint32_t(batch), bitmap, lgc, wpre, ctot, cblk, nchunks, cpre,
                                            skeys, srows, slots, max_cap, hdr);
  const int64_t wgrid = (words + kThreads - 1) / kThreads;
  dense_insert<<<unsigned(wgrid < 4096 ? wgrid : 4096), kThreads, 0, st>>>(bitmap, lgc, wpre, ctot, cblk, nchunks,
                                                                          g, slots, hdr);
  return hipGetLastError();
}

hipError_t launch_lookup(const TableRef& t, const int32_t* q, int64_t nq, int32_t* out, hipStream_t st) {
  if (nq > 0)
    table_lookup<<<grid_for(nq, kThreads), kThreads, 0, st>>>(t, reinterpret_cast<const int4*>(q), nq, out);
  return hipGetLastError();
}

}  // namespace trsc
