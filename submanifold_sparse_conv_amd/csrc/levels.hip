// Moving between resolution levels. The pages build one neighbour table per
// resolution level ("Porting TRELLIS.2 From Python to Rust and Metal", section
// V) and change level in their decoders by pixel-shuffle / Channel2Spatial
// upsampling driven by subdivision predictions (TRELLIS.2 MLX port README,
// repository tree and pipeline list). Conventions: the parent of (b, x, y, z)
// is (b, x >> 1, y >> 1, z >> 1); child o = 4 dx + 2 dy + dz of (b, x, y, z) is
// (b, 2x + dx, 2y + dy, 2z + dz); a parent row of 8C channels holds channel c of
// child o at c * 8 + o.
//
// Parent level. In the Morton key (x above y above z in every bit triple) the
// low three bits are exactly (x & 1, y & 1, z & 1) = the octant, and the key
// of the parent is the key shifted right by three. The hash's sorted keys are
// therefore already grouped by parent in parent Morton order: the parent level
// is the runs of equal key >> 3, found with a flag / scan / write pass and no
// new sort. The first position of a run writes the parent's coordinates and
// its whole 8-entry children row (a run has at most 8 positions).
//
// Finer level. Row i keeps the children named by the bits of keep[i]; fine
// rows follow (row, octant) order: an exclusive scan of the popcounts.
#include "common.h"
#include "launch.h"

namespace trsc {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = 4;                        // items per thread
constexpr int kBlockItems = kThreads * kPer;   // 1024

// Inclusive scan of v over the workgroup (256 threads); returns the total in *total.
__device__ int64_t block_scan(int64_t v, int64_t* sh, int64_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int w = 0; w < kThreads / 64; ++w) {
    if (w < wave) before += sh[w];
    all += sh[w];
  }
  __syncthreads();
  *total = all;
  return v + before;
}

__device__ inline uint64_t parent_of(uint64_t key) {
  return (key & ~((uint64_t(1) << 48) - 1)) | ((key & ((uint64_t(1) << 48) - 1)) >> 3);
}

__device__ inline bool is_head(const uint64_t* skeys, int64_t pos) {
  return pos == 0 || parent_of(skeys[pos]) != parent_of(skeys[pos - 1]);
}

// Per-block counts of the items a block produces.
__global__ __launch_bounds__(kThreads) void ds_count(const uint64_t* __restrict__ skeys, int64_t n,
                                                     int64_t* __restrict__ part) {
  __shared__ int64_t sh[kThreads / 64];
  const int64_t b0 = int64_t(blockIdx.x) * kBlockItems;
  int64_t c = 0;
  for (int q = 0; q < kPer; ++q) {
    const int64_t pos = b0 + q * kThreads + threadIdx.x;
    if (pos < n && is_head(skeys, pos)) ++c;
  }
  int64_t total;
  block_scan(c, sh, &total);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

__device__ inline int popc8(const uint8_t* keep, int64_t i) { return keep ? __popc(unsigned(keep[i])) : 8; }

__global__ __launch_bounds__(kThreads) void sd_count(const int32_t* __restrict__ coords, const uint8_t* keep,
                                                     int64_t n, int64_t* __restrict__ part,
                                                     uint32_t* __restrict__ flags) {
  __shared__ int64_t sh[kThreads / 64];
  const int64_t b0 = int64_t(blockIdx.x) * kBlockItems;
  int64_t c = 0;
  bool bad = false;
  for (int q = 0; q < kPer; ++q) {
    const int64_t i = b0 + q * kThreads + threadIdx.x;
    if (i >= n) continue;
    const int4 p = reinterpret_cast<const int4*>(coords)[i];
    bad |= p.x < 0 || p.x > 65535 || p.y < 0 || p.y > 32767 || p.z < 0 || p.z > 32767 || p.w < 0 || p.w > 32767;
    c += popc8(keep, i);
  }
  if (bad) atomicOr(flags, kFlagCoordRange);
  int64_t total;
  block_scan(c, sh, &total);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

// Exclusive scan of part[0..nb) in place, total into *total. One workgroup.
__global__ __launch_bounds__(kThreads) void scan_parts(int64_t* __restrict__ part, int64_t nb,
                                                       int64_t* __restrict__ total) {
  __shared__ int64_t sh[kThreads / 64];
  int64_t carry = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += kThreads) {
    const int64_t b = b0 + threadIdx.x;
    const int64_t v = b < nb ? part[b] : 0;
    int64_t t;
    const int64_t inc = block_scan(v, sh, &t);
    if (b < nb) part[b] = carry + inc - v;
    carry += t;
  }
  if (threadIdx.x == 0) *total = carry;
}

__global__ __launch_bounds__(kThreads) void ds_write(const uint64_t* __restrict__ skeys,
                                                     const int32_t* __restrict__ srows, int64_t n,
                                                     const int64_t* __restrict__ part, int64_t cap,
                                                     int32_t* __restrict__ coarse, int32_t* __restrict__ children) {
  __shared__ int64_t sh[kThreads / 64];
  const int64_t b0 = int64_t(blockIdx.x) * kBlockItems;
  // thread t owns positions b0 + t*kPer .. +kPer (contiguous, so the scan is in position order)
  bool head[kPer];
  int64_t c = 0;
  for (int q = 0; q < kPer; ++q) {
    const int64_t pos = b0 + int64_t(threadIdx.x) * kPer + q;
    head[q] = pos < n && is_head(skeys, pos);
    c += head[q];
  }
  int64_t total;
  int64_t qi = part[blockIdx.x] + block_scan(c, sh, &total) - c;  // parent index of this thread's first head
  for (int q = 0; q < kPer; ++q) {
    if (!head[q]) continue;
    const int64_t pos = b0 + int64_t(threadIdx.x) * kPer + q;
    if (qi < cap) {
      const uint64_t pk = parent_of(skeys[pos]);
      const uint64_t m = pk & ((uint64_t(1) << 48) - 1);
      reinterpret_cast<int4*>(coarse)[qi] =
          make_int4(int(pk >> 48), int(compact3(m >> 2)), int(compact3(m >> 1)), int(compact3(m)));
      int32_t row[8] = {-1, -1, -1, -1, -1, -1, -1, -1};
      for (int64_t r = pos; r < n && r < pos + 8 && parent_of(skeys[r]) == pk; ++r)
        row[skeys[r] & 7] = srows[r];
      int4* dst = reinterpret_cast<int4*>(children + qi * 8);
      dst[0] = make_int4(row[0], row[1], row[2], row[3]);
      dst[1] = make_int4(row[4], row[5], row[6], row[7]);
    }
    ++qi;
  }
}

__global__ __launch_bounds__(kThreads) void sd_write(const int32_t* __restrict__ coords, const uint8_t* keep,
                                                     int64_t n, const int64_t* __restrict__ part, int64_t cap,
                                                     int32_t* __restrict__ fine, int32_t* __restrict__ children) {
  __shared__ int64_t sh[kThreads / 64];
  const int64_t b0 = int64_t(blockIdx.x) * kBlockItems;
  int64_t c = 0;
  for (int q = 0; q < kPer; ++q) {
    const int64_t i = b0 + int64_t(threadIdx.x) * kPer + q;
    if (i < n) c += popc8(keep, i);
  }
  int64_t total;
  int64_t f = part[blockIdx.x] + block_scan(c, sh, &total) - c;
  for (int q = 0; q < kPer; ++q) {
    const int64_t i = b0 + int64_t(threadIdx.x) * kPer + q;
    if (i >= n) break;
    const int4 p = reinterpret_cast<const int4*>(coords)[i];
    const unsigned bits = keep ? unsigned(keep[i]) : 0xFFu;
    int32_t row[8];
    for (int o = 0; o < 8; ++o) {
      if (!((bits >> o) & 1u)) {
        row[o] = -1;
        continue;
      }
      row[o] = f < cap ? int32_t(f) : -1;
      if (f < cap)
        reinterpret_cast<int4*>(fine)[f] =
            make_int4(p.x, 2 * p.y + ((o >> 2) & 1), 2 * p.z + ((o >> 1) & 1), 2 * p.w + (o & 1));
      ++f;
    }
    int4* dst = reinterpret_cast<int4*>(children + i * 8);
    dst[0] = make_int4(row[0], row[1], row[2], row[3]);
    dst[1] = make_int4(row[4], row[5], row[6], row[7]);
  }
}

// Channel2Spatial / Spatial2Channel for 16-byte groups: V channels of the fine
// rows (V = 16 / sizeof(T)) against the 8V contiguous parent elements
// c * 8 + o, c in the group. Each thread moves one group of one parent and
// transposes V x 8 elements in registers.
template <typename T, bool kToFine>
__global__ __launch_bounds__(kThreads) void regroup(const int32_t* __restrict__ children, int64_t n_coarse,
                                                    T* __restrict__ xc, T* __restrict__ xf, int c_fine) {
  constexpr int V = 16 / sizeof(T);
  const int groups = c_fine / V;
  const int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= n_coarse * groups) return;
  const int64_t q = e / groups;
  const int g = int(e - q * groups);
  const int4 ca = reinterpret_cast<const int4*>(children)[2 * q];
  const int4 cb = reinterpret_cast<const int4*>(children)[2 * q + 1];
  const int32_t ch[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
  uint4* pc = reinterpret_cast<uint4*>(xc + q * 8 * c_fine + int64_t(g) * V * 8);  // 8V elements, 8 uint4
  if constexpr (kToFine) {
    alignas(16) T in[V * 8];
#pragma unroll
    for (int u = 0; u < 8; ++u) reinterpret_cast<uint4*>(in)[u] = pc[u];
#pragma unroll
    for (int o = 0; o < 8; ++o) {
      if (ch[o] < 0) continue;
      alignas(16) T out[V];
#pragma unroll
      for (int c = 0; c < V; ++c) out[c] = in[c * 8 + o];
      *reinterpret_cast<uint4*>(xf + int64_t(ch[o]) * c_fine + g * V) = *reinterpret_cast<const uint4*>(out);
    }
  } else {
    alignas(16) T in[8][V];
#pragma unroll
    for (int o = 0; o < 8; ++o) {
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(in[o]) =
          ch[o] >= 0 ? *reinterpret_cast<const uint4*>(xf + int64_t(ch[o]) * c_fine + g * V) : z;
    }
    alignas(16) T out[V * 8];
#pragma unroll
    for (int c = 0; c < V; ++c)
#pragma unroll
      for (int o = 0; o < 8; ++o) out[c * 8 + o] = in[o][c];
#pragma unroll
    for (int u = 0; u < 8; ++u) pc[u] = reinterpret_cast<const uint4*>(out)[u];
  }
}

}  // namespace

int64_t level_blocks(int64_t n) { return (n + kBlockItems - 1) / kBlockItems; }

hipError_t launch_downsample(const uint64_t* skeys, const int32_t* srows, int64_t n, int64_t cap, int64_t* part,
                             int64_t* total, int32_t* coarse, int32_t* children, hipStream_t st) {
  const int64_t nb = level_blocks(n);
  if (nb > 0) ds_count<<<unsigned(nb), kThreads, 0, st>>>(skeys, n, part);
  scan_parts<<<1, kThreads, 0, st>>>(part, nb, total);
  if (nb > 0) ds_write<<<unsigned(nb), kThreads, 0, st>>>(skeys, srows, n, part, cap, coarse, children);
  return hipGetLastError();
}

hipError_t launch_subdivide(const int32_t* coords, const uint8_t* keep, int64_t n, int64_t cap, int64_t* part,
                            int64_t* total, uint32_t* flags, int32_t* fine, int32_t* children, hipStream_t st) {
  const int64_t nb = level_blocks(n);
  if (nb > 0) sd_count<<<unsigned(nb), kThreads, 0, st>>>(coords, keep, n, part, flags);
  scan_parts<<<1, kThreads, 0, st>>>(part, nb, total);
  if (nb > 0) sd_write<<<unsigned(nb), kThreads, 0, st>>>(coords, keep, n, part, cap, fine, children);
  return hipGetLastError();
}

// The same moves through an LDS tile of whole parent rows (kTileBytes), so that
// both sides of the move are read and written in contiguous 16-byte pieces
// across the lanes: the parent rows as one contiguous block, each child row
// as consecutive pieces. A parent row holds 8C elements, element c * 8 + o at
// 16-byte piece (c * 8 + o) * sizeof(T) / 16; pieces are stored XOR-swizzled
// within each 128-byte run (piece p at p ^ ((p >> 3) & 7)) so that the lanes
// of one LDS access, which step through the channel groups of a child row,
// fall on different banks.
constexpr int kTileBytes = 16384;

__device__ inline int swz_piece(int p) { return p ^ ((p >> 3) & 7); }

template <typename T, bool kToFine>
__global__ __launch_bounds__(kThreads) void regroup_tile(const int32_t* __restrict__ children, int64_t n_coarse,
                                                         T* __restrict__ xc, T* __restrict__ xf, int c_fine,
                                                         int per_wg) {
  constexpr int E = int(sizeof(T)), V = 16 / E;
  __shared__ __attribute__((aligned(16))) unsigned char tile[kTileBytes];
  const int row_pieces = c_fine * 8 * E / 16;   // 16-byte pieces per parent row
  const int groups = c_fine / V;                // 16-byte pieces per child row
  const int64_t q0 = int64_t(blockIdx.x) * per_wg;
  const int np = int(n_coarse - q0 < per_wg ? n_coarse - q0 : per_wg);
  const int pieces = np * row_pieces;
  uint4* const tp = reinterpret_cast<uint4*>(tile);
  uint4* const gc = reinterpret_cast<uint4*>(xc + q0 * 8 * c_fine);
  auto elem_at = [&](int q, int c, int o) -> T* {  // element c * 8 + o of parent row q in the tile
    const int byte = (c * 8 + o) * E;
    return reinterpret_cast<T*>(tile + (q * row_pieces + swz_piece(byte >> 4)) * 16 + (byte & 15));
  };
  // swz_piece only permutes pieces within aligned runs of 8, and a parent row is a whole
  // number of such runs (c_fine * 8 * E / 16 = c_fine * E / 2 with V | c_fine), so every
  // row's pieces stay inside its own slot of the tile.
  if constexpr (kToFine) {
    for (int p = threadIdx.x; p < pieces; p += kThreads) {
      const int q = p / row_pieces, k = p - q * row_pieces;
      tp[q * row_pieces + swz_piece(k)] = gc[p];
    }
    __syncthreads();
    for (int t = threadIdx.x; t < np * 8 * groups; t += kThreads) {
      const int g = t % groups, qo = t / groups, o = qo & 7, q = qo >> 3;
      const int32_t child = children[(q0 + q) * 8 + o];
      if (child < 0) continue;
      alignas(16) T out[V];
#pragma unroll
      for (int c = 0; c < V; ++c) out[c] = *elem_at(q, g * V + c, o);
      *reinterpret_cast<uint4*>(xf + int64_t(child) * c_fine + g * V) = *reinterpret_cast<const uint4*>(out);
    }
  } else {
    for (int t = threadIdx.x; t < np * 8 * groups; t += kThreads) {
      const int g = t % groups, qo = t / groups, o = qo & 7, q = qo >> 3;
      const int32_t child = children[(q0 + q) * 8 + o];
      alignas(16) T in[V];
      *reinterpret_cast<uint4*>(in) = child >= 0
                                          ? *reinterpret_cast<const uint4*>(xf + int64_t(child) * c_fine + g * V)
                                          : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int c = 0; c < V; ++c) *elem_at(q, g * V + c, o) = in[c];
    }
    __syncthreads();
    for (int p = threadIdx.x; p < pieces; p += kThreads) {
      const int q = p / row_pieces, k = p - q * row_pieces;
      gc[p] = tp[q * row_pieces + swz_piece(k)];
    }
  }
}

hipError_t launch_regroup(const int32_t* children, int64_t n_coarse, void* xc, void* xf, int c_fine, int elem_bytes,
                          bool to_fine, hipStream_t st) {
  const int64_t items = n_coarse * (c_fine / (16 / elem_bytes));
  if (items == 0) return hipSuccess;
  const int64_t row_bytes = int64_t(c_fine) * 8 * elem_bytes;
  if (row_bytes <= kTileBytes && row_bytes % 128 == 0) {  // whole parent rows fit the tile
    const int per_wg = int(kTileBytes / row_bytes);
    const int64_t g = (n_coarse + per_wg - 1) / per_wg;
    if (g > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (elem_bytes == 2) {
      if (to_fine)
        regroup_tile<uint16_t, true><<<unsigned(g), kThreads, 0, st>>>(
            children, n_coarse, static_cast<uint16_t*>(xc), static_cast<uint16_t*>(xf), c_fine, per_wg);
      else
        regroup_tile<uint16_t, false><<<unsigned(g), kThreads, 0, st>>>(
            children, n_coarse, static_cast<uint16_t*>(xc), static_cast<uint16_t*>(xf), c_fine, per_wg);
    } else {
      if (to_fine)
        regroup_tile<float, true><<<unsigned(g), kThreads, 0, st>>>(
            children, n_coarse, static_cast<float*>(xc), static_cast<float*>(xf), c_fine, per_wg);
      else
        regroup_tile<float, false><<<unsigned(g), kThreads, 0, st>>>(
            children, n_coarse, static_cast<float*>(xc), static_cast<float*>(xf), c_fine, per_wg);
    }
    return hipGetLastError();
  }
  const unsigned grid = unsigned((items + kThreads - 1) / kThreads);
  if (elem_bytes == 2) {
    if (to_fine)
      regroup<uint16_t, true><<<grid, kThreads, 0, st>>>(children, n_coarse, static_cast<uint16_t*>(xc),
                                                          static_cast<uint16_t*>(xf), c_fine);
    else
      regroup<uint16_t, false><<<grid, kThreads, 0, st>>>(children, n_coarse, static_cast<uint16_t*>(xc),
                                                           static_cast<uint16_t*>(xf), c_fine);
  } else {
    if (to_fine)
      regroup<float, true><<<grid, kThreads, 0, st>>>(children, n_coarse, static_cast<float*>(xc),
                                                       static_cast<float*>(xf), c_fine);
    else
      regroup<float, false><<<grid, kThreads, 0, st>>>(children, n_coarse, static_cast<float*>(xc),
                                                        static_cast<float*>(xf), c_fine);
  }
  return hipGetLastError();
}

}  // namespace trsc
