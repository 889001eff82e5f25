// Host-side launchers of the library's kernels (internal).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"
#include "tr_sparseconv.h"

namespace trsc {

int64_t sort_blocks(int64_t n);    // radix-sort workgroups (tiles) for n keys
int64_t pack_partials(int64_t n);  // partial triples (OR, AND, range flag) of the packing pass
constexpr int kSortBuckets = 1 << kMaxDigitBits;
// Packs keys / rows (into both sort buffers) and the partials (OR, AND, range
// flag) from which the sort's first histogram pass builds the header (flags,
// digits of the sort); for n = 0 it writes the header itself.
// Spatial components must be < lim and object indices < blim (65536 each
// without a grid).
hipError_t launch_pack(const int32_t* coords, int64_t n, uint32_t lim, uint32_t blim, uint64_t* keys, int32_t* rows,
                       uint64_t* keys2, int32_t* rows2, unsigned long long* part, HashHeader* hdr, hipStream_t st);
// kSortPasses LSD radix passes (digits from the header; the leading ones may be
// empty) keys1 -> keys0 -> keys1 -> keys0 -> keys1, then the single-workgroup
// pass over any further bits: the sorted keys and rows end in keys1 / rows1.
// counts: sort_blocks(n) * kSortBuckets words.
hipError_t launch_sort(uint64_t* keys0, int32_t* rows0, uint64_t* keys1, int32_t* rows1, int64_t n,
                       HashHeader* hdr, const unsigned long long* part, uint32_t* counts, uint32_t* totals,
                       hipStream_t st);
hipError_t launch_blocks(const uint64_t* keys, int64_t n, BlockSlot* slots, uint32_t max_cap,
                         uint32_t* part, HashHeader* hdr, hipStream_t st);
hipError_t launch_lookup(const TableRef& t, const int32_t* q, int64_t nq, int32_t* out, hipStream_t st);
// Morton sort and block table of voxels in a known grid (x, y, z < 2^g, object
// < batch) from an occupancy bitmap of nchunks chunks of 2^lgc 64-bit words
// (cells (b << 3g) | low 3g Morton bits; lgc = dense_chunk_log2(words), which
// keeps nchunks <= dense_max_chunks()); wpre: one word per bitmap word; ctot,
// cblk, cpre (the chunks' first positions, written for the kernel map): one
// word per chunk.
int dense_max_chunks();
int dense_chunk_log2(int64_t words);
hipError_t launch_dense_hash(const int32_t* coords, int64_t n, int g, int batch, unsigned long long* bitmap,
                             int lgc, int nchunks, uint32_t* wpre, uint32_t* ctot, uint32_t* cblk, uint32_t* cpre,
                             uint64_t* skeys, int32_t* srows, BlockSlot* slots, uint32_t max_cap, HashHeader* hdr,
                             hipStream_t st);

// Kernel map (nbr, caller order; mask, Morton order) and the gather-GEMM row
// order: grows / gmask = Morton order regrouped inside each kHaloTM-voxel tile
// by the octant pattern of the neighbour mask (the halo plan's tile order).

// Halo plan of the gather-GEMM over tiles of kHaloTM Morton-consecutive voxels:
// per tile, the rows in tile order (octant-regrouped inside the tile), the
// tile's distinct neighbour rows ("halo", numbered from slot 1; slot 0 stands
// for an absent neighbour) and the slot of every (row, tap). One record of
// kPlanBytes per tile, sections 1 KB-aligned:
//   [kPlanHdr]   HaloHeader
//   [kPlanRows]  int32 caller row of halo slot s (s = 1 .. nh), kHaloCap entries
//   [kPlanCrow]  int32 caller row at tile position r (-1 past the end)
//   [kPlanMask]  uint32 27-bit neighbour mask at tile position r
//   [kPlanSlots] uint16 LDS byte offset, in the gather-GEMM's halo of
//                kHaloRowBytes-byte rows, of the row of (tap k, position r) --
//                slot s * kHaloRowBytes + (((s >> 2) & 3) << 4) -- at
//                k * kHaloTM + sidx(r), sidx(r) = 128 (r / 128) + 4 (r % 32) +
//                (r / 32) % 4: a lane's four 32-row blocks at one tap are adjacent
constexpr int kHaloTM = 256;
constexpr int kHaloCap = 736;     // halo slots of one tile, slot 0 included
constexpr int kHaloHashBits = 12;
constexpr int kHaloHash = 1 << kHaloHashBits;  // dedup table entries
constexpr int kHaloProbes = 64;   // a longer probe run marks the tile as not fitting
constexpr int kHaloRowBytes = 64; // halo rows in LDS: 32 half-precision channels
static_assert(kHaloCap * kHaloRowBytes + 48 < 65536, "halo offsets fit in 16 bits");
constexpr int kPlanHdr = 0, kPlanRows = 1024, kPlanCrow = 4096, kPlanMask = 5120, kPlanSlots = 6144;
constexpr int kPlanSlotBytes = 27 * kHaloTM * 2;  // 13,824
constexpr int kPlanBytes = kPlanSlots + 14336;    // slots padded to whole kilobytes
static_assert(kPlanRows + kHaloCap * 4 <= kPlanCrow && kPlanSlotBytes <= 14336, "plan record layout");
struct HaloHeader {
  int32_t nh;         // halo rows (slots 1 .. nh); -1: the halo does not fit, gather from global memory
  uint32_t tmask;     // taps some row of the tile has
  uint16_t fm[27];    // bit b: 32-row block b (rows 32b .. 32b + 31) has tap k
};
inline int64_t halo_tiles(int64_t n) { return (n + kHaloTM - 1) / kHaloTM; }
// A tile's work estimate (written by the plan, one uint16 per tile): the
// (32-row block, tap) pairs that multiply, three times that when nh < 0.
constexpr int kHaloMaxCost = 3 * 27 * (kHaloTM / 32);
// The tiles in the gather-GEMM's launch order: decreasing cost (ties in tile
// order), so that the hardware's in-order dispatch of workgroups to free slots
// runs the longest tiles first and the shortest fill the end.
hipError_t launch_halo_order(const uint16_t* costs, int64_t tiles, int32_t* order, hipStream_t st);

// dense: the hash's occupancy bitmap when it was built in a known grid (the
// block records are read from it instead of the table), else null. plan:
// halo_tiles(n) records of kPlanBytes.
hipError_t launch_kmap(const uint64_t* skeys, int64_t n, const TableRef& t, const DenseRef* dense, int32_t* nbr,
                       uint32_t* mask, int32_t* grows, uint32_t* gmask, unsigned char* plan, uint16_t* costs,
                       int32_t* order, hipStream_t st);

// Forward kernels. `srows` is the row order of the tiles (position -> caller
// row), `mask` the 27-bit neighbour mask of the voxel at each position.
struct Epilogue {
  const float* bias;     // [c_out] or null
  const void* residual;  // [n, c_out] in the output type, or null
  int act;               // kAct*
};
struct ConvArgs {
  const int32_t* nbr;   // [n, 27] caller order
  const int32_t* srows; // [n]
  const uint32_t* mask; // [n] Morton order
  const unsigned char* plan;  // halo plan records (halo_tiles(n) x kPlanBytes)
  const int32_t* order;       // halo tiles in launch order
  int64_t n;
  const void* x;
  const void* w;
  void* y;
  int c_in, c_out;
  int x_dtype, w_dtype, y_dtype;  // TR_SC_*
  Epilogue epi;
};
hipError_t launch_forward_simple_f32(const ConvArgs& a, hipStream_t st);
// wp[k][co][ci] = w[k][ci][co] (bf16 or fp16), the matrix-core operand layout,
// followed by 256 zero bytes (packed_weight_elems elements, then the zeros).
__host__ __device__ inline int64_t packed_weight_elems(int c_in, int c_out) {
  return (int64_t(27) * c_in * c_out + 127) / 128 * 128;  // keeps the zero block 256-byte aligned
}
hipError_t launch_pack_weights(const void* w, void* wp, int c_in, int c_out, hipStream_t st);
// Shapes the halo gather-GEMM takes (half-precision features). Their packed
// weights carry, after the zero block, a second copy in MFMA fragment order:
// fragment (32-channel chunk c, tap k, 16-channel step s, 32-column block b)
// is 64 lanes x 8 halves at ((c * 27 + k) * 2 + s) * (c_out / 32) + b, lane l
// holding column 32 b + l % 32, input channels 32 c + 16 s + 8 (l / 32) .. + 8
// -- one contiguous kilobyte per fragment, the stages of the gather-GEMM
// (chunk-major, taps in order) at a constant stride.
inline bool halo_shape(int c_in, int c_out) {
  return c_in % 64 == 0 && c_in <= 1024 && (c_out == 32 || c_out == 64 || (c_out % 128 == 0 && c_out <= 1024));
}
__host__ __device__ inline int64_t frag_weight_offset(int c_in, int c_out) {  // in halves
  return packed_weight_elems(c_in, c_out) + 128;  // after the 256-byte zero block
}
inline int64_t packed_half_bytes(int c_in, int c_out) {
  const int64_t base = packed_weight_elems(c_in, c_out) * 2 + 256;
  return halo_shape(c_in, c_out) ? base + int64_t(27) * c_in * c_out * 2 : base;
}
// Fragment-order copy of a [27][c_out][c_in] packing (wp) at wp + frag_weight_offset.
hipError_t launch_pack_frag(void* wp, int c_in, int c_out, hipStream_t st);
hipError_t launch_forward_mfma(const ConvArgs& a, const void* wp, hipStream_t st);

// Backward. Data-gradient weights: the forward packing of the c_out -> c_in
// convolution with taps reversed (packed_weight_elems(c_out, c_in) elements and
// the zero block for half types; [27][c_out][c_in] for fp32).
hipError_t launch_pack_dgrad(const void* w, void* wp, int c_in, int c_out, int dtype, hipStream_t st);

// Weight gradient: split of the positions into `splits` ranges of `range`
// positions; partials [splits][27][c_in][c_out] fp32 when splits > 1.
struct WgradPlan {
  int ti, tj, tiles_i, tiles, splits;
  int64_t range;
  size_t partial_bytes;
};
WgradPlan plan_wgrad(int64_t n, int c_in, int c_out);
struct WgradCall {
  const int32_t* nbr;
  const int32_t* grows;
  const uint32_t* gmask;
  int64_t n;
  const void* x;
  const void* dy;
  float* dw;        // [27, c_in, c_out]
  float* partials;  // plan_wgrad(...).partial_bytes
  void* zeros;      // 256 bytes of workspace
  int c_in, c_out, dtype;
};
hipError_t launch_wgrad(const WgradCall& c, hipStream_t st);

// Resolution levels: per-1024-item block partials (int64) scanned in place; the
// produced count goes to *total.
int64_t level_blocks(int64_t n);
hipError_t launch_downsample(const uint64_t* skeys, const int32_t* srows, int64_t n, int64_t cap, int64_t* part,
                             int64_t* total, int32_t* coarse, int32_t* children, hipStream_t st);
hipError_t launch_subdivide(const int32_t* coords, const uint8_t* keep, int64_t n, int64_t cap, int64_t* part,
                            int64_t* total, uint32_t* flags, int32_t* fine, int32_t* children, hipStream_t st);
hipError_t launch_regroup(const int32_t* children, int64_t n_coarse, void* xc, void* xf, int c_fine, int elem_bytes,
                          bool to_fine, hipStream_t st);

}  // namespace trsc
