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
// Packs keys / rows and initialises the header (flags, digits of the sort).
hipError_t launch_pack(const int32_t* coords, int64_t n, uint64_t* keys, int32_t* rows,
                       unsigned long long* part, HashHeader* hdr, hipStream_t st);
// Three LSD radix passes (digits from the header) keys0 -> keys1 -> keys0 ->
// keys1, then the single-workgroup pass over any further bits: the sorted keys
// and rows end in keys1 / rows1. counts: sort_blocks(n) * kSortBuckets words.
hipError_t launch_sort(uint64_t* keys0, int32_t* rows0, uint64_t* keys1, int32_t* rows1, int64_t n,
                       const HashHeader* hdr, uint32_t* counts, uint32_t* totals, hipStream_t st);
hipError_t launch_blocks(const uint64_t* keys, int64_t n, BlockSlot* slots, uint32_t max_cap,
                         uint32_t* part, HashHeader* hdr, hipStream_t st);
hipError_t launch_lookup(const TableRef& t, const int32_t* q, int64_t nq, int32_t* out, hipStream_t st);

// Kernel map (nbr, caller order; mask, Morton order) and the gather-GEMM row
// order: grows / gmask = Morton order regrouped inside windows of kGroupWindow
// voxels by the octant pattern of the neighbour mask.
constexpr int kGroupWindow = 4096;
hipError_t launch_kmap(const uint64_t* skeys, int64_t n, const TableRef& t, int32_t* nbr, uint32_t* mask,
                       int32_t* grows, uint32_t* gmask, hipStream_t st);

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
inline int64_t packed_weight_elems(int c_in, int c_out) {
  return (int64_t(27) * c_in * c_out + 127) / 128 * 128;  // keeps the zero block 256-byte aligned
}
hipError_t launch_pack_weights(const void* w, void* wp, int c_in, int c_out, hipStream_t st);
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
