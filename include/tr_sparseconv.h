/* tr_sparseconv.h -- C ABI of the submanifold sparse 3D convolution library
 * (gfx950 / MI355X, HIP).
 *
 * The operation. For a set of N active voxels with integer coordinates
 * (b, x, y, z), features x[N, C_in] and tap-major weights w[27, C_in, C_out],
 * the library computes, for every active voxel i and output channel co,
 *
 *     y[i, co] = sum over taps k (0..26) whose neighbour j = nbr[i][k] is active,
 *                sum over ci of  w[k, ci, co] * x[j, ci]
 *
 * and writes output rows only at the active voxels. The pages define it as a
 * spatial hash of the active voxels followed, per kernel position, by a gather
 * of neighbour features, a product with that position's weights and a sum into
 * the output ("Running TRELLIS.2 on a Mac (1/3)", section "Swapping out the CUDA
 * libraries one at a time", sparse 3D convolution paragraph); as a neighbour
 * table built once per resolution level and a gather-GEMM over it with
 * half-precision inputs and single-precision accumulation ("Porting TRELLIS.2
 * From Python to Rust and Metal", section V); with features kept sparse rather
 * than materialised on a dense grid (mlx-diffuser TRELLIS guide, section "Why it
 * fits better on a Mac").
 *
 * Conventions.
 *  - Coordinates: int32 rows (b, x, y, z), each component in [0, 65536)
 *    (startup packet, page 5, section 5, fixture table row B).
 *  - Features: row-major [N, C] (same table, rows C-D). Row i of every per-voxel
 *    array (x, y, nbr) belongs to coordinate row i as the caller gave it.
 *  - Weights: tap-major [27, C_in, C_out] (startup packet, section 5 conv
 *    conventions and section 8), tap k = 9*Kd + 3*Kh + Kw.
 *  - Tap k reads the voxel at (x + Kd - 1, y + Kh - 1, z + Kw - 1) in the same
 *    object b: cross-correlation, equal to a dense 3x3x3 convolution with zero
 *    padding 1 evaluated at the active sites. A neighbour outside [0, 65536) on
 *    any axis does not exist.
 *
 * Memory and streams. Every tensor pointer is a DEVICE pointer owned by the
 * caller, who must keep it alive while a handle that refers to it is in use.
 * `stream` is a hipStream_t (NULL = the null stream). Work is enqueued on it;
 * only tr_sparseconv_status and the level calls that return a row count
 * (tr_sparseconv_downsample, tr_sparseconv_subdivide) wait for the device.
 * Handles are small host structs; destroying one frees that struct only, never
 * device memory.
 *
 * Errors. Every int-returning call returns TR_SC_OK (0) or a negative
 * tr_sc_status. A failed call enqueues nothing further and records a message
 * for tr_sparseconv_last_error() (thread-local). Problems that only the device
 * can see (coordinates out of range, duplicate coordinates, a full table) are
 * kept in a status word inside the hash workspace and returned by
 * tr_sparseconv_status.
 */
#ifndef TR_SPARSECONV_H
#define TR_SPARSECONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TR_SC_OK = 0,
  TR_SC_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad handle      */
  TR_SC_ERR_COORD_RANGE = -2, /* a coordinate component outside [0, 65536)    */
  TR_SC_ERR_DUPLICATE = -3,   /* the same (b, x, y, z) given twice            */
  TR_SC_ERR_CAPACITY = -4,    /* hash table ran out of slots                  */
  TR_SC_ERR_WORKSPACE = -5,   /* workspace smaller than the *_workspace_bytes */
  TR_SC_ERR_UNSUPPORTED = -6, /* dtype / channel count the library lacks      */
  TR_SC_ERR_HIP = -7          /* a HIP runtime call failed                    */
} tr_sc_status;

typedef enum { TR_SC_F32 = 0, TR_SC_BF16 = 1, TR_SC_F16 = 2 } tr_sc_dtype;

/* Activation of the fused epilogue (tr_sparseconv_forward_fused). */
typedef enum {
  TR_SC_ACT_NONE = 0,
  TR_SC_ACT_RELU = 1, /* max(v, 0)                 */
  TR_SC_ACT_SILU = 2  /* v / (1 + exp(-v))         */
} tr_sc_act;

typedef struct tr_sc_hash tr_sc_hash; /* coordinate hash (opaque)  */
typedef struct tr_sc_kmap tr_sc_kmap; /* kernel map (opaque)       */

/* Library version, (major << 16) | minor. */
int tr_sparseconv_version(void);

/* ------------------------------------------------------------------------
 * Coordinate hash.
 * The "spatial hash of the active voxels" of the definition above. The voxels
 * are sorted along a Morton (Z-order) curve and inserted into an
 * open-addressing table in the workspace.
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace tr_sparseconv_build_hash needs for n voxels
 * (0 for n < 0). */
size_t tr_sparseconv_hash_workspace_bytes(int64_t n);

/* coords    device int32 [n, 4] (b, x, y, z); read during this call only.
 * n         number of voxels, 0 <= n <= 2^30 (n = 0 is valid: empty hash).
 * workspace device buffer of >= tr_sparseconv_hash_workspace_bytes(n) bytes,
 *           256-byte aligned; it holds the table and must outlive the handle.
 * out       receives a new handle (release with tr_sparseconv_hash_destroy).
 * Enqueues the whole build on `stream` and returns without waiting for the
 * device. Coordinates with a component outside [0, 65536) and duplicate
 * coordinates are found on the device and reported by tr_sparseconv_status;
 * until then the hash of such input must not be used. */
int tr_sparseconv_build_hash(const int32_t* coords, int64_t n, void* workspace,
                             size_t ws_bytes, void* stream, tr_sc_hash** out);

/* The same hash for voxels in a known grid: spatial components in
 * [0, 2^grid_log2), object index b in [0, batch) -- the resolution of a level,
 * which every level of the pages' decoders has ("Running TRELLIS.2 on a Mac
 * (1/3)", the resolutions of the cascade). The result is the same as
 * tr_sparseconv_build_hash's: the same Morton order (tr_sparseconv_hash_sorted_rows),
 * the same lookups and kernel map. When the grid's occupancy bitmap
 * (batch * 2^(3 grid_log2) bits) is at most 32 MB, the order comes from that
 * bitmap (a voxel's position is the number of occupied cells before its own)
 * in five kernels instead of the radix sort's passes; otherwise this is
 * tr_sparseconv_build_hash with the grid's bounds as the range check.
 * grid_log2 in [2, 16], batch in [1, 65536] (else TR_SC_ERR_INVALID_ARG).
 * Coordinates outside the grid and duplicates are reported by
 * tr_sparseconv_status as TR_SC_ERR_COORD_RANGE and TR_SC_ERR_DUPLICATE. */
size_t tr_sparseconv_hash_grid_workspace_bytes(int64_t n, int grid_log2, int batch);
int tr_sparseconv_build_hash_grid(const int32_t* coords, int64_t n, int grid_log2, int batch,
                                  void* workspace, size_t ws_bytes, void* stream, tr_sc_hash** out);

/* Device-found errors of the build, read from the workspace status word:
 * TR_SC_OK, TR_SC_ERR_COORD_RANGE, TR_SC_ERR_DUPLICATE or TR_SC_ERR_CAPACITY.
 * Synchronises `stream`. */
int tr_sparseconv_status(const tr_sc_hash* h, void* stream);

/* Number of voxels the hash was built over. */
int64_t tr_sparseconv_hash_size(const tr_sc_hash* h);

/* Test hook. q: device int32 [nq, 4] queries; idx: device int32 [nq] receives
 * the caller row of each query, or -1 when it is not an active voxel (also for
 * components outside [0, 65536)). */
int tr_sparseconv_hash_lookup(const tr_sc_hash* h, const int32_t* q, int64_t nq,
                              int32_t* idx, void* stream);

/* Test hook. perm: device int32 [n] receives the caller row at each position
 * of the Morton order (stable: equal keys cannot occur in a valid set). */
int tr_sparseconv_hash_sorted_rows(const tr_sc_hash* h, int32_t* perm, void* stream);

void tr_sparseconv_hash_destroy(tr_sc_hash* h);

/* ------------------------------------------------------------------------
 * Kernel map (the neighbour table, built once per resolution level and reused
 * by every layer at that level -- "Porting TRELLIS.2 ...", section V).
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace tr_sparseconv_build_kernel_map needs. */
size_t tr_sparseconv_kmap_workspace_bytes(int64_t n);

/* h         hash from tr_sparseconv_build_hash (its workspace must stay alive).
 * nbr       device int32 [n, 27] output: nbr[i*27 + k] = caller row of the
 *           neighbour of voxel i at tap k, or -1. nbr[i*27 + 13] = i.
 *           Owned by the caller; the kernel map reads it in every forward.
 * workspace device buffer >= tr_sparseconv_kmap_workspace_bytes(n) bytes
 *           (per-voxel neighbour masks in Morton order, the gather-GEMM's row
 *           order, and per tile of 256 Morton-consecutive voxels the plan of
 *           the halo gather-GEMM: 20,480 bytes, plus the tiles' launch order);
 *           must outlive the handle.
 * out       receives a new handle (release with tr_sparseconv_kmap_destroy). */
int tr_sparseconv_build_kernel_map(const tr_sc_hash* h, int32_t* nbr, void* workspace,
                                   size_t ws_bytes, void* stream, tr_sc_kmap** out);

void tr_sparseconv_kmap_destroy(tr_sc_kmap* m);

/* ------------------------------------------------------------------------
 * Forward: the gather-GEMM over the kernel map.
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace tr_sparseconv_forward needs (the packed weights,
 * see tr_sparseconv_pack_weights below). */
size_t tr_sparseconv_forward_workspace_bytes(int c_in, int c_out, int dtype);

/* m      kernel map of the voxel set.
 * x      device [n, c_in] features, dtype `dtype`.
 * w      device [27, c_in, c_out] weights, dtype `dtype`.
 * y      device [n, c_out] output, dtype `dtype`; every element is written.
 * dtype  TR_SC_BF16 / TR_SC_F16: half inputs, fp32 accumulation, output
 *        rounded to the same half type (nearest, ties to even); needs
 *        c_in % 8 == 0 and c_out % 8 == 0.
 *        TR_SC_F32: fp32 inputs, fp32 accumulation and output; any c >= 1.
 * No atomics: the result is the same bit for bit on every call. x and y must
 * not overlap; y == x is rejected with TR_SC_ERR_INVALID_ARG. */
int tr_sparseconv_forward(const tr_sc_kmap* m, const void* x, const void* w, void* y,
                          int c_in, int c_out, int dtype, void* workspace,
                          size_t ws_bytes, void* stream);

/* tr_sparseconv_forward for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, result bits and errors as
 * tr_sparseconv_forward, without the workspace: the packed weights go to a
 * scratch array inside the library, 8 MiB per GPU, held until the process
 * ends; the call itself allocates nothing. Limit: the packed half-precision
 * weights, tr_sparseconv_packed_weights_bytes(c_in, c_out, dtype), must fit in
 * 8 MiB: 27 * c_in * c_out * 2 + 256 bytes, plus a second copy of the
 * 27 * c_in * c_out * 2 bytes in the halo kernel's fragment order for its
 * shapes (c_in a multiple of 64 up to 1024; c_out 32, 64 or a multiple of 128
 * up to 1024). E.g. 256 x 256 (7.1 MB) or 392 x 392 (8.3 MB) fit, 384 x 384
 * (15.9 MB) does not; else TR_SC_ERR_WORKSPACE and nothing is enqueued (fp32
 * reads w in place and has no limit). Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (two streams or threads) race; `stream`
 * must belong to the current device. */
int tr_sparseconv_forward_noalloc(const tr_sc_kmap* m, const void* x, const void* w, void* y,
                                  int c_in, int c_out, int dtype, void* stream);

/* The two halves of tr_sparseconv_forward, for callers that reuse one set of
 * weights across many calls (a layer applied to many inputs):
 *
 * tr_sparseconv_pack_weights: wp (device, >= tr_sparseconv_packed_weights_bytes
 * bytes, 16-byte aligned, caller-owned) receives w [27, c_in, c_out] re-laid
 * out for the matrix cores (bf16, f16: [27, c_out, c_in]; f32: unchanged copy).
 * tr_sparseconv_forward_packed: as tr_sparseconv_forward, reading the packed
 * weights. Same argument rules and errors as tr_sparseconv_forward. */
size_t tr_sparseconv_packed_weights_bytes(int c_in, int c_out, int dtype);
int tr_sparseconv_pack_weights(const void* w, int c_in, int c_out, int dtype, void* wp,
                               size_t wp_bytes, void* stream);
int tr_sparseconv_forward_packed(const tr_sc_kmap* m, const void* x, const void* wp, void* y,
                                 int c_in, int c_out, int dtype, void* stream);

/* The gather-GEMM with its epilogue fused into the same pass, and mixed
 * precision. The pages fuse bias, activation, residual add and the output
 * rounding into the convolution pass ("Porting TRELLIS.2 From Python to Rust
 * and Metal", section V), and keep the decoders' incoming latent in fp32 while
 * the layers after it run in half precision (same page, section IV).
 *
 *   y[i, co] = round_y( act( conv(x, w)[i, co] + bias[co] ) + residual[i, co] )
 *
 * computed in fp32 and rounded once, to y's type.
 * m         kernel map.
 * x         device [n, c_in], type x_dtype.
 * wp        packed weights of type w_dtype (tr_sparseconv_pack_weights).
 * w_dtype   TR_SC_BF16 or TR_SC_F16: x_dtype is w_dtype, or TR_SC_F32 (fp32
 *           features, never rounded to half first: x is carried as a sum of
 *           half terms, each multiplied exactly -- 3 bf16 terms hold x
 *           exactly; 2 fp16 terms hold it to within 2^-23 |x| + 2^-25 and
 *           need |x| < 65504); y_dtype is w_dtype or TR_SC_F32; c_in
 *           and c_out multiples of 8; x, y, residual 16-byte aligned.
 *           TR_SC_F32: x_dtype = y_dtype = TR_SC_F32, any c >= 1.
 * bias      device fp32 [c_out], or NULL for none.
 * act       tr_sc_act.
 * residual  device [n, c_out] of type y_dtype, or NULL. It may be y itself
 *           (in-place residual add); otherwise it must not overlap y.
 * y         device [n, c_out], type y_dtype; every element is written. x must
 *           not overlap y.
 * Errors as tr_sparseconv_forward; TR_SC_ERR_UNSUPPORTED for other dtype
 * combinations. */
int tr_sparseconv_forward_fused(const tr_sc_kmap* m, const void* x, int x_dtype, const void* wp,
                                int w_dtype, const float* bias, int act, const void* residual,
                                void* y, int y_dtype, int c_in, int c_out, void* stream);

/* ------------------------------------------------------------------------
 * Backward: the gradients of L = sum_i <y[i], dy[i]> for y = the convolution
 * of x with w. From the forward sum above, each term w[k, ci, co] * x[j, ci]
 * with j = nbr[i][k] contributes w[k, ci, co] * dy[i, co] to dx[j, ci] and
 * x[j, ci] * dy[i, co] to dw[k, ci, co].
 * ------------------------------------------------------------------------ */

/* Data gradient. Voxel i reads j at tap k exactly when j reads i at tap 26 - k,
 * so dx is the forward gather-GEMM over the same kernel map with input dy and
 * mirrored, transposed weights.
 * tr_sparseconv_pack_weights_dgrad: w [27, c_in, c_out] (dtype) -> wp, of
 *   >= tr_sparseconv_packed_weights_bytes(c_in, c_out, dtype) bytes, 16-byte
 *   aligned, caller-owned.
 * tr_sparseconv_backward_data: dy [n, c_out] (dy_dtype), wp from
 *   tr_sparseconv_pack_weights_dgrad (w_dtype), dx [n, c_in] (dx_dtype; every
 *   element written). Type rules, alignment and errors as
 *   tr_sparseconv_forward_fused with (x, y) = (dy, dx). */
int tr_sparseconv_pack_weights_dgrad(const void* w, int c_in, int c_out, int dtype, void* wp,
                                     size_t wp_bytes, void* stream);
int tr_sparseconv_backward_data(const tr_sc_kmap* m, const void* dy, int dy_dtype, const void* wp,
                                int w_dtype, void* dx, int dx_dtype, int c_in, int c_out,
                                void* stream);

/* Weight gradient dw [27, c_in, c_out], fp32, every element written.
 * x [n, c_in] and dy [n, c_out] share dtype (bf16, f16 with c_in, c_out
 * multiples of 8 and 16-byte aligned pointers; or f32). The half-precision
 * path sums over voxel pairs on the matrix cores in fp32, split over ranges of
 * voxels whose partial sums are added in a fixed order (no atomics: the same
 * bits on every call). workspace: >= tr_sparseconv_backward_weights_workspace_bytes
 * bytes, 256-byte aligned (0 bytes for f32). */
size_t tr_sparseconv_backward_weights_workspace_bytes(int64_t n, int c_in, int c_out, int dtype);
int tr_sparseconv_backward_weights(const tr_sc_kmap* m, const void* x, const void* dy, float* dw,
                                   int c_in, int c_out, int dtype, void* workspace,
                                   size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Resolution levels. The pages build one neighbour table per resolution level
 * ("Porting TRELLIS.2 ...", section V) and move between levels with
 * pixel-shuffle / Channel2Spatial upsampling driven by subdivision
 * predictions (TRELLIS.2 MLX port README: repository tree, pipeline list).
 * Conventions: the parent of (b, x, y, z) is (b, x >> 1, y >> 1, z >> 1);
 * child o = 4 dx + 2 dy + dz of (b, x, y, z) is (b, 2x + dx, 2y + dy, 2z + dz);
 * a parent feature row of 8C channels holds channel c of child o at c * 8 + o.
 * A `children` table is int32 [n_coarse, 8]: the row of child o, or -1.
 * ------------------------------------------------------------------------ */

/* Workspace bytes of tr_sparseconv_downsample / tr_sparseconv_subdivide over n
 * input rows (256-byte aligned buffer). */
size_t tr_sparseconv_level_workspace_bytes(int64_t n);

/* Parent level of the voxel set of h: coarse_coords int32 [cap, 4] receives
 * the parents ordered by b, then Z-order of (x, y, z); children [cap, 8] their
 * children (rows of h's coordinate array). *n_coarse receives the count (one
 * small read-back: the call waits for `stream`). TR_SC_ERR_CAPACITY if more
 * than cap parents (cap = n always suffices). No sort: the hash's Morton
 * order already groups children by parent. */
int tr_sparseconv_downsample(const tr_sc_hash* h, int32_t* coarse_coords, int32_t* children,
                             int64_t cap, void* workspace, size_t ws_bytes, void* stream,
                             int64_t* n_coarse);

/* Finer level: coords int32 [n, 4] (16-byte aligned); keep uint8 [n], bit o
 * set = child o exists (NULL: all eight). fine_coords int32 [cap, 4] receives
 * the children in (row, octant) order, children [n, 8] their fine rows.
 * *n_fine receives the count (read back; waits for `stream`).
 * TR_SC_ERR_COORD_RANGE if a component is negative or a child would leave
 * [0, 65536); TR_SC_ERR_CAPACITY if more than cap children (8n suffices). */
int tr_sparseconv_subdivide(const int32_t* coords, int64_t n, const uint8_t* keep,
                            int32_t* fine_coords, int32_t* children, int64_t cap,
                            void* workspace, size_t ws_bytes, void* stream, int64_t* n_fine);

/* Channel2Spatial: x_fine[children[q][o], c] = x_coarse[q, c * 8 + o]
 * (x_coarse [n_coarse, 8 c_fine], x_fine [*, c_fine]; fine rows that are no
 * one's child are left as they are). Spatial2Channel, its inverse gather:
 * x_coarse[q, c * 8 + o] = x_fine[children[q][o], c], or 0 where child o is
 * absent. dtype: f32 (c_fine % 4 == 0), bf16 or f16 (c_fine % 8 == 0); all
 * pointers 16-byte aligned. Pure data movement: bit-exact. */
int tr_sparseconv_channel2spatial(const int32_t* children, int64_t n_coarse, const void* x_coarse,
                                  void* x_fine, int c_fine, int dtype, void* stream);
int tr_sparseconv_spatial2channel(const int32_t* children, int64_t n_coarse, const void* x_fine,
                                  void* x_coarse, int c_fine, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * Measured ceilings (for the benchmark's roofline fractions; they compute
 * nothing of the convolution). Both enqueue one kernel on `stream`.
 * ------------------------------------------------------------------------ */

/* bf16 matrix-core ceiling: `grid` workgroups of four waves, each wave issuing
 * `iters` rounds of four independent 32x32x16 bf16 multiply-accumulates.
 * out: device float [grid * 256], receives one value per thread (caller-owned).
 * tr_sparseconv_ceiling_mfma_flops gives the flops of one launch (0 for
 * non-positive arguments). Errors: TR_SC_ERR_INVALID_ARG for a null out or
 * non-positive grid / iters; TR_SC_ERR_HIP if the launch fails. */
int64_t tr_sparseconv_ceiling_mfma_flops(int grid, int iters);
int tr_sparseconv_ceiling_mfma(float* out, int grid, int iters, void* stream);

/* HBM streaming ceiling: dst[0, bytes) = src[0, bytes) with 16-byte accesses
 * by `grid` workgroups of 256 threads (grid-stride). src and dst are
 * caller-owned device buffers, 16-byte aligned, not overlapping; bytes a
 * multiple of 16. Errors: TR_SC_ERR_INVALID_ARG otherwise; TR_SC_ERR_HIP if the
 * launch fails. */
int tr_sparseconv_ceiling_copy(const void* src, void* dst, size_t bytes, int grid, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* tr_sparseconv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TR_SPARSECONV_H */
