// C ABI of the library (declared in include/tr_sparseconv.h): argument checks,
// workspace layout, launches. No device memory is allocated here; every buffer
// comes from the caller.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "common.h"
#include "launch.h"
#include "tr_sparseconv.h"

using namespace trsc;

namespace {

constexpr uint32_t kHashMagic = 0x48534354u;  // "TCSH"
constexpr uint32_t kKmapMagic = 0x4D4B4354u;  // "TCKM"
constexpr int64_t kMaxN = int64_t(1) << 30;  // table capacity 2^31 slots at most

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(TR_SC_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

uint32_t table_capacity(int64_t n) {  // largest table: power of two >= 2n (one block per voxel), >= 16
  uint64_t p = 16;
  while (p < uint64_t(2 * n) && p < (uint64_t(1) << 31)) p <<= 1;
  return uint32_t(p);
}

// Hash workspace: header | keys[2][n] | rows[2][n] | radix counts | digit
// totals | per-workgroup partials | block slots[capacity].
struct HashLayout {
  size_t hdr, keys0, keys1, rows0, rows1, counts, totals, parts, slots, total;
  uint32_t cap;
};

HashLayout hash_layout(int64_t n) {
  HashLayout l{};
  const size_t un = size_t(n);
  size_t o = 0;
  l.hdr = o;
  o += align_up(sizeof(HashHeader), 256);
  l.keys0 = o;
  o += align_up(un * 8, 256);
  l.keys1 = o;
  o += align_up(un * 8, 256);
  l.rows0 = o;
  o += align_up(un * 4, 256);
  l.rows1 = o;
  o += align_up(un * 4, 256);
  l.counts = o;
  o += align_up(size_t(sort_blocks(n)) * kSortBuckets * 4, 256);
  l.totals = o;
  o += kSortBuckets * 4;
  l.parts = o;
  o += align_up(size_t(pack_partials(n)) * 24, 256);
  l.cap = table_capacity(n);
  l.slots = o;
  o += size_t(l.cap) * sizeof(BlockSlot);
  l.total = o;
  return l;
}

}  // namespace

struct tr_sc_hash {
  uint32_t magic;
  int64_t n;
  HashHeader* hdr;
  TableRef table;         // block slots, header (capacity, shift), sorted rows
  const uint64_t* skeys;  // sorted keys
  bool has_dense;         // built in a known grid from an occupancy bitmap
  DenseRef dense;
};

struct tr_sc_kmap {
  uint32_t magic;
  int64_t n;
  const int32_t* nbr;
  const int32_t* grows;        // tile row order (position -> caller row)
  const uint32_t* gmask;       // neighbour mask of each position
  const unsigned char* plan;   // halo plan records of the gather-GEMM
  const int32_t* order;        // its tiles in launch order
};

extern "C" {

int tr_sparseconv_version(void) { return (0 << 16) | 1; }

const char* tr_sparseconv_last_error(void) { return g_last_error.c_str(); }

size_t tr_sparseconv_hash_workspace_bytes(int64_t n) {
  if (n < 0 || n > kMaxN) return 0;
  return hash_layout(n).total;
}

static int build_hash_radix(const char* who, const int32_t* coords, int64_t n, uint32_t lim, uint32_t blim,
                            void* workspace, size_t ws_bytes, void* stream, tr_sc_hash** out) {
  if (out == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "%s: out is NULL", who);
  *out = nullptr;
  if (n < 0 || n > kMaxN) return fail(TR_SC_ERR_INVALID_ARG, "%s: n = %lld out of [0, 2^30]", who, (long long)n);
  if (n > 0 && coords == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "%s: coords is NULL", who);
  if (workspace == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "%s: workspace is NULL", who);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TR_SC_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned", who);
  if (reinterpret_cast<uintptr_t>(coords) % 16 != 0)
    return fail(TR_SC_ERR_INVALID_ARG, "%s: coords not 16-byte aligned", who);
  const HashLayout l = hash_layout(n);
  if (ws_bytes < l.total)
    return fail(TR_SC_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", who, ws_bytes, l.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  HashHeader* hdr = reinterpret_cast<HashHeader*>(ws + l.hdr);
  uint64_t* keys[2] = {reinterpret_cast<uint64_t*>(ws + l.keys0), reinterpret_cast<uint64_t*>(ws + l.keys1)};
  int32_t* rows[2] = {reinterpret_cast<int32_t*>(ws + l.rows0), reinterpret_cast<int32_t*>(ws + l.rows1)};
  uint32_t* counts = reinterpret_cast<uint32_t*>(ws + l.counts);
  uint32_t* totals = reinterpret_cast<uint32_t*>(ws + l.totals);
  unsigned long long* parts = reinterpret_cast<unsigned long long*>(ws + l.parts);
  BlockSlot* slots = reinterpret_cast<BlockSlot*>(ws + l.slots);

  // No host wait: the digits of the sort are chosen on the device from the key
  // bits that vary; range and duplicate errors are left in the header for
  // tr_sparseconv_status.
  hipError_t e = launch_pack(coords, n, lim, blim, keys[0], rows[0], keys[1], rows[1], parts, hdr, st);
  if (e != hipSuccess) return hip_fail(e, who);
  const int cur = 1;
  if (n > 0) {
    e = launch_sort(keys[0], rows[0], keys[1], rows[1], n, hdr, parts, counts, totals, st);
    if (e != hipSuccess) return hip_fail(e, who);
  }
  e = launch_blocks(keys[cur], n, slots, l.cap, reinterpret_cast<uint32_t*>(parts), hdr, st);
  if (e != hipSuccess) return hip_fail(e, who);

  tr_sc_hash* h = new tr_sc_hash;
  h->magic = kHashMagic;
  h->n = n;
  h->hdr = hdr;
  h->table = TableRef{slots, hdr, rows[cur]};
  h->skeys = keys[cur];
  h->has_dense = false;
  h->dense = DenseRef{};
  *out = h;
  return TR_SC_OK;
}

int tr_sparseconv_build_hash(const int32_t* coords, int64_t n, void* workspace, size_t ws_bytes,
                             void* stream, tr_sc_hash** out) {
  return build_hash_radix("build_hash", coords, n, 0x10000u, 0x10000u, workspace, ws_bytes, stream, out);
}

// The occupancy-bitmap build applies when the grid's bitmap is at most 32 MB
// (4M words of 64 cells).
constexpr int64_t kDenseMaxWords = int64_t(1) << 22;
static int64_t grid_words(int g, int batch) {  // 64-cell words of a batch x (2^g)^3 grid, g >= 2
  return int64_t(batch) << (3 * g - 6);
}
static bool grid_dense(int64_t n, int g, int batch) {
  return n > 0 && (3 * g - 6 <= 22) && grid_words(g, batch) <= kDenseMaxWords;
}

// Grid workspace (bitmap build): header | keys[n] | rows[n] | bitmap | word
// prefixes | chunk totals | chunk block counts | chunk first positions | block
// slots.
struct GridLayout {
  size_t hdr, keys, rows, bitmap, wpre, ctot, cblk, cpre, slots, total;
  int lgc, nchunks;
  uint32_t cap;
};
static GridLayout grid_layout(int64_t n, int g, int batch) {
  GridLayout l{};
  const int64_t words = grid_words(g, batch);
  l.lgc = dense_chunk_log2(words);
  l.nchunks = int((words + (int64_t(1) << l.lgc) - 1) >> l.lgc);
  const size_t w = size_t(l.nchunks) << l.lgc;
  size_t o = 0;
  l.hdr = o;
  o += align_up(sizeof(HashHeader), 256);
  l.keys = o;
  o += align_up(size_t(n) * 8, 256);
  l.rows = o;
  o += align_up(size_t(n) * 4, 256);
  l.bitmap = o;
  o += align_up(w * 8, 256);
  l.wpre = o;
  o += align_up(w * 4, 256);
  l.ctot = o;
  o += align_up(size_t(l.nchunks) * 4, 256);
  l.cblk = o;
  o += align_up(size_t(l.nchunks) * 4, 256);
  l.cpre = o;
  o += align_up(size_t(l.nchunks) * 4, 256);
  l.cap = table_capacity(n < words ? n : words);
  l.slots = o;
  o += size_t(l.cap) * sizeof(BlockSlot);
  l.total = o;
  return l;
}

static bool grid_args_ok(int grid_log2, int batch) {
  return grid_log2 >= 2 && grid_log2 <= 16 && batch >= 1 && batch <= 65536;
}

size_t tr_sparseconv_hash_grid_workspace_bytes(int64_t n, int grid_log2, int batch) {
  if (n < 0 || n > kMaxN || !grid_args_ok(grid_log2, batch)) return 0;
  return grid_dense(n, grid_log2, batch) ? grid_layout(n, grid_log2, batch).total : hash_layout(n).total;
}

int tr_sparseconv_build_hash_grid(const int32_t* coords, int64_t n, int grid_log2, int batch, void* workspace,
                                  size_t ws_bytes, void* stream, tr_sc_hash** out) {
  if (out == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "build_hash_grid: out is NULL");
  *out = nullptr;
  if (!grid_args_ok(grid_log2, batch))
    return fail(TR_SC_ERR_INVALID_ARG, "build_hash_grid: grid_log2 = %d outside [2, 16] or batch = %d outside [1, 65536]",
                grid_log2, batch);
  if (n < 0 || n > kMaxN)
    return fail(TR_SC_ERR_INVALID_ARG, "build_hash_grid: n = %lld out of [0, 2^30]", (long long)n);
  if (!grid_dense(n, grid_log2, batch))
    return build_hash_radix("build_hash_grid", coords, n, 1u << grid_log2, uint32_t(batch), workspace, ws_bytes,
                            stream, out);
  if (coords == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "build_hash_grid: coords is NULL");
  if (workspace == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "build_hash_grid: workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TR_SC_ERR_INVALID_ARG, "build_hash_grid: workspace not 256-byte aligned");
  if (reinterpret_cast<uintptr_t>(coords) % 16 != 0)
    return fail(TR_SC_ERR_INVALID_ARG, "build_hash_grid: coords not 16-byte aligned");
  const GridLayout l = grid_layout(n, grid_log2, batch);
  if (ws_bytes < l.total)
    return fail(TR_SC_ERR_WORKSPACE, "build_hash_grid: workspace %zu bytes < %zu needed", ws_bytes, l.total);
  char* ws = static_cast<char*>(workspace);
  HashHeader* hdr = reinterpret_cast<HashHeader*>(ws + l.hdr);
  uint64_t* keys = reinterpret_cast<uint64_t*>(ws + l.keys);
  int32_t* rows = reinterpret_cast<int32_t*>(ws + l.rows);
  BlockSlot* slots = reinterpret_cast<BlockSlot*>(ws + l.slots);
  const hipError_t e = launch_dense_hash(
      coords, n, grid_log2, batch, reinterpret_cast<unsigned long long*>(ws + l.bitmap), l.lgc, l.nchunks,
      reinterpret_cast<uint32_t*>(ws + l.wpre), reinterpret_cast<uint32_t*>(ws + l.ctot),
      reinterpret_cast<uint32_t*>(ws + l.cblk), reinterpret_cast<uint32_t*>(ws + l.cpre), keys, rows, slots, l.cap,
      hdr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "build_hash_grid");
  tr_sc_hash* h = new tr_sc_hash;
  h->magic = kHashMagic;
  h->n = n;
  h->hdr = hdr;
  h->table = TableRef{slots, hdr, rows};
  h->skeys = keys;
  h->has_dense = true;
  h->dense = DenseRef{reinterpret_cast<const unsigned long long*>(ws + l.bitmap),
                      reinterpret_cast<const uint32_t*>(ws + l.wpre), reinterpret_cast<const uint32_t*>(ws + l.cpre),
                      l.lgc, l.nchunks, grid_log2};
  *out = h;
  return TR_SC_OK;
}

int tr_sparseconv_status(const tr_sc_hash* h, void* stream) {
  if (h == nullptr || h->magic != kHashMagic) return fail(TR_SC_ERR_INVALID_ARG, "status: bad hash handle");
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t flags = 0;
  hipError_t e = hipMemcpyAsync(&flags, &h->hdr->flags, sizeof(flags), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "status");
  if (flags & kFlagCoordRange) return fail(TR_SC_ERR_COORD_RANGE, "status: coordinate out of range");
  if (flags & kFlagDuplicate) return fail(TR_SC_ERR_DUPLICATE, "status: duplicate coordinates");
  if (flags & kFlagCapacity) return fail(TR_SC_ERR_CAPACITY, "status: hash table full");
  return TR_SC_OK;
}

int64_t tr_sparseconv_hash_size(const tr_sc_hash* h) {
  if (h == nullptr || h->magic != kHashMagic) return -1;
  return h->n;
}

int tr_sparseconv_hash_lookup(const tr_sc_hash* h, const int32_t* q, int64_t nq, int32_t* idx,
                              void* stream) {
  if (h == nullptr || h->magic != kHashMagic) return fail(TR_SC_ERR_INVALID_ARG, "hash_lookup: bad hash handle");
  if (nq < 0) return fail(TR_SC_ERR_INVALID_ARG, "hash_lookup: nq < 0");
  if (nq > 0 && (q == nullptr || idx == nullptr)) return fail(TR_SC_ERR_INVALID_ARG, "hash_lookup: NULL buffer");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0)
    return fail(TR_SC_ERR_INVALID_ARG, "hash_lookup: queries not 16-byte aligned");
  hipError_t e = launch_lookup(h->table, q, nq, idx, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hash_lookup");
  return TR_SC_OK;
}

int tr_sparseconv_hash_sorted_rows(const tr_sc_hash* h, int32_t* perm, void* stream) {
  if (h == nullptr || h->magic != kHashMagic) return fail(TR_SC_ERR_INVALID_ARG, "hash_sorted_rows: bad hash handle");
  if (h->n == 0) return TR_SC_OK;
  if (perm == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "hash_sorted_rows: perm is NULL");
  hipError_t e = hipMemcpyAsync(perm, h->table.srows, size_t(h->n) * 4, hipMemcpyDeviceToDevice,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hash_sorted_rows");
  return TR_SC_OK;
}

void tr_sparseconv_hash_destroy(tr_sc_hash* h) {
  if (h != nullptr && h->magic == kHashMagic) {
    h->magic = 0;
    delete h;
  }
}

// Kernel-map workspace: mask[n] (Morton order) | grows[n] | gmask[n] (tile
// order) | halo plan (one record per tile of kHaloTM voxels) | the tiles'
// launch order | their costs.
size_t tr_sparseconv_kmap_workspace_bytes(int64_t n) {
  if (n < 0 || n > kMaxN) return 0;
  return 3 * align_up(size_t(n) * 4, 256) + size_t(halo_tiles(n)) * kPlanBytes +
         align_up(size_t(halo_tiles(n)) * 4, 256) + align_up(size_t(halo_tiles(n)) * 2, 256) + 256;
}

int tr_sparseconv_build_kernel_map(const tr_sc_hash* h, int32_t* nbr, void* workspace, size_t ws_bytes,
                                   void* stream, tr_sc_kmap** out) {
  if (out == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "build_kernel_map: out is NULL");
  *out = nullptr;
  if (h == nullptr || h->magic != kHashMagic) return fail(TR_SC_ERR_INVALID_ARG, "build_kernel_map: bad hash handle");
  if (workspace == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "build_kernel_map: workspace is NULL");
  if (h->n > 0 && nbr == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "build_kernel_map: nbr is NULL");
  const size_t need = tr_sparseconv_kmap_workspace_bytes(h->n);
  if (ws_bytes < need)
    return fail(TR_SC_ERR_WORKSPACE, "build_kernel_map: workspace %zu bytes < %zu needed", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TR_SC_ERR_INVALID_ARG, "build_kernel_map: workspace not 256-byte aligned");
  const size_t part = align_up(size_t(h->n) * 4, 256);
  uint32_t* mask = static_cast<uint32_t*>(workspace);
  int32_t* grows = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + part);
  uint32_t* gmask = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + 2 * part);
  unsigned char* plan = static_cast<unsigned char*>(workspace) + 3 * part;
  int32_t* order = reinterpret_cast<int32_t*>(plan + size_t(halo_tiles(h->n)) * kPlanBytes);
  uint16_t* costs = reinterpret_cast<uint16_t*>(reinterpret_cast<unsigned char*>(order) +
                                                align_up(size_t(halo_tiles(h->n)) * 4, 256));
  hipError_t e = launch_kmap(h->skeys, h->n, h->table, h->has_dense ? &h->dense : nullptr, nbr, mask, grows, gmask,
                             plan, costs, order, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "build_kernel_map");
  tr_sc_kmap* m = new tr_sc_kmap;
  m->magic = kKmapMagic;
  m->n = h->n;
  m->nbr = nbr;
  m->grows = grows;
  m->gmask = gmask;
  m->plan = plan;
  m->order = order;
  *out = m;
  return TR_SC_OK;
}

void tr_sparseconv_kmap_destroy(tr_sc_kmap* m) {
  if (m != nullptr && m->magic == kKmapMagic) {
    m->magic = 0;
    delete m;
  }
}

size_t tr_sparseconv_packed_weights_bytes(int c_in, int c_out, int dtype) {
  if (c_in <= 0 || c_out <= 0) return 0;
  const size_t elems = size_t(27) * size_t(c_in) * size_t(c_out);
  if (dtype == TR_SC_BF16 || dtype == TR_SC_F16)
    return size_t(packed_half_bytes(c_in, c_out));  // + zero block (+ fragment-order copy)
  if (dtype == TR_SC_F32) return align_up(elems * 4, 256);
  return 0;
}

size_t tr_sparseconv_forward_workspace_bytes(int c_in, int c_out, int dtype) {
  if (dtype == TR_SC_F32) return 0;  // the fp32 path reads w in place
  return tr_sparseconv_packed_weights_bytes(c_in, c_out, dtype);
}

namespace {

bool is_half(int dtype) { return dtype == TR_SC_BF16 || dtype == TR_SC_F16; }

int check_channels(const char* who, int c_in, int c_out, int dtype) {
  if (c_in <= 0 || c_out <= 0) return fail(TR_SC_ERR_INVALID_ARG, "%s: c_in = %d, c_out = %d", who, c_in, c_out);
  if (dtype != TR_SC_F32 && !is_half(dtype)) return fail(TR_SC_ERR_UNSUPPORTED, "%s: dtype %d", who, dtype);
  if (is_half(dtype) && (c_in % 8 != 0 || c_out % 8 != 0))
    return fail(TR_SC_ERR_UNSUPPORTED, "%s: half precision needs c_in and c_out multiples of 8 (got %d, %d)", who,
                c_in, c_out);
  return TR_SC_OK;
}

bool misaligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 != 0; }

// Launches the gather-GEMM of an already validated call.
int run_forward(const char* who, const tr_sc_kmap* m, const void* x, int x_dtype, const void* wp, int w_dtype,
                void* y, int y_dtype, const Epilogue& epi, int c_in, int c_out, hipStream_t st) {
  if (x == nullptr || wp == nullptr || y == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "%s: NULL tensor", who);
  if (x == y) return fail(TR_SC_ERR_INVALID_ARG, "%s: x and y are the same buffer", who);
  if (int64_t(m->n) * c_out >= (int64_t(1) << 40) || int64_t(m->n) * c_in >= (int64_t(1) << 40))
    return fail(TR_SC_ERR_UNSUPPORTED, "%s: tensor too large", who);
  ConvArgs a{m->nbr, m->grows, m->gmask, m->plan, m->order, m->n, x, wp, y, c_in, c_out, x_dtype, w_dtype, y_dtype, epi};
  hipError_t e;
  if (w_dtype == TR_SC_F32) {
    e = launch_forward_simple_f32(a, st);
  } else {
    if (misaligned16(x) || misaligned16(y) || misaligned16(wp) || misaligned16(epi.residual))
      return fail(TR_SC_ERR_INVALID_ARG, "%s: x, y, residual and packed weights must be 16-byte aligned", who);
    e = launch_forward_mfma(a, wp, st);
  }
  if (e != hipSuccess) return hip_fail(e, who);
  return TR_SC_OK;
}

}  // namespace

int tr_sparseconv_pack_weights(const void* w, int c_in, int c_out, int dtype, void* wp, size_t wp_bytes,
                               void* stream) {
  const int c = check_channels("pack_weights", c_in, c_out, dtype);
  if (c != TR_SC_OK) return c;
  if (w == nullptr || wp == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "pack_weights: NULL pointer");
  const size_t need = tr_sparseconv_packed_weights_bytes(c_in, c_out, dtype);
  if (wp_bytes < need) return fail(TR_SC_ERR_WORKSPACE, "pack_weights: %zu bytes < %zu needed", wp_bytes, need);
  if (misaligned16(wp)) return fail(TR_SC_ERR_INVALID_ARG, "pack_weights: wp not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (is_half(dtype))
    e = launch_pack_weights(w, wp, c_in, c_out, st);
  else
    e = hipMemcpyAsync(wp, w, size_t(27) * c_in * c_out * 4, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "pack_weights");
  return TR_SC_OK;
}

int tr_sparseconv_forward_packed(const tr_sc_kmap* m, const void* x, const void* wp, void* y, int c_in,
                                 int c_out, int dtype, void* stream) {
  if (m == nullptr || m->magic != kKmapMagic)
    return fail(TR_SC_ERR_INVALID_ARG, "forward_packed: bad kernel-map handle");
  const int c = check_channels("forward_packed", c_in, c_out, dtype);
  if (c != TR_SC_OK) return c;
  if (m->n == 0) return TR_SC_OK;
  return run_forward("forward_packed", m, x, dtype, wp, dtype, y, dtype, Epilogue{nullptr, nullptr, kActNone},
                     c_in, c_out, static_cast<hipStream_t>(stream));
}

int tr_sparseconv_forward(const tr_sc_kmap* m, const void* x, const void* w, void* y, int c_in, int c_out,
                          int dtype, void* workspace, size_t ws_bytes, void* stream) {
  if (m == nullptr || m->magic != kKmapMagic) return fail(TR_SC_ERR_INVALID_ARG, "forward: bad kernel-map handle");
  const int c = check_channels("forward", c_in, c_out, dtype);
  if (c != TR_SC_OK) return c;
  const size_t need = tr_sparseconv_forward_workspace_bytes(c_in, c_out, dtype);
  if (ws_bytes < need) return fail(TR_SC_ERR_WORKSPACE, "forward: workspace %zu bytes < %zu needed", ws_bytes, need);
  if (need > 0 && workspace == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "forward: workspace is NULL");
  if (m->n == 0) return TR_SC_OK;
  if (w == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "forward: NULL tensor");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Epilogue none{nullptr, nullptr, kActNone};
  if (dtype == TR_SC_F32) return run_forward("forward", m, x, dtype, w, dtype, y, dtype, none, c_in, c_out, st);
  if (misaligned16(workspace)) return fail(TR_SC_ERR_INVALID_ARG, "forward: workspace not 16-byte aligned");
  hipError_t e = launch_pack_weights(w, workspace, c_in, c_out, st);
  if (e != hipSuccess) return hip_fail(e, "forward: pack");
  return run_forward("forward", m, x, dtype, workspace, dtype, y, dtype, none, c_in, c_out, st);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// tr_sparseconv_forward without a workspace argument and without allocating:
// the packed weights go to `scratch`, a file-scope device array. Each GPU the
// library runs on holds its own copy of the array (at its own address) until
// the process ends. In host code the array's name is only a stand-in: the
// device address of the current GPU's copy is resolved once per device with
// hipGetSymbolAddress and kept in g_scratch_ptr; only that address is passed to
// kernels. Calls on one GPU share its copy: calls that overlap in time on one
// GPU (two streams, two threads) race on it.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];

// Device address of the current device's copy of `scratch`, resolved on the
// first call on that device, with that device current.
hipError_t scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace

extern "C" {

int tr_sparseconv_forward_noalloc(const tr_sc_kmap* m, const void* x, const void* w, void* y, int c_in,
                                  int c_out, int dtype, void* stream) {
  if (m == nullptr || m->magic != kKmapMagic)
    return fail(TR_SC_ERR_INVALID_ARG, "forward_noalloc: bad kernel-map handle");
  const int c = check_channels("forward_noalloc", c_in, c_out, dtype);
  if (c != TR_SC_OK) return c;
  const size_t need = tr_sparseconv_forward_workspace_bytes(c_in, c_out, dtype);
  if (need > kNoAllocScratchBytes)
    return fail(TR_SC_ERR_WORKSPACE,
                "forward_noalloc: packed weights of %zu bytes exceed the %zu-byte scratch array "
                "(the packed weights, tr_sparseconv_packed_weights_bytes, must fit)",
                need, kNoAllocScratchBytes);
  if (m->n == 0) return TR_SC_OK;
  if (w == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "forward_noalloc: NULL tensor");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Epilogue none{nullptr, nullptr, kActNone};
  if (dtype == TR_SC_F32)  // the fp32 path reads w in place: no scratch
    return run_forward("forward_noalloc", m, x, dtype, w, dtype, y, dtype, none, c_in, c_out, st);
  void* wp = nullptr;
  hipError_t e = scratch_of_current_device(&wp);
  if (e != hipSuccess) return hip_fail(e, "forward_noalloc: scratch address");
  e = launch_pack_weights(w, wp, c_in, c_out, st);
  if (e != hipSuccess) return hip_fail(e, "forward_noalloc: pack");
  return run_forward("forward_noalloc", m, x, dtype, wp, dtype, y, dtype, none, c_in, c_out, st);
}

int tr_sparseconv_forward_fused(const tr_sc_kmap* m, const void* x, int x_dtype, const void* wp, int w_dtype,
                                const float* bias, int act, const void* residual, void* y, int y_dtype,
                                int c_in, int c_out, void* stream) {
  if (m == nullptr || m->magic != kKmapMagic)
    return fail(TR_SC_ERR_INVALID_ARG, "forward_fused: bad kernel-map handle");
  const int c = check_channels("forward_fused", c_in, c_out, w_dtype);
  if (c != TR_SC_OK) return c;
  if (act != TR_SC_ACT_NONE && act != TR_SC_ACT_RELU && act != TR_SC_ACT_SILU)
    return fail(TR_SC_ERR_INVALID_ARG, "forward_fused: activation %d", act);
  const bool ok_types = w_dtype == TR_SC_F32
                            ? (x_dtype == TR_SC_F32 && y_dtype == TR_SC_F32)
                            : ((x_dtype == w_dtype || x_dtype == TR_SC_F32) &&
                               (y_dtype == w_dtype || y_dtype == TR_SC_F32));
  if (!ok_types)
    return fail(TR_SC_ERR_UNSUPPORTED, "forward_fused: x dtype %d, weight dtype %d, y dtype %d", x_dtype, w_dtype,
                y_dtype);
  if (m->n == 0) return TR_SC_OK;
  if (x == y) return fail(TR_SC_ERR_INVALID_ARG, "forward_fused: x and y are the same buffer");
  return run_forward("forward_fused", m, x, x_dtype, wp, w_dtype, y, y_dtype, Epilogue{bias, residual, act}, c_in,
                     c_out, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// Backward.
// ---------------------------------------------------------------------------
int tr_sparseconv_pack_weights_dgrad(const void* w, int c_in, int c_out, int dtype, void* wp, size_t wp_bytes,
                                     void* stream) {
  const int c = check_channels("pack_weights_dgrad", c_in, c_out, dtype);
  if (c != TR_SC_OK) return c;
  if (w == nullptr || wp == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "pack_weights_dgrad: NULL pointer");
  const size_t need = tr_sparseconv_packed_weights_bytes(c_out, c_in, dtype);
  if (wp_bytes < need)
    return fail(TR_SC_ERR_WORKSPACE, "pack_weights_dgrad: %zu bytes < %zu needed", wp_bytes, need);
  if (misaligned16(wp) || (is_half(dtype) && misaligned16(w)))
    return fail(TR_SC_ERR_INVALID_ARG, "pack_weights_dgrad: w and wp must be 16-byte aligned");
  const hipError_t e = launch_pack_dgrad(w, wp, c_in, c_out, dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pack_weights_dgrad");
  return TR_SC_OK;
}

int tr_sparseconv_backward_data(const tr_sc_kmap* m, const void* dy, int dy_dtype, const void* wpd, int w_dtype,
                                void* dx, int dx_dtype, int c_in, int c_out, void* stream) {
  if (m == nullptr || m->magic != kKmapMagic)
    return fail(TR_SC_ERR_INVALID_ARG, "backward_data: bad kernel-map handle");
  const int c = check_channels("backward_data", c_in, c_out, w_dtype);
  if (c != TR_SC_OK) return c;
  const bool ok_types = w_dtype == TR_SC_F32
                            ? (dy_dtype == TR_SC_F32 && dx_dtype == TR_SC_F32)
                            : ((dy_dtype == w_dtype || dy_dtype == TR_SC_F32) &&
                               (dx_dtype == w_dtype || dx_dtype == TR_SC_F32));
  if (!ok_types)
    return fail(TR_SC_ERR_UNSUPPORTED, "backward_data: dy dtype %d, weight dtype %d, dx dtype %d", dy_dtype,
                w_dtype, dx_dtype);
  if (m->n == 0) return TR_SC_OK;
  if (dy == dx) return fail(TR_SC_ERR_INVALID_ARG, "backward_data: dy and dx are the same buffer");
  // the forward gather-GEMM of the c_out -> c_in convolution with the mirrored taps
  return run_forward("backward_data", m, dy, dy_dtype, wpd, w_dtype, dx, dx_dtype,
                     Epilogue{nullptr, nullptr, kActNone}, c_out, c_in, static_cast<hipStream_t>(stream));
}

size_t tr_sparseconv_backward_weights_workspace_bytes(int64_t n, int c_in, int c_out, int dtype) {
  if (n < 0 || c_in <= 0 || c_out <= 0) return 0;
  if (dtype == TR_SC_F32) return 0;
  return 256 + align_up(plan_wgrad(n, c_in, c_out).partial_bytes, 256);
}

int tr_sparseconv_backward_weights(const tr_sc_kmap* m, const void* x, const void* dy, float* dw, int c_in,
                                   int c_out, int dtype, void* workspace, size_t ws_bytes, void* stream) {
  if (m == nullptr || m->magic != kKmapMagic)
    return fail(TR_SC_ERR_INVALID_ARG, "backward_weights: bad kernel-map handle");
  const int c = check_channels("backward_weights", c_in, c_out, dtype);
  if (c != TR_SC_OK) return c;
  const size_t need = tr_sparseconv_backward_weights_workspace_bytes(m->n, c_in, c_out, dtype);
  if (ws_bytes < need)
    return fail(TR_SC_ERR_WORKSPACE, "backward_weights: workspace %zu bytes < %zu needed", ws_bytes, need);
  if (need > 0 && (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
    return fail(TR_SC_ERR_INVALID_ARG, "backward_weights: workspace NULL or not 256-byte aligned");
  if (dw == nullptr || (m->n > 0 && (x == nullptr || dy == nullptr)))
    return fail(TR_SC_ERR_INVALID_ARG, "backward_weights: NULL tensor");
  if (is_half(dtype) && (misaligned16(x) || misaligned16(dy) || misaligned16(dw)))
    return fail(TR_SC_ERR_INVALID_ARG, "backward_weights: x, dy and dw must be 16-byte aligned");
  if (int64_t(m->n) * c_out >= (int64_t(1) << 40) || int64_t(m->n) * c_in >= (int64_t(1) << 40))
    return fail(TR_SC_ERR_UNSUPPORTED, "backward_weights: tensor too large");
  char* ws = static_cast<char*>(workspace);
  WgradCall call{m->nbr, m->grows, m->gmask, m->n, x, dy, dw,
                 need > 0 ? reinterpret_cast<float*>(ws + 256) : nullptr, ws, c_in, c_out, dtype};
  const hipError_t e = launch_wgrad(call, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "backward_weights");
  return TR_SC_OK;
}

// ---------------------------------------------------------------------------
// Resolution levels.
// ---------------------------------------------------------------------------
namespace {

struct LevelHeader {
  int64_t total;
  uint32_t flags;
  uint32_t pad;
};

__global__ void level_header_init(LevelHeader* h) {
  if (threadIdx.x == 0) {
    h->total = 0;
    h->flags = 0;
  }
}

// Reads the produced count (and flags) back; waits for `st`.
int level_readback(const char* who, LevelHeader* dh, int64_t cap, hipStream_t st, int64_t* count) {
  LevelHeader host{};
  hipError_t e = hipMemcpyAsync(&host, dh, sizeof(host), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, who);
  *count = host.total;
  if (host.flags & kFlagCoordRange)
    return fail(TR_SC_ERR_COORD_RANGE, "%s: a coordinate component is negative or its children leave [0, 65536)",
                who);
  if (host.total > cap)
    return fail(TR_SC_ERR_CAPACITY, "%s: %lld rows produced, capacity %lld", who, (long long)host.total,
                (long long)cap);
  return TR_SC_OK;
}

}  // namespace

size_t tr_sparseconv_level_workspace_bytes(int64_t n) {
  if (n < 0) return 0;
  return 256 + align_up(size_t(level_blocks(n)) * 8, 256);
}

int tr_sparseconv_downsample(const tr_sc_hash* h, int32_t* coarse_coords, int32_t* children, int64_t cap,
                             void* workspace, size_t ws_bytes, void* stream, int64_t* n_coarse) {
  if (h == nullptr || h->magic != kHashMagic) return fail(TR_SC_ERR_INVALID_ARG, "downsample: bad hash handle");
  if (n_coarse == nullptr || cap < 0) return fail(TR_SC_ERR_INVALID_ARG, "downsample: bad output arguments");
  *n_coarse = 0;
  const size_t need = tr_sparseconv_level_workspace_bytes(h->n);
  if (ws_bytes < need) return fail(TR_SC_ERR_WORKSPACE, "downsample: workspace %zu bytes < %zu", ws_bytes, need);
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TR_SC_ERR_INVALID_ARG, "downsample: workspace NULL or not 256-byte aligned");
  if (cap > 0 && (coarse_coords == nullptr || children == nullptr || misaligned16(coarse_coords) ||
                  misaligned16(children)))
    return fail(TR_SC_ERR_INVALID_ARG, "downsample: outputs NULL or not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  LevelHeader* dh = static_cast<LevelHeader*>(workspace);
  int64_t* part = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + 256);
  level_header_init<<<1, 64, 0, st>>>(dh);
  hipError_t e = launch_downsample(h->skeys, h->table.srows, h->n, cap, part, &dh->total, coarse_coords, children,
                                   st);
  if (e != hipSuccess) return hip_fail(e, "downsample");
  return level_readback("downsample", dh, cap, st, n_coarse);
}

int tr_sparseconv_subdivide(const int32_t* coords, int64_t n, const uint8_t* keep, int32_t* fine_coords,
                            int32_t* children, int64_t cap, void* workspace, size_t ws_bytes, void* stream,
                            int64_t* n_fine) {
  if (n_fine == nullptr || n < 0 || cap < 0 || n > kMaxN)
    return fail(TR_SC_ERR_INVALID_ARG, "subdivide: bad sizes or output count pointer");
  *n_fine = 0;
  const size_t need = tr_sparseconv_level_workspace_bytes(n);
  if (ws_bytes < need) return fail(TR_SC_ERR_WORKSPACE, "subdivide: workspace %zu bytes < %zu", ws_bytes, need);
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TR_SC_ERR_INVALID_ARG, "subdivide: workspace NULL or not 256-byte aligned");
  if (n > 0 && (coords == nullptr || children == nullptr || misaligned16(coords) || misaligned16(children)))
    return fail(TR_SC_ERR_INVALID_ARG, "subdivide: coords / children NULL or not 16-byte aligned");
  if (cap > 0 && (fine_coords == nullptr || misaligned16(fine_coords)))
    return fail(TR_SC_ERR_INVALID_ARG, "subdivide: fine_coords NULL or not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  LevelHeader* dh = static_cast<LevelHeader*>(workspace);
  int64_t* part = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + 256);
  level_header_init<<<1, 64, 0, st>>>(dh);
  hipError_t e = launch_subdivide(coords, keep, n, cap, part, &dh->total, &dh->flags, fine_coords, children, st);
  if (e != hipSuccess) return hip_fail(e, "subdivide");
  return level_readback("subdivide", dh, cap, st, n_fine);
}

namespace {
int regroup_call(const char* who, const int32_t* children, int64_t n_coarse, const void* src, void* dst,
                 int c_fine, int dtype, bool to_fine, void* stream) {
  if (n_coarse < 0 || c_fine <= 0) return fail(TR_SC_ERR_INVALID_ARG, "%s: n_coarse %lld, c_fine %d", who,
                                                (long long)n_coarse, c_fine);
  if (dtype != TR_SC_F32 && !is_half(dtype)) return fail(TR_SC_ERR_UNSUPPORTED, "%s: dtype %d", who, dtype);
  const int v = dtype == TR_SC_F32 ? 4 : 8;
  if (c_fine % v != 0)
    return fail(TR_SC_ERR_UNSUPPORTED, "%s: c_fine must be a multiple of %d for this dtype", who, v);
  if (n_coarse == 0) return TR_SC_OK;
  if (children == nullptr || src == nullptr || dst == nullptr) return fail(TR_SC_ERR_INVALID_ARG, "%s: NULL", who);
  if (misaligned16(children) || misaligned16(src) || misaligned16(dst))
    return fail(TR_SC_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", who);
  void* xc = to_fine ? const_cast<void*>(src) : dst;
  void* xf = to_fine ? dst : const_cast<void*>(src);
  const hipError_t e = launch_regroup(children, n_coarse, xc, xf, c_fine, dtype == TR_SC_F32 ? 4 : 2, to_fine,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, who);
  return TR_SC_OK;
}
}  // namespace

int tr_sparseconv_channel2spatial(const int32_t* children, int64_t n_coarse, const void* x_coarse, void* x_fine,
                                  int c_fine, int dtype, void* stream) {
  return regroup_call("channel2spatial", children, n_coarse, x_coarse, x_fine, c_fine, dtype, true, stream);
}

int tr_sparseconv_spatial2channel(const int32_t* children, int64_t n_coarse, const void* x_fine, void* x_coarse,
                                  int c_fine, int dtype, void* stream) {
  return regroup_call("spatial2channel", children, n_coarse, x_fine, x_coarse, c_fine, dtype, false, stream);
}

}  // extern "C"
