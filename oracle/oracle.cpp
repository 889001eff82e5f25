// CPU oracle for the submanifold sparse 3D convolution.
//
// TEST INFRASTRUCTURE. Only the tests, the package entry's smoke check and the
// benchmark's CPU-baseline leg load this code. It is deliberately plain and slow,
// and it shares no code, header, table or constant with the HIP library.
//
// What it computes, and where the pages define it:
//   * The operator: a spatial hash of the active voxels; for every kernel
//     position the neighbour features are gathered, multiplied by that
//     position's weights and added into the output of the voxel -- "Running
//     TRELLIS.2 on a Mac (1/3)", section "Swapping out the CUDA libraries one at
//     a time", sparse 3D convolution paragraph. The same sum as a gather-GEMM over
//     a neighbour table built once per resolution level -- "Porting TRELLIS.2
//     From Python to Rust and Metal", section V.
//   * Output only at active sites ("submanifold"; features stay sparse) --
//     mlx-diffuser TRELLIS guide, section "Why it fits better on a Mac".
//   * Coordinates are (b, x, y, z) integer rows; features are [N, C] rows --
//     startup packet (page 5), section 5, parity fixture table, rows B-D.
//   * Weights are tap-major [Kvol = 27, C_in, C_out], reshaped from the on-disk
//     (C_out, Kd, Kh, Kw, C_in) layout, so tap k = 9*Kd + 3*Kh + Kw -- startup
//     packet, section 5 (conv conventions table and notes) and section 8.
//
// Readings where the pages are silent (each also listed in the design notes):
//   * Kd, Kh, Kw run along x, y, z in the order the coordinates list them, and
//     tap (Kd, Kh, Kw) reads the voxel at (x + Kd - 1, y + Kh - 1, z + Kw - 1):
//     cross-correlation, the same as a dense 3x3x3 convolution with zero padding
//     of 1 evaluated at the active sites. Agreement with TRELLIS's own sign
//     convention is "parity unpinned": no TRELLIS layer or fixture is available.
//   * Neighbours exist only inside the same batch index b; a neighbour outside
//     [0, 2^16) on any axis does not exist (zero padding).
//   * Every coordinate component must lie in [0, 2^16); a repeated coordinate
//     is an error (a sparse tensor's coordinates form a set).
//
// Arithmetic: inputs are widened exactly to double by the caller; every output
// y[i, co] = sum over k = 0..26 with nbr[i][k] >= 0, then over ci = 0..C_in-1,
// of W[k, ci, co] * x[nbr[i][k], ci], accumulated in double in exactly that
// (k, ci) order and never rounded.
#include <algorithm>
#include <array>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

constexpr int kOk = 0;
constexpr int kErrInvalid = -1;
constexpr int kErrCoordRange = -2;
constexpr int kErrDuplicate = -3;

constexpr int64_t kAxisLimit = int64_t(1) << 16;

// Plain positional packing of (b, x, y, z), 16 bits each.
inline uint64_t pack_key(int64_t b, int64_t x, int64_t y, int64_t z) {
  return (((uint64_t(b) * kAxisLimit + uint64_t(x)) * kAxisLimit + uint64_t(y)) * kAxisLimit) +
         uint64_t(z);
}

inline bool in_range(int64_t v) { return v >= 0 && v < kAxisLimit; }

struct Table {
  std::unordered_map<uint64_t, int32_t> map;
  std::vector<int32_t> coords;  // copy of the caller's [n, 4] rows
  int64_t n = 0;
};

// Tap k -> offset (dx, dy, dz), each in {-1, 0, 1}.
inline void tap_offset(int k, int& dx, int& dy, int& dz) {
  dx = k / 9 - 1;
  dy = (k / 3) % 3 - 1;
  dz = k % 3 - 1;
}

}  // namespace

extern "C" {

// Builds the coordinate -> row map, inserting rows in caller order. Returns 0,
// -2 for a component outside [0, 2^16), -3 for a repeated coordinate, -1 for
// bad arguments. On success *out receives a handle for oc_free.
int oc_build(const int32_t* coords, int64_t n, void** out) {
  if (out == nullptr || n < 0 || (n > 0 && coords == nullptr) || n > INT32_MAX) return kErrInvalid;
  *out = nullptr;
  Table* t = new Table;
  t->n = n;
  t->coords.assign(coords, coords + 4 * n);
  t->map.reserve(size_t(n) * 2 + 1);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t* c = coords + 4 * i;
    if (!in_range(c[0]) || !in_range(c[1]) || !in_range(c[2]) || !in_range(c[3])) {
      delete t;
      return kErrCoordRange;
    }
    auto ins = t->map.emplace(pack_key(c[0], c[1], c[2], c[3]), int32_t(i));
    if (!ins.second) {
      delete t;
      return kErrDuplicate;
    }
  }
  *out = t;
  return kOk;
}

void oc_free(void* h) { delete static_cast<Table*>(h); }

// idx[q] = row of query coordinate q, or -1 if it is not active (including
// queries with a component outside [0, 2^16)).
int oc_lookup(const void* h, const int32_t* q, int64_t nq, int32_t* idx) {
  const Table* t = static_cast<const Table*>(h);
  if (t == nullptr || nq < 0 || (nq > 0 && (q == nullptr || idx == nullptr))) return kErrInvalid;
  for (int64_t i = 0; i < nq; ++i) {
    const int32_t* c = q + 4 * i;
    int32_t r = -1;
    if (in_range(c[0]) && in_range(c[1]) && in_range(c[2]) && in_range(c[3])) {
      auto it = t->map.find(pack_key(c[0], c[1], c[2], c[3]));
      if (it != t->map.end()) r = it->second;
    }
    idx[i] = r;
  }
  return kOk;
}

// nbr[i * 27 + k] = row of the voxel at (b_i, x_i + dx_k, y_i + dy_k, z_i + dz_k),
// or -1 when that voxel is not active or lies outside [0, 2^16).
int oc_kernel_map(const void* h, int32_t* nbr) {
  const Table* t = static_cast<const Table*>(h);
  if (t == nullptr || (t->n > 0 && nbr == nullptr)) return kErrInvalid;
  const int64_t n = t->n;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const int32_t* c = t->coords.data() + 4 * i;
    for (int k = 0; k < 27; ++k) {
      int dx, dy, dz;
      tap_offset(k, dx, dy, dz);
      const int64_t x = int64_t(c[1]) + dx, y = int64_t(c[2]) + dy, z = int64_t(c[3]) + dz;
      int32_t r = -1;
      if (in_range(x) && in_range(y) && in_range(z)) {
        auto it = t->map.find(pack_key(c[0], x, y, z));
        if (it != t->map.end()) r = it->second;
      }
      nbr[i * 27 + k] = r;
    }
  }
  return kOk;
}

// y[r, co] for each requested row r (rows == NULL: every row 0..n-1, and y is
// [n, c_out]; otherwise y is [nrows, c_out] in the order of `rows`).
// x is [n, c_in] and w is [27, c_in, c_out], both double, row-major.
int oc_forward(const int32_t* nbr, int64_t n, const int64_t* rows, int64_t nrows,
               const double* x, const double* w, int c_in, int c_out, double* y) {
  if (n < 0 || c_in <= 0 || c_out <= 0) return kErrInvalid;
  const int64_t m = rows ? nrows : n;
  if (m < 0) return kErrInvalid;
  if (m > 0 && (nbr == nullptr || x == nullptr || w == nullptr || y == nullptr)) return kErrInvalid;
  for (int64_t q = 0; q < (rows ? nrows : 0); ++q)
    if (rows[q] < 0 || rows[q] >= n) return kErrInvalid;
#pragma omp parallel
  {
    std::vector<double> acc(static_cast<size_t>(c_out));
#pragma omp for schedule(dynamic, 64)
    for (int64_t q = 0; q < m; ++q) {
      const int64_t i = rows ? rows[q] : q;
      std::fill(acc.begin(), acc.end(), 0.0);
      for (int k = 0; k < 27; ++k) {
        const int32_t j = nbr[i * 27 + k];
        if (j < 0) continue;
        const double* xr = x + int64_t(j) * c_in;
        const double* wk = w + int64_t(k) * c_in * c_out;
        for (int ci = 0; ci < c_in; ++ci) {
          const double xv = xr[ci];
          const double* wr = wk + int64_t(ci) * c_out;
          for (int co = 0; co < c_out; ++co) acc[size_t(co)] += wr[co] * xv;
        }
      }
      std::memcpy(y + q * c_out, acc.data(), sizeof(double) * size_t(c_out));
    }
  }
  return kOk;
}

// The fused epilogue of the gather-GEMM: the pages fuse the bias, the
// activation, the residual add and the output rounding into the convolution
// pass ("Porting TRELLIS.2 ...", section V). Reading: out = act(y + bias) +
// residual, rounded once at the end (here: never, fp64). act: 0 none, 1 ReLU max(v, 0),
// 2 SiLU v / (1 + exp(-v)). bias is [c_out] or NULL; residual is [m, c_out]
// (the rows of y, in the same order) or NULL. Applied in place on y [m, c_out].
int oc_epilogue(double* y, int64_t m, int c_out, const double* bias, const double* residual, int act) {
  if (m < 0 || c_out <= 0 || act < 0 || act > 2) return kErrInvalid;
  if (m > 0 && y == nullptr) return kErrInvalid;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i) {
    for (int co = 0; co < c_out; ++co) {
      double v = y[i * c_out + co];
      if (bias) v += bias[co];
      if (act == 1) v = v > 0.0 ? v : 0.0;
      if (act == 2) v = v / (1.0 + std::exp(-v));
      if (residual) v += residual[i * c_out + co];
      y[i * c_out + co] = v;
    }
  }
  return kOk;
}

// Backward of the convolution (the gradients of L = sum_i <y[i], dy[i]>),
// written from the forward sum above: every term w[k, ci, co] * x[j, ci] with
// j = nbr[i][k] >= 0 contributes
//   dx[j, ci]     += w[k, ci, co] * dy[i, co]     (data gradient)
//   dw[k, ci, co] += x[j, ci]     * dy[i, co]     (weight gradient).
//
// Data gradient, for the output rows `rows` (all rows if NULL): the terms that
// land on row j are found by a full scan of nbr for entries equal to j (the
// inverse of the map, built here from nbr alone), then summed in (i, k, co)
// order in fp64.
int oc_backward_data(const int32_t* nbr, int64_t n, const int64_t* rows, int64_t nrows,
                     const double* dy, const double* w, int c_in, int c_out, double* dx) {
  if (n < 0 || c_in <= 0 || c_out <= 0) return kErrInvalid;
  const int64_t m = rows ? nrows : n;
  if (m < 0) return kErrInvalid;
  if (m > 0 && (nbr == nullptr || dy == nullptr || w == nullptr || dx == nullptr)) return kErrInvalid;
  for (int64_t q = 0; q < (rows ? nrows : 0); ++q)
    if (rows[q] < 0 || rows[q] >= n) return kErrInvalid;
  // inverse map in CSR form: for each j, the (i, k) with nbr[i][k] == j, by i then k
  std::vector<int64_t> start(size_t(n) + 1, 0);
  for (int64_t e = 0; e < n * 27; ++e) {
    const int32_t j = nbr[e];
    if (j < -1 || j >= n) return kErrInvalid;
    if (j >= 0) ++start[size_t(j) + 1];
  }
  for (int64_t j = 0; j < n; ++j) start[size_t(j) + 1] += start[size_t(j)];
  std::vector<int64_t> fill(start.begin(), start.end() - 1);
  std::vector<int64_t> src(size_t(start[size_t(n)]));
  for (int64_t e = 0; e < n * 27; ++e)
    if (nbr[e] >= 0) src[size_t(fill[size_t(nbr[e])]++)] = e;  // e = i * 27 + k
#pragma omp parallel
  {
    std::vector<double> acc(static_cast<size_t>(c_in));
#pragma omp for schedule(dynamic, 64)
    for (int64_t q = 0; q < m; ++q) {
      const int64_t j = rows ? rows[q] : q;
      std::fill(acc.begin(), acc.end(), 0.0);
      for (int64_t t = start[size_t(j)]; t < start[size_t(j) + 1]; ++t) {
        const int64_t i = src[size_t(t)] / 27;
        const int k = int(src[size_t(t)] % 27);
        const double* g = dy + i * c_out;
        const double* wk = w + int64_t(k) * c_in * c_out;
        for (int ci = 0; ci < c_in; ++ci) {
          double sacc = 0.0;
          for (int co = 0; co < c_out; ++co) sacc += wk[int64_t(ci) * c_out + co] * g[co];
          acc[size_t(ci)] += sacc;
        }
      }
      std::memcpy(dx + q * c_in, acc.data(), sizeof(double) * size_t(c_in));
    }
  }
  return kOk;
}

// Weight gradient, for the (tap, input channel) entries listed in sel (pairs
// k, ci; all 27 * c_in in (k, ci) order if NULL): dw_sel[s, co] = sum over i
// with nbr[i][k] = j >= 0, in order of i, of x[j, ci] * dy[i, co], in fp64.
int oc_backward_weights(const int32_t* nbr, int64_t n, const double* x, const double* dy, int c_in,
                        int c_out, const int32_t* sel, int64_t nsel, double* dw) {
  if (n < 0 || c_in <= 0 || c_out <= 0) return kErrInvalid;
  const int64_t m = sel ? nsel : int64_t(27) * c_in;
  if (m < 0 || (m > 0 && dw == nullptr) || (n > 0 && (nbr == nullptr || x == nullptr || dy == nullptr)))
    return kErrInvalid;
  for (int64_t s = 0; s < (sel ? nsel : 0); ++s)
    if (sel[2 * s] < 0 || sel[2 * s] > 26 || sel[2 * s + 1] < 0 || sel[2 * s + 1] >= c_in) return kErrInvalid;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t s = 0; s < m; ++s) {
    const int k = sel ? sel[2 * s] : int(s / c_in);
    const int ci = sel ? sel[2 * s + 1] : int(s % c_in);
    double* out = dw + s * c_out;
    std::fill(out, out + c_out, 0.0);
    for (int64_t i = 0; i < n; ++i) {
      const int32_t j = nbr[i * 27 + k];
      if (j < 0) continue;
      const double xv = x[int64_t(j) * c_in + ci];
      const double* g = dy + i * c_out;
      for (int co = 0; co < c_out; ++co) out[co] += xv * g[co];
    }
  }
  return kOk;
}

// ---------------------------------------------------------------------------
// Moving between resolution levels. The pages build one neighbour table per
// resolution level ("Porting TRELLIS.2 ...", section V); their decoders change
// level with pixel-shuffle / Channel2Spatial upsampling driven by subdivision
// predictions (TRELLIS.2 MLX port README, repository tree and pipeline list).
// Readings (listed in the design notes): the parent of (b, x, y, z) is
// (b, x >> 1, y >> 1, z >> 1); the children of (b, x, y, z) are
// (b, 2x + dx, 2y + dy, 2z + dz) with octant o = 4 dx + 2 dy + dz; a parent
// row of 8C channels holds child o's channel c at c * 8 + o (the channel order
// of a pixel shuffle).
// ---------------------------------------------------------------------------

// Z-order rank of (x, y, z): bit i of x, y, z at bits 3i + 2, 3i + 1, 3i.
static uint64_t zorder(uint32_t x, uint32_t y, uint32_t z) {
  uint64_t key = 0;
  for (int i = 0; i < 16; ++i) {
    key |= uint64_t((x >> i) & 1u) << (3 * i + 2);
    key |= uint64_t((y >> i) & 1u) << (3 * i + 1);
    key |= uint64_t((z >> i) & 1u) << (3 * i);
  }
  return key;
}

// Coarser level: the set of parents, ordered by batch index, then Z-order of
// (x, y, z); children[q * 8 + o] = the row of child o of parent q, or -1.
int oc_downsample(const int32_t* coords, int64_t n, int32_t* coarse, int32_t* children, int64_t* n_coarse) {
  if (n < 0 || n_coarse == nullptr || (n > 0 && (coords == nullptr || coarse == nullptr || children == nullptr)))
    return kErrInvalid;
  std::unordered_map<uint64_t, int64_t> parent;  // packed parent coordinate -> index in `order`
  std::vector<std::array<int32_t, 4>> order;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t* c = coords + 4 * i;
    if (!in_range(c[0]) || !in_range(c[1]) || !in_range(c[2]) || !in_range(c[3])) return kErrCoordRange;
    const std::array<int32_t, 4> pc{c[0], c[1] >> 1, c[2] >> 1, c[3] >> 1};
    if (parent.emplace(pack_key(pc[0], pc[1], pc[2], pc[3]), int64_t(order.size())).second) order.push_back(pc);
  }
  std::vector<int64_t> rank(order.size());
  for (size_t q = 0; q < order.size(); ++q) rank[q] = int64_t(q);
  std::sort(rank.begin(), rank.end(), [&](int64_t a, int64_t b) {
    const auto& A = order[size_t(a)];
    const auto& B = order[size_t(b)];
    if (A[0] != B[0]) return A[0] < B[0];
    return zorder(uint32_t(A[1]), uint32_t(A[2]), uint32_t(A[3])) <
           zorder(uint32_t(B[1]), uint32_t(B[2]), uint32_t(B[3]));
  });
  std::vector<int64_t> pos(order.size());
  for (size_t r = 0; r < rank.size(); ++r) pos[size_t(rank[r])] = int64_t(r);
  const int64_t m = int64_t(order.size());
  for (int64_t q = 0; q < m; ++q)
    for (int e = 0; e < 4; ++e) coarse[4 * pos[size_t(q)] + e] = order[size_t(q)][size_t(e)];
  std::fill(children, children + 8 * m, -1);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t* c = coords + 4 * i;
    const int64_t q = pos[size_t(parent.at(pack_key(c[0], c[1] >> 1, c[2] >> 1, c[3] >> 1)))];
    const int o = 4 * (c[1] & 1) + 2 * (c[2] & 1) + (c[3] & 1);
    children[8 * q + o] = int32_t(i);
  }
  *n_coarse = m;
  return kOk;
}

// Finer level: for each row i in order and octant o = 0..7 with bit o of
// keep[i] set (all 8 if keep is NULL), the next fine row is child o of i.
// children[i * 8 + o] = that fine row, or -1. Fine coordinates must stay below
// 2^16 on every axis.
int oc_subdivide(const int32_t* coords, int64_t n, const uint8_t* keep, int32_t* fine, int32_t* children,
                 int64_t* n_fine) {
  if (n < 0 || n_fine == nullptr || (n > 0 && (coords == nullptr || fine == nullptr || children == nullptr)))
    return kErrInvalid;
  int64_t f = 0;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t* c = coords + 4 * i;
    if (!in_range(c[0]) || !in_range(2 * c[1] + 1) || !in_range(2 * c[2] + 1) || !in_range(2 * c[3] + 1) ||
        c[1] < 0 || c[2] < 0 || c[3] < 0)
      return kErrCoordRange;
    for (int o = 0; o < 8; ++o) {
      if (keep != nullptr && !((keep[i] >> o) & 1)) {
        children[8 * i + o] = -1;
        continue;
      }
      fine[4 * f + 0] = c[0];
      fine[4 * f + 1] = 2 * c[1] + ((o >> 2) & 1);
      fine[4 * f + 2] = 2 * c[2] + ((o >> 1) & 1);
      fine[4 * f + 3] = 2 * c[3] + (o & 1);
      children[8 * i + o] = int32_t(f);
      ++f;
    }
  }
  *n_fine = f;
  return kOk;
}

// x_fine[children[q * 8 + o], c] = x_coarse[q, c * 8 + o] (Channel2Spatial):
// with to_fine = 1 from coarse [n_coarse, 8 C] to fine [n_fine, C]; with
// to_fine = 0 the inverse gather, x_coarse[q, c * 8 + o] = x_fine[child, c] or
// 0 where child o is absent (Spatial2Channel).
int oc_regroup(const int32_t* children, int64_t n_coarse, int64_t n_fine, int c_fine, int to_fine,
               double* x_coarse, double* x_fine) {
  if (n_coarse < 0 || n_fine < 0 || c_fine <= 0) return kErrInvalid;
  for (int64_t q = 0; q < n_coarse; ++q)
    for (int o = 0; o < 8; ++o) {
      const int32_t f = children[8 * q + o];
      if (f < -1 || f >= n_fine) return kErrInvalid;
      for (int c = 0; c < c_fine; ++c) {
        double& xc = x_coarse[q * 8 * c_fine + int64_t(c) * 8 + o];
        if (to_fine) {
          if (f >= 0) x_fine[int64_t(f) * c_fine + c] = xc;
        } else {
          xc = f >= 0 ? x_fine[int64_t(f) * c_fine + c] : 0.0;
        }
      }
    }
  return kOk;
}

int oc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"
