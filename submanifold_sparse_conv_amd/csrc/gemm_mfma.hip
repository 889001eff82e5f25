// Gather-GEMM on the matrix cores (bf16 or fp16 operands, fp32 accumulate):
// the compute half of the sparse convolution -- a gather-GEMM over the neighbour
// table with half-precision inputs and single-precision accumulation
// ("Porting TRELLIS.2 From Python to Rust and Metal", section V), i.e. the
// per-kernel-position gather -> matmul -> sum of "Running TRELLIS.2 on a Mac
// (1/3)" (sparse 3D convolution paragraph).
//
// Output-stationary: a workgroup owns a tile of TM voxels (consecutive in
// Morton order) x TN output channels and keeps it in registers for the whole
// reduction over taps and input channels, then writes every row once at the
// voxel's caller index. No atomics, fixed (tap, channel) order: results are
// the same bit for bit on every run.
//
// Two families of kernels. fwd_halo (below, the shapes of halo_shape: half
// features, C_in a multiple of 64 up to 1024, C_out 32, 64 or a multiple of
// 128) stages each 256-voxel tile's distinct neighbour rows in LDS once per
// 32-channel chunk and reads every tap's operand from there, following a plan
// the kernel map builds per tile. fwd_rows / fwd_lds take the other shapes:
//
// K loop: the taps some row of the tile needs (OR of the rows' 27-bit
// neighbour masks), each split into 64-channel chunks ("stages"). Each of the
// four waves owns 16*FM whole rows of the tile and all TN columns, so every
// gathered feature row is read by one wave only. fwd_rows loads its MFMA A
// fragments from global memory straight into registers, one stage ahead;
// fwd_lds copies the rows into a per-wave LDS slot in a coalesced lane layout
// and reads the fragments from there (the faster gather; chosen for narrow
// outputs and large 64-wide layers). The stage's weight slice, which all four
// waves read, is copied into LDS with global_load_lds (double-buffered,
// XOR-swizzled 128-byte rows). Matrix instruction: v_mfma_f32_16x16x32_bf16 /
// _f16.
//
// Precision paths: half features with half weights; or fp32 features with half
// weights, each fp32 value carried as a sum of half terms (the pages' decoders
// keep their incoming latent in fp32 and run the layers after it in half --
// "Porting TRELLIS.2 ...", section IV). Output: half or fp32, after a fused
// bias / activation / residual epilogue.
//
// Weights are first re-laid out to [27][C_out][C_in] (input channels
// contiguous), the operand order of the matrix instruction, followed by a
// 256-byte block of zeros (the copy source of absent neighbours).
#include <mutex>
#include <utility>

#include "common.h"
#include "launch.h"

namespace trsc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

// f(std::integral_constant<int, 0>{}) .. f(std::integral_constant<int, N-1>{}),
// unrolled at compile time.
template <class F, int... J>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// The two half types of the matrix cores: their MFMA and conversions.
template <bool F16>
struct Half;
template <>
struct Half<false> {
  typedef bf16x8 vec;
  typedef __bf16 elt;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mma32(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float widen(uint16_t h) { return bf16_to_f32(h); }
  static __device__ __forceinline__ uint16_t narrow(float v) { return f32_to_bf16_rne(v); }
};
template <>
struct Half<true> {
  typedef f16x8 vec;
  typedef _Float16 elt;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mma32(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float widen(uint16_t h) {
    return float(__builtin_bit_cast(_Float16, h));
  }
  static __device__ __forceinline__ uint16_t narrow(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));  // nearest, ties to even
  }
};

// fp32 features as a sum of XT half-precision terms, x = t0 + t1 (+ t2):
// each term is the rounding of what the earlier ones left over, and every
// remainder is exact in fp32. A half weight times a half term is exact in the
// fp32 accumulator, so the XT products carry x itself rather than x rounded to
// half precision: three bf16 terms hold all 24 significant bits; two fp16 terms
// hold x to within 2^-23 |x| (2^-25 absolute where the second term is below
// the fp16 normal range).
template <class H, int XT>
__device__ __forceinline__ void split_terms(const uint4 (&raw)[2], typename H::vec (&t)[XT]) {
  const float* f = reinterpret_cast<const float*>(raw);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float r = f[e];
#pragma unroll
    for (int q = 0; q < XT; ++q) {
      const typename H::elt h = static_cast<typename H::elt>(r);
      t[q][e] = h;
      if (q + 1 < XT) r -= static_cast<float>(h);
    }
  }
}

struct RowsArgs {
  const int32_t* nbr;
  const unsigned char* plan;  // halo plan records (fwd_halo)
  const int32_t* order;       // halo tiles in launch order (fwd_halo)
  const int32_t* srows;
  const uint32_t* vmask;
  int64_t n;
  const void* x;          // [n, c_in]: half (XT = 1) or fp32 (XT > 1)
  const uint16_t* wp;     // packed [27][c_out][c_in] half weights
  const uint16_t* zeros;  // 256 zero bytes
  void* y;                // [n, c_out]: half or fp32 (y_f32)
  const float* bias;      // [c_out] or null
  const void* residual;   // [n, c_out], y's type, or null; may be y itself
  int act, y_f32;
  int c_in, c_out, n_tiles_n;
};

// Epilogue, fused into the same pass as the pages fuse theirs (bias,
// activation, residual add and the output rounding -- "Porting TRELLIS.2 ...",
// section V): v = act(acc + bias) in fp32, staged per 16-row block in this
// wave's own LDS region `sO` (8 rows of TN floats); then each lane adds the
// residual to 16 bytes' worth of one output row and rounds once, to the output
// type. acc[i][j] holds rows 16 i + 4 kg + e of the wave's rows and columns
// n0 + 16 j + lr; crow[i] is the caller row of the wave's row 16 i + lr (or
// -1). The caller has waited for all of its loads: `sO` is free.
template <int FM, int FN, class H>
__device__ __forceinline__ void store_tile(const RowsArgs& p, const f32x4 (&acc)[FM][FN], const int32_t (&crow)[FM],
                                           int n0, float* sO) {
  constexpr int TN = 16 * FN;
  const int c_out = p.c_out;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, kg = lane >> 4;
  float bv[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int c = n0 + j * 16 + lr;
    bv[j] = (p.bias != nullptr && c < c_out) ? p.bias[c] : 0.f;
  }

  // Staged row r (8 per pass) holds TN floats in 16-byte pieces; piece q sits
  // at q ^ osw(r), which puts the two rows one write instruction touches on
  // different banks and keeps each aligned group of four pieces contiguous.
  constexpr int PPR = TN / 4;
  auto spos = [](int r, int q) { return r * TN + ((q ^ (((r >> 2) & 1) << 2 & (PPR - 1))) << 2); };
  const int act = p.act;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // D rows 4 kg + e of this fragment: lanes with kg >> 1 == h hold rows 8h .. 8h + 7
      if ((kg >> 1) == h) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = (kg & 1) * 4 + e, c = j * 16 + lr;
            sO[spos(r, c >> 2) + (c & 3)] = activate(acc[i][j][e] + bv[j], act);
          }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
      if (!p.y_f32) {
        constexpr int OPR = TN / 8;
#pragma unroll
        for (int q = lane; q < 8 * OPR; q += 64) {
          const int r = q / OPR, cc = q % OPR;
          const int32_t row = __shfl(crow[i], 8 * h + r, 64);
          const int co = n0 + cc * 8;
          if (row >= 0 && co < c_out) {
            const float4 lo = *reinterpret_cast<const float4*>(sO + spos(r, 2 * cc));
            const float4 hi = *reinterpret_cast<const float4*>(sO + spos(r, 2 * cc + 1));
            float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            const int64_t off = int64_t(row) * c_out + co;
            if (p.residual != nullptr) {
              const uint4 rr = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.residual) + off);
              const uint16_t* rh = reinterpret_cast<const uint16_t*>(&rr);
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] += H::widen(rh[e]);
            }
            uint4 o;
            uint16_t* oh = reinterpret_cast<uint16_t*>(&o);
#pragma unroll
            for (int e = 0; e < 8; ++e) oh[e] = H::narrow(v[e]);
            store_stream(reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.y) + off), o);
          }
        }
      } else {
        constexpr int OPR = TN / 4;
#pragma unroll
        for (int q = lane; q < 8 * OPR; q += 64) {
          const int r = q / OPR, cc = q % OPR;
          const int32_t row = __shfl(crow[i], 8 * h + r, 64);
          const int co = n0 + cc * 4;
          if (row >= 0 && co < c_out) {
            float4 v = *reinterpret_cast<const float4*>(sO + spos(r, cc));
            const int64_t off = int64_t(row) * c_out + co;
            if (p.residual != nullptr) {
              const float4 rr = *reinterpret_cast<const float4*>(static_cast<const float*>(p.residual) + off);
              v.x += rr.x, v.y += rr.y, v.z += rr.z, v.w += rr.w;
            }
            store_stream(reinterpret_cast<uint4*>(static_cast<float*>(p.y) + off),
                         uint4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)});
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next pass overwrites
    }
  }
}

// Wave w of the workgroup owns rows [16*FM*w, 16*FM*(w+1)) of the tile and all
// TN = 16*FN output channels. The tile's rows of the neighbour table are copied
// into LDS once; a tap's gather indices are read from there one tap ahead, the
// A fragments and the weight slice are loaded one stage ahead.
template <int FM, int FN, bool F16, int XT>
__global__ __launch_bounds__(kThreads, 2) void fwd_rows(const RowsArgs p) {
  typedef Half<F16> H;
  typedef typename H::vec hvec;
  constexpr int WM = 16 * FM, TM = 4 * WM, TN = 16 * FN;
  constexpr int KC = 64, ROWB = KC * 2;
  constexpr int AV = XT == 1 ? 1 : 2;         // 16-byte loads per 8 input channels
  constexpr int BBUF = TN * ROWB;             // weight slice of one stage
  constexpr int OSTAGE = 4 * 8 * TN * 4;      // 8 fp32 output rows per wave, four waves
  __shared__ __attribute__((aligned(1024))) unsigned char bbuf0[BBUF > OSTAGE ? BBUF : OSTAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char bbuf1[BBUF];
  __shared__ int32_t s_taps[27];
  __shared__ uint32_t s_mask;
  __shared__ int32_t s_idx[TM * 27];  // the tile's neighbour rows, [row][tap]

  const int c_in = p.c_in, c_out = p.c_out;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t t0 = int64_t(tile / p.n_tiles_n) * TM;
  const int n0 = (tile % p.n_tiles_n) * TN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kg = lane >> 4;

  // This lane's rows (one per row fragment) and the taps the tile needs.
  int32_t crow[FM];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t t = t0 + wave * WM + i * 16 + lr;
    crow[i] = t < p.n ? p.srows[t] : -1;
    if (t < p.n) m |= p.vmask[t];
  }
  for (int o = 32; o > 0; o >>= 1) m |= __shfl_xor(m, o, 64);
  if (tid == 0) s_mask = 0;
  __syncthreads();
  if (lane == 0) atomicOr(&s_mask, m);
  __syncthreads();
  const uint32_t tmask = __builtin_amdgcn_readfirstlane(s_mask);
  if (tid < 27 && ((tmask >> tid) & 1u)) s_taps[__popc(tmask & ((1u << tid) - 1u))] = tid;
  // The tile's rows of the neighbour table, 27 taps each, copied once into LDS:
  // two threads per row, 14 and 13 taps, their loads in flight together.
  {
    const int64_t rows_left = p.n - t0;
    const int nrows = rows_left < TM ? int(rows_left) : TM;
    const int h = tid & 1;
    for (int r = tid >> 1; r < TM; r += kThreads / 2) {
      const bool ok = r < nrows;
      const int32_t cr = ok ? p.srows[t0 + r] : 0;
      int32_t v[14];
#pragma unroll
      for (int j = 0; j < 14; ++j) {
        const int k = h * 14 + j;
        v[j] = (ok && k < 27) ? p.nbr[int64_t(cr) * 27 + k] : -1;
      }
#pragma unroll
      for (int j = 0; j < 14; ++j) {
        const int k = h * 14 + j;
        if (k < 27) s_idx[r * 27 + k] = v[j];
      }
    }
  }
  __syncthreads();
  const int ntaps = __popc(tmask);
  const int nchunks = (c_in + KC - 1) / KC;
  const int nstages = ntaps * nchunks;

  int32_t srcL[FM], srcF[FM];  // gather rows of the tap being issued / being fetched
  auto fetch_idx = [&](int ti, int32_t (&dst)[FM]) {
    const int k = s_taps[ti];
#pragma unroll
    for (int i = 0; i < FM; ++i) dst[i] = s_idx[(wave * WM + i * 16 + lr) * 27 + k];
  };
  // Issue stage st: A fragments into registers, weight slice into LDS.
  auto issue = [&](int st, uint4 (&a)[FM][2][AV], unsigned char* bdst) {
    const int ti = st / nchunks;
    const int c0 = (st - ti * nchunks) * KC;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int c = c0 + kk * 32 + kg * 8;
        const bool ok = srcL[i] >= 0 && c < c_in;
        const int64_t off = int64_t(srcL[i]) * c_in + c;
        const unsigned char* g =
            ok ? static_cast<const unsigned char*>(p.x) + off * (XT == 1 ? 2 : 4)
               : reinterpret_cast<const unsigned char*>(p.zeros);
#pragma unroll
        for (int v = 0; v < AV; ++v) a[i][kk][v] = reinterpret_cast<const uint4*>(g)[v];
      }
    const uint16_t* wk = p.wp + int64_t(s_taps[ti]) * c_out * c_in;
#pragma unroll
    for (int i = wave; i < TN / 8; i += 4) {
      const int col = i * 8 + (lane >> 3);
      const int c = c0 + swz(col, lane & 7) * 8;
      const void* g = (n0 + col < c_out && c < c_in)
                          ? static_cast<const void*>(wk + int64_t(n0 + col) * c_in + c)
                          : static_cast<const void*>(p.zeros);
      copy16_to_lds(g, bdst + i * 1024);
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint4 (&a)[FM][2][AV], const unsigned char* bsrc) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int chunk = kk * 4 + kg;
      hvec av[FM][XT];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (XT == 1)
          av[i][0] = *reinterpret_cast<const hvec*>(&a[i][kk][0]);
        else
          split_terms<H, XT>(a[i][kk], av[i]);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = j * 16 + lr;
        const hvec b = *reinterpret_cast<const hvec*>(bsrc + r * ROWB + swz(r, chunk) * 16);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < XT; ++q) acc[i][j] = H::mma(av[i][q], b, acc[i][j]);
      }
    }
  };

  // One stage: wait for everything issued (stage st, issued a full stage
  // earlier), barrier (every wave's weight copies have landed and the other
  // buffer is free), issue stage st+1, fetch indices for the tap after, compute.
  auto step = [&](int st, const uint4 (&aC)[FM][2][AV], uint4 (&aN)[FM][2][AV], const unsigned char* bC,
                  unsigned char* bN) {
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("s_barrier" ::: "memory");
    if (st + 1 < nstages) {
      if ((st + 1) % nchunks == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i) srcL[i] = srcF[i];
      }
      issue(st + 1, aN, bN);
      if (st + 2 < nstages && (st + 2) % nchunks == 0) fetch_idx((st + 2) / nchunks, srcF);
    }
    compute(aC, bC);
  };

  uint4 a0[FM][2][AV], a1[FM][2][AV];
  if (nstages > 0) {
    fetch_idx(0, srcL);
    issue(0, a0, bbuf0);
    if (1 < nstages && 1 % nchunks == 0) fetch_idx(1, srcF);
  }
  for (int st = 0; st < nstages; st += 2) {
    step(st, a0, a1, bbuf0, bbuf1);
    if (st + 1 < nstages) step(st + 1, a1, a0, bbuf1, bbuf0);
  }

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  store_tile<FM, FN, H>(p, acc, crow, n0, reinterpret_cast<float*>(bbuf0) + wave * 8 * TN);
}

// The same output-stationary tile with the gathered feature rows staged
// through LDS. A lane's 16 bytes of an MFMA A fragment come from a row that the
// other 15 lanes of its 16-lane group do not touch; a gather in that lane
// layout moves ~16 bytes per clock per CU, while eight consecutive lanes on one
// 128-byte row segment move ~50 (measured on gfx950, rows in L2). So each wave
// copies its rows of a stage (16 * FM rows x 64 channels, one 128-byte segment
// each) with global_load_lds in the coalesced layout, eight rows per
// instruction, into its own LDS slot, and reads its A fragments back with
// ds_read_b128. Chunk c of row r sits at chunk position c ^ ((r >> 1) & 7):
// the 16 rows one 16-lane group of a fragment read touches then fall on 16
// different 16-byte bank groups. At the start of a stage the wave moves its
// fragments into registers and refills the slot with the next stage's rows;
// the slot is private to the wave (no barrier for it), the weight slice stays
// shared as in fwd_rows. Each copy lane fetches its row's neighbour index per
// tap from the neighbour table, one tap ahead. Bit-identical to fwd_rows (same
// products, same order).
template <int FM, int FN, bool F16>
__global__ __launch_bounds__(kThreads, 3) void fwd_lds(const RowsArgs p) {
  typedef Half<F16> H;
  typedef typename H::vec hvec;
  constexpr int WM = 16 * FM, TM = 4 * WM, TN = 16 * FN;
  constexpr int KC = 64, ROWB = KC * 2;
  constexpr int ABUF = WM * ROWB;             // one wave's rows of one stage
  constexpr int BBUF = TN * ROWB;             // weight slice of one stage
  constexpr int OSTAGE = 4 * 8 * TN * 4;      // 8 fp32 output rows per wave, four waves
  constexpr int NQ = WM / 8;                  // row copies per wave and stage (8 rows each)
  __shared__ __attribute__((aligned(1024))) unsigned char bbuf0[BBUF > OSTAGE ? BBUF : OSTAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char bbuf1[BBUF];
  __shared__ __attribute__((aligned(1024))) unsigned char abuf[4 * ABUF];
  __shared__ int32_t s_taps[27];
  __shared__ uint32_t s_mask;

  const int c_in = p.c_in, c_out = p.c_out;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t t0 = int64_t(tile / p.n_tiles_n) * TM;
  const int n0 = (tile % p.n_tiles_n) * TN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kg = lane >> 4;
  unsigned char* const aw = abuf + wave * ABUF;

  // This lane's rows (one per row fragment) and the taps the tile needs.
  int32_t crow[FM];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t t = t0 + wave * WM + i * 16 + lr;
    crow[i] = t < p.n ? p.srows[t] : -1;
    if (t < p.n) m |= p.vmask[t];
  }
  for (int o = 32; o > 0; o >>= 1) m |= __shfl_xor(m, o, 64);
  if (tid == 0) s_mask = 0;
  __syncthreads();
  if (lane == 0) atomicOr(&s_mask, m);
  __syncthreads();
  const uint32_t tmask = __builtin_amdgcn_readfirstlane(s_mask);
  if (tid < 27 && ((tmask >> tid) & 1u)) s_taps[__popc(tmask & ((1u << tid) - 1u))] = tid;
  __syncthreads();
  const int ntaps = __popc(tmask);
  const int nchunks = (c_in + KC - 1) / KC;
  const int nstages = ntaps * nchunks;

  // Copy lanes: copy q of a stage moves the wave's rows 8q .. 8q + 7; lane l
  // takes row 8q + (l >> 3) and the chunk stored at position l & 7. nrow[q]:
  // that row's 27 entries of the neighbour table (null past the end).
  const int32_t* nrow[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t t = t0 + wave * WM + 8 * q + (lane >> 3);
    nrow[q] = t < p.n ? p.nbr + int64_t(p.srows[t]) * 27 : nullptr;
  }
  int32_t srcL[NQ], srcF[NQ];  // gather rows of the copy lanes: tap being issued / being fetched
  auto fetch_idx = [&](int ti, int32_t (&dst)[NQ]) {
    const int k = s_taps[ti];
#pragma unroll
    for (int q = 0; q < NQ; ++q) dst[q] = nrow[q] != nullptr ? nrow[q][k] : -1;
  };
  auto issue_a = [&](int st) {
    const int ti = st / nchunks;
    const int c0 = (st - ti * nchunks) * KC;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int r = 8 * q + (lane >> 3);
      const int c = c0 + (((lane & 7) ^ ((r >> 1) & 7)) << 3);
      const void* g = (srcL[q] >= 0 && c < c_in)
                          ? static_cast<const void*>(static_cast<const uint16_t*>(p.x) + int64_t(srcL[q]) * c_in + c)
                          : static_cast<const void*>(p.zeros);
      copy16_to_lds(g, aw + q * 1024);
    }
  };
  auto issue_b = [&](int st, unsigned char* bdst) {
    const int ti = st / nchunks;
    const int c0 = (st - ti * nchunks) * KC;
    const uint16_t* wk = p.wp + int64_t(s_taps[ti]) * c_out * c_in;
#pragma unroll
    for (int i = wave; i < TN / 8; i += 4) {
      const int col = i * 8 + (lane >> 3);
      const int c = c0 + swz(col, lane & 7) * 8;
      const void* g = (n0 + col < c_out && c < c_in)
                          ? static_cast<const void*>(wk + int64_t(n0 + col) * c_in + c)
                          : static_cast<const void*>(p.zeros);
      copy16_to_lds(g, bdst + i * 1024);
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A fragment (i, kk) of this lane: row 16 i + lr, chunk 4 kk + kg.
  auto a_off = [&](int i, int kk) {
    const int r = 16 * i + lr;
    return (8 * r + ((4 * kk + kg) ^ ((r >> 1) & 7))) * 16;
  };
  auto compute = [&](const hvec (&av)[FM][2], const unsigned char* bsrc) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int chunk = kk * 4 + kg;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = j * 16 + lr;
        const hvec b = *reinterpret_cast<const hvec*>(bsrc + r * ROWB + swz(r, chunk) * 16);
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[i][j] = H::mma(av[i][kk], b, acc[i][j]);
      }
    }
  };

  // One stage: wait for everything issued (stage st, issued a stage earlier),
  // barrier (every wave's weight copies have landed; the other weight buffer
  // is free), take this wave's A fragments out of its slot, refill the slot
  // with stage st+1 and issue st+1's weight slice, fetch the indices of the
  // tap after, multiply.
  auto step = [&](int st, const unsigned char* bC, unsigned char* bN) {
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("s_barrier" ::: "memory");
    hvec av[FM][2];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) av[i][kk] = *reinterpret_cast<const hvec*>(aw + a_off(i, kk));
    if (st + 1 < nstages) {
      if ((st + 1) % nchunks == 0) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) srcL[q] = srcF[q];
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the fragments are out of the slot
      issue_a(st + 1);
      issue_b(st + 1, bN);
      if (st + 2 < nstages && (st + 2) % nchunks == 0) fetch_idx((st + 2) / nchunks, srcF);
    }
    compute(av, bC);
  };

  if (nstages > 0) {
    fetch_idx(0, srcL);
    if (1 < nstages && 1 % nchunks == 0) fetch_idx(1, srcF);
    issue_a(0);
    issue_b(0, bbuf0);
  }
  for (int st = 0; st < nstages; st += 2) {
    step(st, bbuf0, bbuf1);
    if (st + 1 < nstages) step(st + 1, bbuf1, bbuf0);
  }

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  store_tile<FM, FN, H>(p, acc, crow, n0, reinterpret_cast<float*>(bbuf0) + wave * 8 * TN);
}

// Epilogue of a wave's block of RB x CB 32x32 fp32 accumulators: acc[b][cb]
// holds rows 32 b + 8 (e / 4) + 4 (lane / 32) + e % 4 (element e) of the
// wave's rows and column n0 + 32 cb + lane % 32. In passes of 16 rows (rows
// 32 b + 16 h ..), v = act(acc + bias) goes to this wave's LDS region `sO` (16
// rows of 32 CB floats, row stride 32 CB + 8 floats so that the two half-waves
// write different banks); then each lane takes 16-byte output pieces of whole
// rows, adds the residual, rounds once and stores at the caller row. crow[q]:
// caller row of the wave's row 64 q + lane (-1: not stored).
template <class H, int RB, int CB>
__device__ __forceinline__ void store_tile32(const RowsArgs& p, const f32x16 (&acc)[RB][CB],
                                             const int32_t (&crow)[(RB + 1) / 2], int n0, float* sO) {
  constexpr int TN = 32 * CB, SR = TN + 8;
  const int c_out = p.c_out;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hw = lane >> 5;
  float bv[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int c = n0 + cb * 32 + l32;
    bv[cb] = (p.bias != nullptr && c < c_out) ? p.bias[c] : 0.f;
  }
  const int act = p.act;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // elements e = 8h .. 8h+7: rows 16h + 8 (e' / 4) + 4 hw + e' % 4 of the block (e' = e - 8h)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * (e >> 2) + 4 * hw + (e & 3);
          sO[r * SR + cb * 32 + l32] = activate(acc[b][cb][8 * h + e] + bv[cb], act);
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
      const int row0 = 32 * b + 16 * h;    // the pass's first row in the wave
      if (!p.y_f32) {
#pragma unroll
        for (int q = lane; q < 16 * (TN / 8); q += 64) {
          const int r = q / (TN / 8), cc = q % (TN / 8);
          const int32_t row = __shfl(crow[(row0 + r) >> 6], (row0 + r) & 63, 64);
          const int co = n0 + cc * 8;
          if (row >= 0 && co < c_out) {
            const float4 lo = *reinterpret_cast<const float4*>(sO + r * SR + cc * 8);
            const float4 hi = *reinterpret_cast<const float4*>(sO + r * SR + cc * 8 + 4);
            float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            const int64_t off = int64_t(row) * c_out + co;
            if (p.residual != nullptr) {
              const uint4 rr = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.residual) + off);
              const uint16_t* rh = reinterpret_cast<const uint16_t*>(&rr);
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] += H::widen(rh[e]);
            }
            uint4 o;
            uint16_t* oh = reinterpret_cast<uint16_t*>(&o);
#pragma unroll
            for (int e = 0; e < 8; ++e) oh[e] = H::narrow(v[e]);
            store_stream(reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.y) + off), o);
          }
        }
      } else {
#pragma unroll
        for (int q = lane; q < 16 * (TN / 4); q += 64) {
          const int r = q / (TN / 4), cc = q % (TN / 4);
          const int32_t row = __shfl(crow[(row0 + r) >> 6], (row0 + r) & 63, 64);
          const int co = n0 + cc * 4;
          if (row >= 0 && co < c_out) {
            float4 v = *reinterpret_cast<const float4*>(sO + r * SR + cc * 4);
            const int64_t off = int64_t(row) * c_out + co;
            if (p.residual != nullptr) {
              const float4 rr = *reinterpret_cast<const float4*>(static_cast<const float*>(p.residual) + off);
              v.x += rr.x, v.y += rr.y, v.z += rr.z, v.w += rr.w;
            }
            store_stream(reinterpret_cast<uint4*>(static_cast<float*>(p.y) + off),
                         uint4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)});
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next pass overwrites
    }
  }
}

// The same output-stationary product with the gathered rows read from a halo:
// over tiles of kHaloTM Morton-consecutive voxels, the tile's distinct
// neighbour rows are copied into LDS once per 32-channel chunk and every tap
// reads its A fragments from there, instead of gathering each (voxel, tap) row
// from global memory. Over a thin surface the halo holds ~1.75 rows per voxel
// against ~17.7 gathered ones. The plan (tile order, halo rows, the LDS
// offset of every (row, tap)'s row, which 32-row blocks have which taps) comes
// from the kernel map (halo_plan.h).
//
// Matrix instruction v_mfma_f32_32x32x16 (bf16 / fp16): on gfx950 it sustains
// ~97 % of the matrix peak from two waves per SIMD, where 16x16x32 stays near
// 62 % whatever the occupancy (measured). The four waves split the 256 x 128
// tile two by two: wave w owns rows 128 (w / 2) .. + 128 (four 32-row blocks)
// and columns n0 + 64 (w % 2) .. + 64 (two 32-column blocks), eight 32x32 fp32
// accumulators.
//
// Stages run chunk-major: for each 32-channel chunk, the tile's taps in order;
// a stage is two 16-channel steps of up to 8 multiplies each. Each wave loads
// its own B fragments straight into registers from the fragment-ordered copy
// of the weights (one contiguous kilobyte per fragment), two stages ahead, so
// the weights need no LDS and the stages need no barrier: the waves only meet
// when a chunk's halo is replaced. The MFMA issue slot of a SIMD is shared with
// all other vector instructions, so a stage keeps those few: A fragment
// addresses are one XOR of offsets stored in the plan, tap and block masks
// live in scalar registers. A 32-row block skips the multiplies of a tap none
// of its rows has. Each output row sums, chunk by chunk, its taps in order
// (two 16-channel products per stage): the same bits whatever the slots, run
// to run.
//
// Halo rows are 64 bytes (four 16-byte pieces); piece q of row r sits at
// position q ^ ((r >> 2) & 3), so 16 rows read at one piece fall on 16
// different bank groups whenever their numbers differ mod 16. A tile whose halo
// does not fit (nh < 0: sparse sets, up to 27 distinct neighbours per voxel)
// gathers its A fragments from global memory in the same order, so its
// results are the same bits. Shapes: halo_shape (c_in a multiple of 64 up to
// 256; c_out 32, 64, 128 or 256). For c_out 64 (32) the item is 256 x 64
// (256 x 32) and the four waves take 64 rows x 64 (32) columns each (template
// WR = 4, CB = 2 or 1).
//
// Work items: blockIdx -> (row tile, column tile) in the plan's launch order;
// when the last round of workgroups would hold few items (split > 0), each of
// the last `split` items becomes kHaloParts workgroups (halo_part), so that
// the last round is short.
constexpr int kHaloKC = 32;
static_assert(kHaloRowBytes == kHaloKC * 2, "halo rows hold one chunk of half-precision channels");

struct HaloLaunch {
  int full;   // work items run whole
  int split;  // items after them, each run as kHaloParts parts
};
constexpr int kHaloParts = kHaloTM / 32;  // one part per 32-row block
// halo_part's LDS, in floats: partial sums of waves 1-3 | output staging | neighbour table
constexpr int kPartNbrAt = 3 * 4 * 16 * 64 + 16 * (32 * 4 + 8);

// One 32-row block of an item (rows 32 blk .. + 31 of the tile, columns
// n0 .. n0 + 32 CB - 1), for the last, short round: the four waves split the input
// channels (wave w takes the 32-channel chunks w, w + 4, ...), gather their A
// fragments straight from global memory with the loads three taps ahead, and
// their partial sums meet in LDS, added in chunk order, before wave 0's
// epilogue. A part's chain of dependent steps is a quarter of a whole item's
// (or less), so the round ends soon after it starts. The sums of a split item
// are added in another order than a whole item's: results equal to rounding,
// and the same bits run to run (the split depends only on the sizes and the
// device).
template <class H, int CB>
__device__ __forceinline__ void halo_part(const RowsArgs& p, const unsigned char* rec, int blk, int n0, float* s_red) {
  typedef typename H::vec hvec;
  static_assert(CB == 1 || CB == 2 || CB == 4, "32, 64 or 128 columns");
  constexpr int D = 3;  // 27 taps = 9 x D: a tap's load set is k % D in every chunk
  const int c_in = p.c_in, c_out = p.c_out;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hw = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const HaloHeader* const hdr = reinterpret_cast<const HaloHeader*>(rec + kPlanHdr);
  const int r = 32 * blk + l32;
  const int32_t crow = reinterpret_cast<const int32_t*>(rec + kPlanCrow)[r];
  uint32_t tm = 0;  // taps the block has
#pragma unroll
  for (int k = 0; k < 27; ++k) tm |= uint32_t((hdr->fm[k] >> blk) & 1u) << k;
  const int nchunks = c_in / kHaloKC;
  // caller rows of the block's rows' neighbours (-1: absent), [tap][row], in
  // LDS past the partial sums and the output staging
  int32_t* const s_nb = reinterpret_cast<int32_t*>(s_red) + kPartNbrAt;
  for (int e = tid; e < 27 * 32; e += kThreads) {
    const int k = e >> 5, rr = 32 * blk + (e & 31);
    const int32_t cr = reinterpret_cast<const int32_t*>(rec + kPlanCrow)[rr];
    const uint32_t m = cr >= 0 ? reinterpret_cast<const uint32_t*>(rec + kPlanMask)[rr] : 0u;
    s_nb[e] = ((m >> k) & 1u) ? p.nbr[int64_t(cr) * 27 + k] : -1;
  }
  __syncthreads();

  const int ncb = c_out / 32, cb0 = n0 / 32;
  const uint4* const wf = reinterpret_cast<const uint4*>(p.wp + frag_weight_offset(c_in, c_out)) + cb0 * 64 + lane;
  const uint16_t* const xs = static_cast<const uint16_t*>(p.x);
  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[cb][e] = 0.f;
  uint4 bq[D][2][CB], aq[D][2];
  // the loads of tap k of chunk c (a chunk past the wave's last reads chunk
  // `wave` again; nothing multiplies it)
  auto issue = [&](int c, int k, uint4 (&b)[2][CB], uint4 (&a)[2]) {
    const int cc = c < nchunks ? c : wave;
    const uint4* f = wf + int64_t((cc * 27 + k) * 2) * ncb * 64;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) b[s][cb] = f[(s * ncb + cb) * 64];
    const int32_t j = s_nb[k * 32 + l32];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const void* g = j >= 0 ? static_cast<const void*>(xs + int64_t(j) * c_in + cc * kHaloKC + (2 * s + hw) * 8)
                             : static_cast<const void*>(p.zeros);
      a[s] = *reinterpret_cast<const uint4*>(g);
    }
  };
  if (wave < nchunks) {
#pragma unroll
    for (int k = 0; k < D; ++k) issue(wave, k, bq[k], aq[k]);
    auto step = [&](int c, int k, uint4 (&b)[2][CB], uint4 (&a)[2]) {
      if ((tm >> k) & 1u) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[cb] = H::mma32(*reinterpret_cast<const hvec*>(&a[s]), *reinterpret_cast<const hvec*>(&b[s][cb]),
                               acc[cb]);
      }
      if (k + D < 27)
        issue(c, k + D, b, a);
      else
        issue(c + 4, k + D - 27, b, a);
    };
    for (int c = wave; c < nchunks; c += 4) {
#pragma unroll 1
      for (int k = 0; k < 27; k += D) {
        step(c, k, bq[0], aq[0]);
        step(c, k + 1, bq[1], aq[1]);
        step(c, k + 2, bq[2], aq[2]);
      }
    }
  }
  // partial sums of waves 1.. into LDS (their accumulator layout), wave 0
  // adds them in chunk order and stores
  __builtin_amdgcn_s_waitcnt(0);
  if (wave > 0 && wave < nchunks) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int e = 0; e < 16; e += 4)
        *reinterpret_cast<float4*>(s_red + (((wave - 1) * CB + cb) * 16 + e) * 64 + lane * 4) =
            make_float4(acc[cb][e], acc[cb][e + 1], acc[cb][e + 2], acc[cb][e + 3]);
  }
  __syncthreads();
  if (wave == 0) {
    for (int w = 1; w < (nchunks < 4 ? nchunks : 4); ++w)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int e = 0; e < 16; e += 4) {
          const float4 v = *reinterpret_cast<const float4*>(s_red + (((w - 1) * CB + cb) * 16 + e) * 64 + lane * 4);
          acc[cb][e] += v.x;
          acc[cb][e + 1] += v.y;
          acc[cb][e + 2] += v.z;
          acc[cb][e + 3] += v.w;
        }
    f32x16 out[1][CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) out[0][cb] = acc[cb];
    const int32_t cr[1] = {lane < 32 ? crow : -1};
    store_tile32<H, 1, CB>(p, out, cr, n0, s_red + 3 * CB * 16 * 64);
  }
}

template <bool F16, int WR, int CB>
__global__ __launch_bounds__(kThreads, 2) void fwd_halo(const RowsArgs p, const HaloLaunch hl) {
  typedef Half<F16> H;
  typedef typename H::vec hvec;
  // WR row groups of waves, CB 32-column blocks per wave: WR 2, CB 2 (2 x 2
  // waves, 128 rows x 64 columns each, a 128-column item); WR 4 (4 x 1 waves,
  // 64 rows x 32 CB columns each, a 32 CB-column item)
  static_assert((WR == 2 && CB == 2) || (WR == 4 && (CB == 1 || CB == 2)), "wave arrangements");
  constexpr int TM = kHaloTM, RB = 8 / WR, TN = 32 * CB * (4 / WR);
  constexpr int WROWS = TM / WR;  // rows per wave
  constexpr int KC = kHaloKC, ROWB = kHaloRowBytes;
  constexpr int HBYTES = kHaloCap * ROWB;
  constexpr int SLOTQ = (kPlanSlotBytes + 1023) / 1024, ROWQ = (kHaloCap * 4 + 1023) / 1024;
  static_assert(HBYTES >= 4 * 16 * (32 * CB + 8) * 4, "the output staging lives in the halo area");
  // LDS: halo | slot table | halo rows' caller rows (a part uses it whole)
  __shared__ __attribute__((aligned(1024))) unsigned char s_lds[HBYTES + (SLOTQ + ROWQ) * 1024];
  static_assert((kPartNbrAt + 27 * 32) * 4 <= HBYTES + (SLOTQ + ROWQ) * 1024, "halo_part's LDS");
  unsigned char* const s_halo = s_lds;
  unsigned char* const s_slotb = s_lds + HBYTES;                  // uint16 [tap][sidx]
  unsigned char* const s_rowb = s_lds + HBYTES + SLOTQ * 1024;    // int32 [slot]

  const int c_in = p.c_in, c_out = p.c_out;
  // Workgroups take the tiles in the plan's order (longest first): the
  // hardware starts them in index order as slots free up, so the shortest
  // tiles and the split parts fill the end.
  const int bid = blockIdx.x;
  int item = bid, part = -1;
  if (bid >= hl.full) {
    item = hl.full + (bid - hl.full) / kHaloParts;
    part = (bid - hl.full) % kHaloParts;
  }
  const int rt = p.order[item / p.n_tiles_n];
  const unsigned char* const rec = p.plan + int64_t(rt) * kPlanBytes;
  if (part >= 0) {
    halo_part<H, TN / 32>(p, rec, part, (item % p.n_tiles_n) * TN, reinterpret_cast<float*>(s_lds));
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hw = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rh = wave / (4 / WR), chf = wave % (4 / WR);
  const int r0 = WROWS * rh;                                // this wave's first row
  const int n0 = (item % p.n_tiles_n) * TN + 32 * CB * chf;  // this wave's first column
  const HaloHeader* const hdr = reinterpret_cast<const HaloHeader*>(rec + kPlanHdr);
  const int nh = hdr->nh;
  // This wave's block masks (its RB 32-row blocks), 4 bits per tap.
  uint64_t bml = 0, bmh = 0;
  {
#pragma unroll
    for (int k = 0; k < 27; ++k) {
      const uint64_t f = (hdr->fm[k] >> (RB * rh)) & ((1u << RB) - 1u);
      if (k < 16) bml |= f << (4 * k);
      else bmh |= f << (4 * (k - 16));
    }
  }
  const int nchunks = c_in / KC;  // even (halo_shape)

  // crow[q]: caller row of this wave's row 64 q + lane (-1: not stored).
  int32_t crow[(RB + 1) / 2];
#pragma unroll
  for (int q = 0; q < (RB + 1) / 2; ++q)
    crow[q] = reinterpret_cast<const int32_t*>(rec + kPlanCrow)[r0 + 64 * q + lane];
  f32x16 acc[RB][CB];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[b][cb][e] = 0.f;

  // B fragments of stage g (chunk g / 27, tap g % 27): steps s = 0, 1 x this
  // wave's column blocks, 16 bytes per lane from one contiguous kilobyte each;
  // the stages' fragments are at a constant stride.
  const int ncb = c_out / 32, cb0 = n0 / 32;
  const uint4* const wf = reinterpret_cast<const uint4*>(p.wp + frag_weight_offset(c_in, c_out)) + cb0 * 64 + lane;
  const int64_t bstride = int64_t(2) * ncb * 64;  // uint4 per stage
  auto load_b = [&](int g, uint4 (&b)[2][CB]) {
    const uint4* f = wf + g * bstride;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) b[s][cb] = f[(s * ncb + cb) * 64];
  };
  // The multiplies of one stage for the blocks in bm, step by step: an
  // accumulator's two products of a stage are a whole step apart, so the
  // second does not wait for the first's result.
  auto mma_stage = [&](uint32_t bm, const hvec (&a)[2][RB], const uint4 (&b)[2][CB]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int blk = 0; blk < RB; ++blk) {
        if ((bm >> blk) & 1u) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[blk][cb] = H::mma32(a[s][blk], *reinterpret_cast<const hvec*>(&b[s][cb]), acc[blk][cb]);
        }
      }
  };
  const int nst = nchunks * 27;  // stages: every chunk runs all 27 taps (a tap no row has multiplies nothing)

  if (nh >= 0) {
    for (int q = wave; q < SLOTQ + ROWQ; q += 4) {
      const bool sl = q < SLOTQ;
      const unsigned char* g =
          sl ? rec + kPlanSlots + q * 1024 + lane * 16 : rec + kPlanRows + (q - SLOTQ) * 1024 + lane * 16;
      copy16_to_lds(g, sl ? s_slotb + q * 1024 : s_rowb + (q - SLOTQ) * 1024);
    }
    __builtin_amdgcn_s_waitcnt(0);
    bare_barrier();
    const int32_t* const s_rows = reinterpret_cast<const int32_t*>(s_rowb);
    // Halo rows of chunk c: slot q*16 + lane/4, piece lane&3 (slot 0 and the
    // slots past the halo read the zero block). The caller rows are read from
    // LDS first, all together, then the copies are issued.
    constexpr int QW = ((kHaloCap + 15) / 16 + 3) / 4;  // copy rounds per wave
    auto fill_halo = [&](int c) {
      const int nq = (nh + 1 + 15) >> 4;
      int32_t rr[QW];
#pragma unroll
      for (int i = 0; i < QW; ++i) {
        const int slot = (wave + 4 * i) * 16 + (lane >> 2);
        rr[i] = slot >= 1 && slot <= nh ? s_rows[slot] : -1;
      }
#pragma unroll
      for (int i = 0; i < QW; ++i) {
        const int q = wave + 4 * i;
        if (q < nq) {
          const int slot = q * 16 + (lane >> 2);
          const int ch = c * KC + (((lane & 3) ^ ((slot >> 2) & 3)) << 3);
          const void* g = rr[i] >= 0 ? static_cast<const void*>(static_cast<const uint16_t*>(p.x) +
                                                                 int64_t(rr[i]) * c_in + ch)
                                     : static_cast<const void*>(p.zeros);
          copy16_to_lds(g, s_halo + q * 1024);
        }
      }
    };
    // LDS offsets of this lane's RB rows (r0 + 32 blk + lane % 32) at tap k
    const unsigned char* const slot_lane = s_slotb + (128 * (r0 >> 7) + l32 * 4 + ((r0 >> 5) & 3)) * 2;
    auto read_slots = [&](int k) {
      if constexpr (RB == 4) return *reinterpret_cast<const uint2*>(slot_lane + k * TM * 2);
      else return uint2{*reinterpret_cast<const uint32_t*>(slot_lane + k * TM * 2), 0u};
    };
    const uint32_t pa = uint32_t(hw) << 4;  // piece 2 s + hw: offset ^ (pa + 32 s)
    auto load_a = [&](uint2 so, hvec (&a)[2][RB]) {
      const uint32_t o4[4] = {so.x & 0xFFFFu, so.x >> 16, so.y & 0xFFFFu, so.y >> 16};
      uint32_t o[RB];
#pragma unroll
      for (int blk = 0; blk < RB; ++blk) o[blk] = o4[blk];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int blk = 0; blk < RB; ++blk)
          a[s][blk] = *reinterpret_cast<const hvec*>(s_halo + (o[blk] ^ (pa + 32u * s)));
    };
    // Registers: A and B fragments in two sets used by alternate stages. A
    // stage multiplies on its set while the next stage's A fragments (read one
    // stage ahead, within a chunk) and the B fragments of the stage after next
    // land in the other set. The slot offsets of a tap are read three stages
    // ahead into one of two registers (by stage parity), so the next stage's A
    // reads wait only for an offset read issued before the previous stage's
    // A reads, not for those reads themselves (LDS reads return in order).
    uint4 b0[2][CB], b1[2][CB];
    hvec a0[2][RB], a1[2][RB];
    load_b(0, b0);
    load_b(1, b1);
    fill_halo(0);
    __builtin_amdgcn_s_waitcnt(0);
    bare_barrier();  // chunk 0's halo has landed
    load_a(read_slots(0), a0);
    uint2 sa = read_slots(1), sb = read_slots(2);  // slots of stages 1 and 2
    // Stage st = 27 c + k. Two stages per iteration (nst is even), so that
    // each stage's register sets are fixed; the stage's loads are issued
    // unconditionally (clamped past the end, read again after a halo refill)
    // so that the waits the compiler places before the multiplies stay exact.
    int c = 0, k = 0;
    auto stage = [&](int st, uint4 (&bc)[2][CB], hvec (&ac)[2][RB], hvec (&an)[2][RB], uint2& so) {
      const uint32_t bm = uint32_t((k < 16 ? bml >> (4 * k) : bmh >> (4 * (k - 16))) & 15u);
      load_a(so, an);                               // the next stage (same chunk unless k == 26)
      so = read_slots(k < 24 ? k + 3 : k - 24);     // three stages ahead
      mma_stage(bm, ac, bc);
      load_b(st + 2 < nst ? st + 2 : st, bc);       // the stage after next
      if (k == 26) {
        if (c + 1 < nchunks) {
          // the next stage opens chunk c + 1: replace the halo once every
          // wave's reads of this chunk are done, then read its first A fragments
          __builtin_amdgcn_s_waitcnt(0xC07F);
          bare_barrier();
          fill_halo(c + 1);
          __builtin_amdgcn_s_waitcnt(0);
          bare_barrier();
          load_a(read_slots(0), an);
        }
        ++c;
        k = 0;
      } else {
        ++k;
      }
    };
    for (int st = 0; st < nst; st += 2) {
      stage(st, b0, a0, a1, sa);
      stage(st + 1, b1, a1, a0, sb);
    }
  } else {
    // Too many distinct neighbours: A fragments straight from global memory.
    // Row r0 + 32 blk + lane % 32: caller row and mask.
    const int32_t* const pc = reinterpret_cast<const int32_t*>(rec + kPlanCrow) + r0;
    const uint32_t* const pm = reinterpret_cast<const uint32_t*>(rec + kPlanMask) + r0;
    int32_t rr[RB];
    uint32_t rm[RB];
#pragma unroll
    for (int blk = 0; blk < RB; ++blk) {
      rr[blk] = pc[32 * blk + l32];
      rm[blk] = pm[32 * blk + l32];
    }
    for (int g = 0; g < nst; ++g) {
      const int c = g / 27, k = g - 27 * (g / 27);
      const uint32_t bm = uint32_t((k < 16 ? bml >> (4 * k) : bmh >> (4 * (k - 16))) & 15u);
      if (bm == 0u) continue;
      uint4 b[2][CB];
      load_b(g, b);
      hvec a[2][RB];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int blk = 0; blk < RB; ++blk) {
          const int32_t j = ((rm[blk] >> k) & 1u) ? p.nbr[int64_t(rr[blk]) * 27 + k] : -1;
          const int ch = c * KC + (2 * s + hw) * 8;
          const void* gp = j >= 0 ? static_cast<const void*>(static_cast<const uint16_t*>(p.x) + int64_t(j) * c_in + ch)
                                  : static_cast<const void*>(p.zeros);
          const uint4 raw = *reinterpret_cast<const uint4*>(gp);
          a[s][blk] = *reinterpret_cast<const hvec*>(&raw);
        }
      }
      mma_stage(bm, a, b);
    }
  }

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  store_tile32<H, RB, CB>(p, acc, crow, n0, reinterpret_cast<float*>(s_halo) + wave * 16 * (32 * CB + 8));
}

// Workgroups that fit on the device at once (two per CU for fwd_halo), per device.
int halo_slots() {
  constexpr int kMaxDev = 64;
  static std::once_flag once[kMaxDev];
  static int slots[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  std::call_once(once[dev], [dev] {
    int cus = 0;
    slots[dev] = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? 2 * cus : 0;
  });
  return slots[dev];
}

template <bool F16, int WR, int CB>
hipError_t launch_halo(const ConvArgs& a, const uint16_t* wp, const uint16_t* zeros, hipStream_t st) {
  constexpr int TM = kHaloTM, TN = 32 * CB * (4 / WR);
  const int64_t mt = (a.n + TM - 1) / TM;
  const int nt = (a.c_out + TN - 1) / TN;
  const int64_t items = mt * nt;
  if (items * kHaloParts > 0x7FFFFFFF) return hipErrorInvalidValue;
  // Split the last round into parts when its parts fit the device's
  // workgroup slots at once.
  HaloLaunch hl{int(items), 0};
  const int64_t slots = halo_slots();
  if (slots > 0 && items > slots) {
    const int64_t last = items - (items - 1) / slots * slots;
    if (last * kHaloParts <= slots) hl = HaloLaunch{int(items - last), int(last)};
  }
  RowsArgs p{a.nbr, a.plan, a.order, a.srows, a.mask, a.n, a.x, wp, zeros, a.y, a.epi.bias, a.epi.residual,
             a.epi.act, a.y_dtype == TR_SC_F32 ? 1 : 0, a.c_in, a.c_out, nt};
  fwd_halo<F16, WR, CB><<<unsigned(hl.full + kHaloParts * hl.split), kThreads, 0, st>>>(p, hl);
  return hipGetLastError();
}

template <int FM, int FN, bool F16>
hipError_t launch_lds(const ConvArgs& a, const uint16_t* wp, const uint16_t* zeros, hipStream_t st) {
  constexpr int TM = 64 * FM, TN = 16 * FN;
  const int64_t mt = (a.n + TM - 1) / TM;
  const int nt = (a.c_out + TN - 1) / TN;
  const int64_t grid = mt * nt;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  RowsArgs p{a.nbr, a.plan, a.order, a.srows, a.mask, a.n, a.x, wp, zeros, a.y, a.epi.bias, a.epi.residual,
             a.epi.act, a.y_dtype == TR_SC_F32 ? 1 : 0, a.c_in, a.c_out, nt};
  fwd_lds<FM, FN, F16><<<unsigned(grid), kThreads, 0, st>>>(p);
  return hipGetLastError();
}

template <int FM, int FN, bool F16, int XT>
hipError_t launch_rows(const ConvArgs& a, const uint16_t* wp, const uint16_t* zeros, hipStream_t st) {
  constexpr int TM = 64 * FM, TN = 16 * FN;
  const int64_t mt = (a.n + TM - 1) / TM;
  const int nt = (a.c_out + TN - 1) / TN;
  const int64_t grid = mt * nt;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  RowsArgs p{a.nbr, a.plan, a.order, a.srows, a.mask, a.n, a.x, wp, zeros, a.y, a.epi.bias, a.epi.residual,
             a.epi.act, a.y_dtype == TR_SC_F32 ? 1 : 0, a.c_in, a.c_out, nt};
  fwd_rows<FM, FN, F16, XT><<<unsigned(grid), kThreads, 0, st>>>(p);
  return hipGetLastError();
}

constexpr int64_t kLdsMinRows = 65536;

template <bool F16>
hipError_t dispatch(const ConvArgs& a, const uint16_t* p, const uint16_t* zeros, hipStream_t st) {
  constexpr int XT = F16 ? 2 : 3;
  if (a.x_dtype == TR_SC_F32) {
    // fp32 features: XT products per multiply; 32-row waves keep the split
    // terms and the wider A fragments within the register budget.
    if (a.c_out >= 128) return launch_rows<2, 8, F16, XT>(a, p, zeros, st);
    if (a.c_out > 32) return launch_rows<2, 4, F16, XT>(a, p, zeros, st);
    if (a.c_out > 16) return launch_rows<2, 2, F16, XT>(a, p, zeros, st);
    return launch_rows<2, 1, F16, XT>(a, p, zeros, st);
  }
  // Wide layers: 64-row waves halve the LDS reads of weight fragments per
  // multiply (the weight slice is read once per wave). Narrow layers: 32-row
  // waves give twice the workgroups and a third wave per SIMD.
  if (halo_shape(a.c_in, a.c_out)) {
    if (a.c_out == 32) return launch_halo<F16, 4, 1>(a, p, zeros, st);
    if (a.c_out == 64) return launch_halo<F16, 4, 2>(a, p, zeros, st);
    return launch_halo<F16, 2, 2>(a, p, zeros, st);
  }
  if (a.c_out >= 128 && a.c_in >= 256) return launch_rows<4, 8, F16, 1>(a, p, zeros, st);
  if (a.c_out >= 128) return launch_rows<2, 8, F16, 1>(a, p, zeros, st);
  // 64-wide layers over a large voxel set (a decoder level): rows through LDS
  // (1.32 -> 1.16 ms per convolution at 3.15M voxels); a small set is
  // latency-bound and keeps the register path.
  if (a.c_out > 32) return a.n >= kLdsMinRows ? launch_lds<2, 4, F16>(a, p, zeros, st)
                                               : launch_rows<2, 4, F16, 1>(a, p, zeros, st);
  if (a.c_out > 16) return launch_lds<4, 2, F16>(a, p, zeros, st);
  return launch_lds<4, 1, F16>(a, p, zeros, st);
}

}  // namespace

hipError_t launch_forward_mfma(const ConvArgs& a, const void* wp, hipStream_t st) {
  const uint16_t* p = static_cast<const uint16_t*>(wp);
  const uint16_t* zeros = p + packed_weight_elems(a.c_in, a.c_out);
  if (a.w_dtype == TR_SC_F16) return dispatch<true>(a, p, zeros, st);
  return dispatch<false>(a, p, zeros, st);
}

}  // namespace trsc
