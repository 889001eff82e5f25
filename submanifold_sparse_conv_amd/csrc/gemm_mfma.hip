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
// K loop: the taps some row of the tile needs (OR of the rows' 27-bit
// neighbour masks), each split into 64-channel chunks ("stages"). Each of the
// four waves owns 16*FM whole rows of the tile and all TN columns, so every
// gathered feature row is read by one wave only: its MFMA A fragments go from
// global memory straight into registers, one stage ahead. The stage's weight
// slice, which all four waves read, is copied into LDS with global_load_lds
// (double-buffered, XOR-swizzled 128-byte rows). Matrix instruction:
// v_mfma_f32_16x16x32_bf16 / _f16.
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
#include "common.h"
#include "launch.h"

namespace trsc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

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

  // Epilogue, fused into the same pass as the pages fuse theirs (bias,
  // activation, residual add and the output rounding -- "Porting TRELLIS.2
  // ...", section V): v = act(acc + bias) in fp32, staged per 16-row block in
  // this wave's LDS region; then each lane adds the residual to 16 bytes' worth
  // of one output row and rounds once, to the output type.
  float bv[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int c = n0 + j * 16 + lr;
    bv[j] = (p.bias != nullptr && c < c_out) ? p.bias[c] : 0.f;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Staged row r (8 per pass) holds TN floats in 16-byte pieces; piece q sits
  // at q ^ osw(r), which puts the two rows one write instruction touches on
  // different banks and keeps each aligned group of four pieces contiguous.
  constexpr int PPR = TN / 4;
  auto spos = [](int r, int q) { return r * TN + ((q ^ (((r >> 2) & 1) << 2 & (PPR - 1))) << 2); };
  float* sO = reinterpret_cast<float*>(bbuf0) + wave * 8 * TN;
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

template <int FM, int FN, bool F16, int XT>
hipError_t launch_rows(const ConvArgs& a, const uint16_t* wp, const uint16_t* zeros, hipStream_t st) {
  constexpr int TM = 64 * FM, TN = 16 * FN;
  const int64_t mt = (a.n + TM - 1) / TM;
  const int nt = (a.c_out + TN - 1) / TN;
  const int64_t grid = mt * nt;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  RowsArgs p{a.nbr, a.srows, a.mask, a.n, a.x, wp, zeros, a.y, a.epi.bias, a.epi.residual,
             a.epi.act, a.y_dtype == TR_SC_F32 ? 1 : 0, a.c_in, a.c_out, nt};
  fwd_rows<FM, FN, F16, XT><<<unsigned(grid), kThreads, 0, st>>>(p);
  return hipGetLastError();
}

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
  if (a.c_out >= 128 && a.c_in >= 256) return launch_rows<4, 8, F16, 1>(a, p, zeros, st);
  if (a.c_out >= 128) return launch_rows<2, 8, F16, 1>(a, p, zeros, st);
  if (a.c_out > 32) return launch_rows<2, 4, F16, 1>(a, p, zeros, st);
  if (a.c_out > 16) return launch_rows<4, 2, F16, 1>(a, p, zeros, st);
  return launch_rows<4, 1, F16, 1>(a, p, zeros, st);
}

}  // namespace

hipError_t launch_forward_mfma(const ConvArgs& a, const void* wp, hipStream_t st) {
  const uint16_t* p = static_cast<const uint16_t*>(wp);
  const uint16_t* zeros = p + packed_weight_elems(a.c_in, a.c_out);
  if (a.w_dtype == TR_SC_F16) return dispatch<true>(a, p, zeros, st);
  return dispatch<false>(a, p, zeros, st);
}

}  // namespace trsc
