// gfx950 (MI355X) kernels for batched Newton–Schulz orthogonalization.
//
//  * gemm_nt_kernel: batched C = A B^T on MFMA (fp16/bf16 32x32x16, fp32
//    32x32x2), fp32 accumulation, LDS double buffering, and a fused fp32
//    epilogue (alpha acc + beta Cin, per-matrix scale, optional transposed
//    store, optional "+ diag * I" second store, non-finite flag).  The
//    symmetric variant runs only tiles on or below the diagonal and writes
//    each result to (i, j) and (j, i); inside a diagonal tile the lower half is
//    written once to both places, so every symmetric output is exactly
//    symmetric (Dion3 paper, Section 5 "Triangular Scheduler" and "Epilogue:
//    Writing to the Transposed Tile"; Appendix C.1 on writing diagonal tiles
//    once).
//  * norm_reduce_kernel / scale_cast_transpose_kernel: the Frobenius
//    normalization X / (s (||X||_F + eps)) and the cast to the compute dtype
//    (Dion3 paper, Alg. 3 steps 2-3), written both as X (n x m) and X^T, with
//    zero padding.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "nsg_internal.h"

namespace nsg {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Mfma;

template <> struct Mfma<NSG_F16> {
  using T = _Float16;
  using frag_t = f16x8;
  static constexpr int KPER = 16;  // K consumed by one MFMA
  static constexpr int FE = 8;     // K elements per lane per MFMA
  static __device__ __forceinline__ f32x16 mma(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<NSG_BF16> {
  using T = __bf16;
  using frag_t = bf16x8;
  static constexpr int KPER = 16;
  static constexpr int FE = 8;
  static __device__ __forceinline__ f32x16 mma(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<NSG_F32> {
  using T = float;
  using frag_t = float;
  static constexpr int KPER = 2;
  static constexpr int FE = 1;
  static __device__ __forceinline__ f32x16 mma(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Round-to-nearest-even conversions from the fp32 epilogue value.
template <typename T> __device__ __forceinline__ T cvt(float v);
template <> __device__ __forceinline__ _Float16 cvt<_Float16>(float v) { return (_Float16)v; }
template <> __device__ __forceinline__ __bf16 cvt<__bf16>(float v) { return (__bf16)v; }
template <> __device__ __forceinline__ float cvt<float>(float v) { return v; }

template <typename T> struct V4 { typedef T type __attribute__((ext_vector_type(4))); };

// Row-major store of a wave's accumulator tiles (values already final), with
// the mirrored store for symmetric launches.  Outside the valid Mv x Nv corner
// zeros are written when `pad`, nothing otherwise.  Inside a diagonal tile only
// the lower half is stored, to both (i, j) and (j, i).  Returns whether every
// valid stored value is finite after rounding.
template <typename TO, bool SYM, int TM, int TN>
__device__ __forceinline__ bool store_tile(const f32x16 (&acc)[TM][TN], TO *o, int64_t ld, int row0, int col0,
                                           int lane, int Mv, int Nv, bool pad, bool diag_tile) {
  bool finite = true;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = col0 + j * 32 + (lane & 31);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int rowb = row0 + i * 32 + 8 * r4 + 4 * (lane >> 5);
        typename V4<TO>::type h;
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = cvt<TO>(acc[i][j][r4 * 4 + q]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = rowb + q;
          const bool valid = row < Mv && col < Nv;
          if ((valid || pad) && (!diag_tile || row >= col)) {
            o[(size_t)row * ld + col] = h[q];
            finite = finite && (!valid || __builtin_isfinite((float)h[q]));
          }
        }
        if constexpr (SYM) {
          if (!diag_tile) {
            *reinterpret_cast<typename V4<TO>::type *>(o + (size_t)col * ld + rowb) = h;
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (rowb + q > col) o[(size_t)col * ld + rowb + q] = h[q];
          }
        }
      }
    }
  }
  return finite;
}

// Transposed store (V^T), 4 consecutive rows of V per lane = 4 contiguous
// elements of V^T.  Workspace output: every element, zeros already in place.
template <typename TO, int TM, int TN>
__device__ __forceinline__ void store_tile_t(const f32x16 (&acc)[TM][TN], TO *o, int64_t ld, int row0, int col0,
                                             int lane) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = col0 + j * 32 + (lane & 31);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int rowb = row0 + i * 32 + 8 * r4 + 4 * (lane >> 5);
        typename V4<TO>::type h;
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = cvt<TO>(acc[i][j][r4 * 4 + q]);
        *reinterpret_cast<typename V4<TO>::type *>(o + (size_t)col * ld + rowb) = h;
      }
    }
}

// ---------------------------------------------------------------------------
// Batched NT GEMM.  Block = WGM x WGN waves; wave tile (BM/WGM) x (BN/WGN)
// made of 32x32 MFMA tiles.  K advances 128 bytes of each operand row per
// stage; LDS rows are padded by 16 bytes so the 16-byte fragment reads of 32
// consecutive rows hit distinct banks.
// ---------------------------------------------------------------------------
template <int DT, int BM, int BN, int WGM, int WGN, bool SYM>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_nt_kernel(const GemmArgs p) {
  using MF = Mfma<DT>;
  using T = typename MF::T;
  using frag_t = typename MF::frag_t;
  constexpr int NT = WGM * WGN * 64;
  constexpr int BK = 128 / (int)sizeof(T);
  constexpr int LDP = BK + 16 / (int)sizeof(T);
  constexpr int CE = 16 / (int)sizeof(T);
  constexpr int CPR = BK / CE;
  constexpr int A_LD = BM * CPR / NT;
  constexpr int B_LD = BN * CPR / NT;
  static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "load split");
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave tile");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T *sA = reinterpret_cast<T *>(smem_raw);
  T *sB = sA + 2 * BM * LDP;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int g = blockIdx.y;

  int tm, tn;
  if constexpr (SYM) {
    // Linear index over the lower triangle (diagonal included), row-major:
    // t = tm (tm + 1) / 2 + tn, 0 <= tn <= tm.
    const int t = blockIdx.x;
    int r = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
    while (r * (r + 1) / 2 > t) --r;
    while ((r + 1) * (r + 2) / 2 <= t) ++r;
    tm = r;
    tn = t - r * (r + 1) / 2;
  } else {
    const int tiles_n = p.N / BN;
    tm = blockIdx.x / tiles_n;
    tn = blockIdx.x - tm * tiles_n;
  }

  const T *gA = reinterpret_cast<const T *>(p.A) + (size_t)g * p.sA + (size_t)tm * BM * p.lda;
  const T *gB = reinterpret_cast<const T *>(p.B) + (size_t)g * p.sB + (size_t)tn * BN * p.ldb;

  u32x4 ra[A_LD], rb[B_LD];
#define NSG_GLOAD(k0)                                                                   \
  do {                                                                                  \
    _Pragma("unroll") for (int i_ = 0; i_ < A_LD; ++i_) {                               \
      const int c_ = tid + i_ * NT;                                                     \
      ra[i_] = *reinterpret_cast<const u32x4 *>(gA + (size_t)(c_ / CPR) * p.lda + (k0) + \
                                               (c_ % CPR) * CE);                        \
    }                                                                                   \
    _Pragma("unroll") for (int i_ = 0; i_ < B_LD; ++i_) {                               \
      const int c_ = tid + i_ * NT;                                                     \
      rb[i_] = *reinterpret_cast<const u32x4 *>(gB + (size_t)(c_ / CPR) * p.ldb + (k0) + \
                                               (c_ % CPR) * CE);                        \
    }                                                                                   \
  } while (0)
#define NSG_SWRITE(stage)                                                                     \
  do {                                                                                        \
    T *a_ = sA + (stage) * BM * LDP;                                                          \
    T *b_ = sB + (stage) * BN * LDP;                                                          \
    _Pragma("unroll") for (int i_ = 0; i_ < A_LD; ++i_) {                                     \
      const int c_ = tid + i_ * NT;                                                           \
      *reinterpret_cast<u32x4 *>(a_ + (c_ / CPR) * LDP + (c_ % CPR) * CE) = ra[i_];           \
    }                                                                                         \
    _Pragma("unroll") for (int i_ = 0; i_ < B_LD; ++i_) {                                     \
      const int c_ = tid + i_ * NT;                                                           \
      *reinterpret_cast<u32x4 *>(b_ + (c_ / CPR) * LDP + (c_ % CPR) * CE) = rb[i_];           \
    }                                                                                         \
  } while (0)

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = p.K / BK;
  NSG_GLOAD(0);
  NSG_SWRITE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) NSG_GLOAD((kt + 1) * BK);
    const T *a = sA + cur * BM * LDP + (wm * WM + (lane & 31)) * LDP + (lane >> 5) * MF::FE;
    const T *b = sB + cur * BN * LDP + (wn * WN + (lane & 31)) * LDP + (lane >> 5) * MF::FE;
#pragma unroll
    for (int ks = 0; ks < BK; ks += MF::KPER) {
      frag_t fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = *reinterpret_cast<const frag_t *>(a + i * 32 * LDP + ks);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = *reinterpret_cast<const frag_t *>(b + j * 32 * LDP + ks);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = MF::mma(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < nk) NSG_SWRITE(cur ^ 1);
    __syncthreads();
  }

  // ---- fp32 epilogue ----
  // Accumulator layout of a 32x32 MFMA tile: lane l, register r holds
  // row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
  float sc = 1.f;
  if (p.gscale != nullptr && p.gpow > 0) {
    const float s = p.gscale[g];
    sc = (p.gpow == 1) ? s : s * s;
  }
  const float alpha = p.alpha * sc, beta = p.beta * sc;
  const int row0 = tm * BM + wm * WM, col0 = tn * BN + wn * WN;
  const T *cin = p.Cin ? reinterpret_cast<const T *>(p.Cin) + (size_t)g * p.sC : nullptr;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = col0 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        float v = alpha * acc[i][j][r];
        if (cin != nullptr) v += beta * (float)cin[(size_t)row * p.ldc + col];
        acc[i][j][r] = (row < p.Mv && col < p.Nv) ? v : 0.f;
      }
    }
  }
  const bool diag_tile = SYM && (tm == tn);
  if (p.out0 != nullptr) {
    bool fin = true;
    if (p.out0_dtype == NSG_F16)
      fin = store_tile<_Float16, SYM, TM, TN>(acc, reinterpret_cast<_Float16 *>(p.out0) + (size_t)g * p.s0, p.ld0,
                                              row0, col0, lane, p.Mv, p.Nv, p.out0_pad != 0, diag_tile);
    else if (p.out0_dtype == NSG_BF16)
      fin = store_tile<__bf16, SYM, TM, TN>(acc, reinterpret_cast<__bf16 *>(p.out0) + (size_t)g * p.s0, p.ld0,
                                            row0, col0, lane, p.Mv, p.Nv, p.out0_pad != 0, diag_tile);
    else
      fin = store_tile<float, SYM, TM, TN>(acc, reinterpret_cast<float *>(p.out0) + (size_t)g * p.s0, p.ld0,
                                           row0, col0, lane, p.Mv, p.Nv, p.out0_pad != 0, diag_tile);
    if (p.status != nullptr && __ballot(!fin) != 0 && lane == 0) p.status[g] = 1;
  }
  if constexpr (!SYM) {
    if (p.out1 != nullptr)
      store_tile_t<T, TM, TN>(acc, reinterpret_cast<T *>(p.out1) + (size_t)g * p.s1, p.ld1, row0, col0, lane);
  }
  if constexpr (SYM) {
    if (p.out2 != nullptr) {
      // second store of the same accumulator with + diag on the (valid) diagonal
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = col0 + j * 32 + (lane & 31);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row == col && row < p.Mv) acc[i][j][r] += p.diag;
          }
        }
      store_tile<T, true, TM, TN>(acc, reinterpret_cast<T *>(p.out2) + (size_t)g * p.s2, p.ld2, row0, col0, lane,
                                  p.Mv, p.Nv, true, diag_tile);
    }
  }
}

#undef NSG_GLOAD
#undef NSG_SWRITE

int tile_m(int cfg) { return cfg == kTile256 ? 256 : 128; }

template <int DT, int BM, int BN, int WGM, int WGN, bool SYM>
static hipError_t launch_one(const GemmArgs &a, hipStream_t s) {
  using T = typename Mfma<DT>::T;
  constexpr int BK = 128 / (int)sizeof(T);
  constexpr int LDP = BK + 16 / (int)sizeof(T);
  const size_t lds = (size_t)2 * (BM + BN) * LDP * sizeof(T);
  auto kern = gemm_nt_kernel<DT, BM, BN, WGM, WGN, SYM>;
  static bool attr_set[64] = {false};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 64 && !attr_set[dev]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  unsigned gx;
  if (SYM) {
    const unsigned t = (unsigned)(a.M / BM);
    gx = t * (t + 1) / 2;
  } else {
    gx = (unsigned)(a.M / BM) * (unsigned)(a.N / BN);
  }
  dim3 grid(gx, (unsigned)a.batch), block(WGM * WGN * 64);
  hipLaunchKernelGGL(kern, grid, block, lds, s, a);
  return hipGetLastError();
}

template <int DT, bool SYM>
static hipError_t launch_cfg(int cfg, const GemmArgs &a, hipStream_t s) {
  if (cfg == kTile256) return launch_one<DT, 256, 256, 2, 2, SYM>(a, s);
  return launch_one<DT, 128, 128, 2, 2, SYM>(a, s);
}

hipError_t launch_gemm(int dtype, bool symmetric, int cfg, const GemmArgs &a, hipStream_t s) {
  if (a.batch == 0 || a.M == 0 || a.N == 0) return hipSuccess;
  switch (dtype) {
    case NSG_F16:
      return symmetric ? launch_cfg<NSG_F16, true>(cfg, a, s) : launch_cfg<NSG_F16, false>(cfg, a, s);
    case NSG_BF16:
      return symmetric ? launch_cfg<NSG_BF16, true>(cfg, a, s) : launch_cfg<NSG_BF16, false>(cfg, a, s);
    default:
      return symmetric ? launch_cfg<NSG_F32, true>(cfg, a, s) : launch_cfg<NSG_F32, false>(cfg, a, s);
  }
}

// ---------------------------------------------------------------------------
// Normalization: fp32 sum of squares with a fixed reduction tree per chunk.
// ---------------------------------------------------------------------------
template <typename TI> __device__ __forceinline__ float to_f32(TI v) { return (float)v; }

__device__ __forceinline__ float block_sum_256(float v, float *red) {
  // fixed-order tree: xor-shuffles inside each wave, then the 4 wave sums
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <typename TI>
__global__ void __launch_bounds__(256) norm_reduce_kernel(const NormReduceArgs p) {
  __shared__ float red[4];
  const int g = blockIdx.y;
  const int64_t start = (int64_t)blockIdx.x * kNormChunk;
  int64_t end = start + kNormChunk;
  if (end > p.elems) end = p.elems;
  const TI *in = reinterpret_cast<const TI *>(p.in) + (size_t)g * p.elems;
  float s = 0.f;
  for (int64_t i = start + threadIdx.x; i < end; i += 256) {
    const float v = to_f32(in[i]);
    s = fmaf(v, v, s);
  }
  s = block_sum_256(s, red);
  if (threadIdx.x == 0) p.partials[(size_t)g * p.nchunks + blockIdx.x] = s;
}

hipError_t launch_norm_reduce(const NormReduceArgs &a, hipStream_t s) {
  if (a.batch == 0 || a.elems == 0) return hipSuccess;
  dim3 grid((unsigned)a.nchunks, (unsigned)a.batch), block(256);
  switch (a.in_dtype) {
    case NSG_F16: hipLaunchKernelGGL(norm_reduce_kernel<_Float16>, grid, block, 0, s, a); break;
    case NSG_BF16: hipLaunchKernelGGL(norm_reduce_kernel<__bf16>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(norm_reduce_kernel<float>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

// Scale by an exact power of two, cast, and write both layouts through a
// 64x64 LDS tile.  Every block recomputes the norm from the partial sums in
// the same fixed order, so all blocks of a matrix agree bit for bit.
template <typename TI, typename TO>
__global__ void __launch_bounds__(256) scale_cast_transpose_kernel(const ScaleArgs p) {
  __shared__ float tile[64][65];
  __shared__ float red[4];
  const int g = blockIdx.z;
  const int tid = threadIdx.x;
  float s = 0.f;
  for (int i = tid; i < p.nchunks; i += 256) s += p.partials[(size_t)g * p.nchunks + i];
  s = block_sum_256(s, red);
  const float nu = sqrtf(s);
  const float kappa = 1.f / (p.safety * (nu + p.eps));
  int e = 0;
  const float r = frexpf(ldexpf(kappa, p.fexp), &e);  // kappa 2^f = r 2^e, r in [0.5, 1)
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
    p.gscale[g] = r;
    if (p.status != nullptr) p.status[g] = 0;
  }
  const int a0 = blockIdx.y * 64, b0 = blockIdx.x * 64;
  const TI *in = reinterpret_cast<const TI *>(p.in) + (size_t)g * (size_t)(p.R * p.C);
#pragma unroll 4
  for (int it = 0; it < 16; ++it) {
    const int idx = it * 256 + tid;
    const int a = idx >> 6, b = idx & 63;
    float v = 0.f;
    if (a0 + a < p.R && b0 + b < p.C) v = to_f32(in[(size_t)(a0 + a) * p.C + (b0 + b)]);
    tile[a][b] = ldexpf(v, e);
  }
  __syncthreads();
  TO *same = reinterpret_cast<TO *>(p.same) + (size_t)g * p.stride;
  TO *swp = reinterpret_cast<TO *>(p.swap) + (size_t)g * p.stride;
#pragma unroll 4
  for (int it = 0; it < 16; ++it) {
    const int idx = it * 256 + tid;
    const int a = idx >> 6, b = idx & 63;
    same[(size_t)(a0 + a) * p.cols_p + (b0 + b)] = cvt<TO>(tile[a][b]);
    swp[(size_t)(b0 + a) * p.rows_p + (a0 + b)] = cvt<TO>(tile[b][a]);
  }
}

template <typename TI>
static void launch_scale_in(const ScaleArgs &a, dim3 grid, hipStream_t s) {
  switch (a.cdtype) {
    case NSG_F16: hipLaunchKernelGGL((scale_cast_transpose_kernel<TI, _Float16>), grid, dim3(256), 0, s, a); break;
    case NSG_BF16: hipLaunchKernelGGL((scale_cast_transpose_kernel<TI, __bf16>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((scale_cast_transpose_kernel<TI, float>), grid, dim3(256), 0, s, a); break;
  }
}

hipError_t launch_scale(const ScaleArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  dim3 grid((unsigned)(a.cols_p / 64), (unsigned)(a.rows_p / 64), (unsigned)a.batch);
  switch (a.in_dtype) {
    case NSG_F16: launch_scale_in<_Float16>(a, grid, s); break;
    case NSG_BF16: launch_scale_in<__bf16>(a, grid, s); break;
    default: launch_scale_in<float>(a, grid, s); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plain copy, for calibrating byte counters.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) copy_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                   size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

hipError_t launch_copy(const void *src, void *dst, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint4 *>(src), reinterpret_cast<uint4 *>(dst), n16);
  return hipGetLastError();
}

}  // namespace nsg
