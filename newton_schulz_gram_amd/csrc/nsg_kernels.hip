// gfx950 (MI355X) kernels for batched Newton–Schulz orthogonalization.
//
//  * gemm256h_kernel (fp16/bf16, 16x16x32 MFMAs), gemm256_kernel (fp32,
//    32x32x2) and gemm_nt_kernel (128 x 128 tiles for small n): batched
//    C = A B^T, fp32 accumulation, LDS double buffering, and a fused fp32
//    epilogue (alpha acc + beta Cin, per-matrix scale, optional transposed
//    store, optional "+ diag * I" second store, non-finite flag).  The
//    symmetric variant runs only tiles on or below the diagonal and writes
//    each result to (i, j) and (j, i); inside a diagonal tile the lower half is
//    written once to both places, so every symmetric output is exactly
//    symmetric (Dion3 paper, Section 5 "Triangular Scheduler" and "Epilogue:
//    Writing to the Transposed Tile"; Appendix C.1 on writing diagonal tiles
//    once).
//  * norm_reduce_kernel, scale_finalize_kernel and scale_cast_transpose16_kernel
//    (16-bit compute dtypes) / scale_cast_transpose_kernel (fp32): the
//    Frobenius normalization X / (s (||X||_F + eps)) and the cast to the
//    compute dtype (Dion3 paper, Alg. 3 steps 2-3), written both as X (n x m)
//    and X^T, with zero padding.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>
#include <type_traits>

#include "nsg_internal.h"

namespace nsg {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void *lds_ptr_t;

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

// fp32 epilogue of one wave's TM x TN accumulator tiles, one 32x32 tile at a
// time (16 values per lane live at once):
//   v = alpha' acc + beta' Cin   (0 outside the valid Mv x Nv corner)
//   out0 = v (row-major; symmetric launches also write the mirror (j, i);
//          inside a diagonal tile only the lower half is stored, to both
//          places, so the result is exactly symmetric)
//   out1 = v^T (general launches), out2 = v + diag I (symmetric launches).
// out0 writes zeros outside the valid corner when out0_pad, nothing otherwise;
// workspace outputs always cover the padding.  Accumulator layout of a 32x32
// MFMA tile: lane l, register r holds row 8 (r/4) + 4 (l/32) + r%4, column
// l%32, so 4 consecutive registers are 4 consecutive rows of one column.
// alpha' and beta' of matrix g: times r^gpow (r = gscale[g]), and times
// 2^(gpow e) as well when the operands are the unscaled input (gexp).  The
// power of two is exact, so reading G in place gives the same values as
// reading the stored X0 = G 2^e.
__device__ __forceinline__ void input_scales(const GemmArgs &p, int g, float &alpha, float &beta) {
  if (p.gscale == nullptr || p.gpow <= 0) return;
  const float sg = p.gscale[g];
  const float sc = (p.gpow == 1) ? sg : sg * sg;
  alpha *= sc;
  beta *= sc;
  if (p.gexp) {
    const int e = reinterpret_cast<const int32_t *>(p.gscale + p.batch)[g];
    if (p.src == kSrcRaw && !raw_exponent_ok(e)) return;  // this matrix reads its scaled copy
    alpha = ldexpf(alpha, p.gpow * e);
    beta = ldexpf(beta, p.gpow * e);
  }
}

template <typename T, typename TO, bool SYM, int TM, int TN>
__device__ __forceinline__ void epilogue(const GemmArgs &p, const f32x16 (&acc)[TM][TN], int g, bool diag_tile,
                                         int row0, int col0, int lane) {
  float alpha = p.alpha, beta = p.beta;
  input_scales(p, g, alpha, beta);
  const T *cin = p.Cin ? reinterpret_cast<const T *>(p.Cin) + (size_t)g * p.sC : nullptr;
  TO *o0 = p.out0 ? reinterpret_cast<TO *>(p.out0) + (size_t)g * p.s0 : nullptr;
  T *o1 = p.out1 ? reinterpret_cast<T *>(p.out1) + (size_t)g * p.s1 : nullptr;
  T *o2 = p.out2 ? reinterpret_cast<T *>(p.out2) + (size_t)g * p.s2 : nullptr;
  const bool pad0 = p.out0_pad != 0;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = col0 + j * 32 + (lane & 31);
      f32x16 v;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        float x = alpha * acc[i][j][r];
        if (cin != nullptr) x = __builtin_fmaf(beta, (float)cin[(size_t)row * p.ldc + col], x);
        v[r] = (row < p.Mv && col < p.Nv) ? x : 0.f;
      }
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int rowb = row0 + i * 32 + 8 * r4 + 4 * (lane >> 5);
        if (o0 != nullptr) {
          typename V4<TO>::type h;
#pragma unroll
          for (int q = 0; q < 4; ++q) h[q] = cvt<TO>(v[r4 * 4 + q]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = rowb + q;
            const bool valid = row < p.Mv && col < p.Nv;
            if ((valid || pad0) && (!diag_tile || row >= col)) {
              o0[(size_t)row * p.ld0 + col] = h[q];
              finite = finite && (!valid || __builtin_isfinite((float)h[q]));
            }
          }
          if constexpr (SYM) {
            if (!diag_tile) {
              *reinterpret_cast<typename V4<TO>::type *>(o0 + (size_t)col * p.ld0 + rowb) = h;
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (rowb + q > col) o0[(size_t)col * p.ld0 + rowb + q] = h[q];
            }
          }
        }
        if constexpr (!SYM) {
          if (o1 != nullptr) {
            typename V4<T>::type h;
#pragma unroll
            for (int q = 0; q < 4; ++q) h[q] = cvt<T>(v[r4 * 4 + q]);
            *reinterpret_cast<typename V4<T>::type *>(o1 + (size_t)col * p.ld1 + rowb) = h;
          }
        }
        if constexpr (SYM) {
          if (o2 != nullptr) {
            typename V4<T>::type h;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int row = rowb + q;
              h[q] = cvt<T>((row == col && row < p.Mv) ? v[r4 * 4 + q] + p.diag : v[r4 * 4 + q]);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (!diag_tile || rowb + q >= col) o2[(size_t)(rowb + q) * p.ld2 + col] = h[q];
            if (!diag_tile) {
              *reinterpret_cast<typename V4<T>::type *>(o2 + (size_t)col * p.ld2 + rowb) = h;
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (rowb + q > col) o2[(size_t)col * p.ld2 + rowb + q] = h[q];
            }
          }
        }
      }
    }
  }
  if (p.status != nullptr && __ballot(!finite) != 0 && lane == 0) p.status[g] = 1;
}

template <typename T, bool SYM, int TM, int TN>
__device__ __forceinline__ void run_epilogue(const GemmArgs &p, const f32x16 (&acc)[TM][TN], int g, bool diag_tile,
                                             int row0, int col0, int lane) {
  if constexpr (SYM) {
    // symmetric products only ever write workspace buffers (compute dtype)
    epilogue<T, T, SYM, TM, TN>(p, acc, g, diag_tile, row0, col0, lane);
    return;
  }
  if (p.out0_dtype == NSG_F16)
    epilogue<T, _Float16, SYM, TM, TN>(p, acc, g, diag_tile, row0, col0, lane);
  else if (p.out0_dtype == NSG_BF16)
    epilogue<T, __bf16, SYM, TM, TN>(p, acc, g, diag_tile, row0, col0, lane);
  else
    epilogue<T, float, SYM, TM, TN>(p, acc, g, diag_tile, row0, col0, lane);
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
  run_epilogue<T, SYM, TM, TN>(p, acc, g, SYM && (tm == tn), tm * BM + wm * WM, tn * BN + wn * WN, lane);
}

#undef NSG_GLOAD
#undef NSG_SWRITE

// ---------------------------------------------------------------------------
// 256x256 batched NT GEMM for large matrices on 32x32 MFMA tiles (the fp32
// path; fp16 / bf16 use gemm256h_kernel below).  NW waves (2 along M), each
// owning a 128 x (512/NW) block of 32x32 MFMA tiles (NW = 4: 128x128, 256
// fp32 accumulators per lane).  Operands stream global -> LDS with direct
// loads (global_load_lds_dwordx4, no register staging) in stages of 128-byte
// row slices (64 fp16 / bf16 or 32 fp32 K elements), double buffered; the
// loads of stage k+1 are in flight while stage k feeds the MFMAs.  Whole
// 128-byte lines matter: measured L2 -> LDS throughput with half-line (64 B)
// row segments is half that with full lines.
//
// LDS layout of one 256-row operand slice: row-major, 128 bytes (8 16-byte
// chunks) per row, chunk c of row r stored at chunk slot c ^ f(r),
// f(r) = (r ^ (r >> 3)) & 7.  A direct-load instruction fills 1 KB = 8 rows,
// each group of 8 consecutive lanes reading one row's 128 contiguous bytes;
// the swizzle spreads an MFMA fragment read of 16 (or 8) consecutive rows at
// one chunk over distinct banks.
//
// Tile order: tile_256 below (groups of 4 tile rows for general products,
// 8 x 8-tile super-blocks of the lower triangle for symmetric ones; each XCD
// takes 32 consecutive tiles of that order at a time).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int slice_swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_slice_off(int r, int c) { return r * 128 + ((c ^ slice_swz(r)) << 4); }

// One direct global -> LDS load of 16 bytes per lane: lane l reads
// base + voff (bytes) and writes LDS bytes [lds + 16 l, lds + 16 l + 16).
// Issued as inline assembly so that the compiler does not add waits for it
// before unrelated LDS reads; the kernel waits (vmcnt) and synchronizes itself
// before reading a stage.
__device__ __forceinline__ void lds_dma16(const void *base, unsigned voff, const void *lds) {
  const unsigned m0v = (unsigned)(size_t)(lds_ptr_t)lds;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(m0v) : "memory");
}

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt left unconstrained (gfx9 encoding).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// 4-byte load per lane from its own 64-bit address into LDS at m0 + 4 lane:
// used only to pull lines into the caches ahead of the direct loads.
__device__ __forceinline__ void lds_touch4(const void *addr, const void *lds) {
  const unsigned m0v = (unsigned)(size_t)(lds_ptr_t)lds;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(addr), "s"(m0v) : "memory");
}
// All of this wave's LDS reads have returned their data.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier that the compiler may not move memory accesses across and
// that implies no wait on outstanding loads (the callers wait explicitly).
__device__ __forceinline__ void raw_barrier() { asm volatile("s_barrier" ::: "memory"); }

constexpr int kStages256 = 2;
// stages between a prefetched slice and its direct load
constexpr int kPrefetchAhead = 2;

// Epilogue stores (16-byte vectors of 8 16-bit values, or of 4 floats).
// General products stream their output tiles past the caches (non-temporal
// stores; cached ones measured about 45% slower on the general 4096 x 4096
// products of an earlier epilogue).  Symmetric products, which store each
// block to two places, use plain stores: with the non-temporal hint their
// epilogues took 16-22% more cycles per tile (calls: GPT-2-small bucket 2.9%
// and MoE bucket 1.3% slower, the others unchanged).
template <bool SYM, typename V> __device__ __forceinline__ void st_out(const V &v, V *p) {
  if constexpr (SYM) *p = v;
  else __builtin_nontemporal_store(v, p);
}

template <typename TO> struct Vec16 { typedef TO type __attribute__((ext_vector_type(16 / sizeof(TO)))); };

// Epilogue of a 256x256 tile through LDS, in two passes of 128 rows.  The
// fp32 tile is staged column-major: column c at c * PITCH floats (PITCH =
// 132), its rows rotated by stage_rot(c) (+4 or -4 rows modulo 128 when bit 3
// of c is set, by bit 0).  The staging writes (16 consecutive columns, one
// 4-row chunk, per 16 lanes) and the block reads below (16 lanes = columns c
// and c + 8, 8 row chunks) then both hit 16 distinct 4-bank groups; without
// the rotation the reads collide 2-way.
//   A: the waves owning the pass's rows write their accumulators.
//   B: thread (rb, cb) = (lane % 8, lane / 8) of wave w owns two 8 x 8 blocks
//      of the pass, at rows 64 (r & 1) + 8 rb and columns 64 (r >> 1) + 8 cb
//      for regions r = w and w + 4.  It reads a block with 16-byte LDS reads
//      (8 rows of one column each), forms v = alpha' acc + beta' Cin (Cin:
//      8 rows of 16 bytes per block, the first block loaded before the
//      staging, the second at the start of the first; v = 0 outside the valid
//      Mv x Nv corner) and stores its 8 rows to out0 (and out2 = v + diag I)
//      and its 8 columns to the transposed copy (the mirror of a symmetric
//      product, or out1) as 16-byte vectors: the 8 lanes of equal rb (rows)
//      or of equal cb (columns) fill 128-byte lines.  out0 writes zeros
//      outside the valid corner when out0_pad, nothing otherwise; blocks that
//      cross the corner, or an out0 that does not take 16-byte stores, store
//      element by element.
// CIN (Cin given) is a template argument: with a run-time test, the wait
// counts the compiler derives for the Cin loads merge with those of a path
// without them, and the first block then waits for loads issued just before
// it.
// Inside a diagonal tile of a symmetric product a block lies below the
// diagonal (stored whole, to both places), above it (skipped: its mirror
// partner stores it) or on it (its lower half, to both places), so the output
// is exactly symmetric.  The non-finite check of out0 (valid elements only)
// runs only when a status array is given.
// Phase A writers: one wave's 128 x 128 accumulators into the column-major
// staging area (16-byte writes of 4 consecutive rows of one column).
// 32x32 MFMA tiles: lane l, register r = row 8 (r/4) + 4 (l/32) + r%4, column l%32.
// Row rotation of a staged column: columns with bit 3 set move their rows by
// +4 (bit 0 clear) or -4 (bit 0 set), modulo 128.
__device__ __forceinline__ int stage_rot(int col) { return (col & 8) ? ((col & 1) ? -4 : 4) : 0; }
template <int PITCH, int TN>
__device__ __forceinline__ void stage_acc(const f32x16 (&acc)[4][TN], float *lds, int wn, int lane) {
  const int sw = stage_rot(lane);  // the low 5 bits of the lane's column are lane % 32
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      float *col = lds + (wn * TN * 32 + j * 32 + (lane & 31)) * PITCH;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4 *>(col + ((i * 32 + 4 * (lane >> 5) + 8 * r4 + sw) & 127)) =
            make_float4(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]);
    }
}
// 16x16 MFMA tiles: lane l, register r = row 4 (l/16) + r, column l%16.
template <int PITCH, int TN>
__device__ __forceinline__ void stage_acc(const f32x4 (&acc)[8][TN], float *lds, int wn, int lane) {
  const int sw = stage_rot(lane);  // the low 4 bits of the lane's column are lane % 16
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      *reinterpret_cast<float4 *>(lds + (wn * TN * 16 + j * 16 + (lane & 15)) * PITCH +
                                  ((i * 16 + 4 * (lane >> 4) + sw) & 127)) =
          make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
}

// Column passes (256 x 256 kernel): pass P stages every row of the tile for
// columns 64 P .. 64 P + 63 of each wave column (wn 128 + ...), so all four
// waves write a quarter (their column blocks 4 P .. 4 P + 3) at once.  Staged
// column s = 64 wn + 16 jj + lane % 16 holds rows 0..255, rotated modulo 256.
template <int PITCH, int P>
__device__ __forceinline__ void stage_acc_cols(const f32x4 (&acc)[8][8], float *lds, int wm, int wn, int lane) {
  const int sw = stage_rot(lane);  // the low 4 bits of the staged column are lane % 16
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 &a = acc[i][4 * P + jj];
      *reinterpret_cast<float4 *>(lds + (wn * 64 + jj * 16 + (lane & 15)) * PITCH +
                                  ((wm * 128 + i * 16 + 4 * (lane >> 4) + sw) & 255)) = make_float4(a[0], a[1], a[2], a[3]);
    }
}

// Bits of the smallest positive fp32 value that rounds (to nearest even) to
// infinity in TO: 65520 for fp16, 0x1.FFp127 for bf16 (halfway above the
// largest bf16, and a tie rounds to the even infinity), +inf for fp32.
template <typename TO> __device__ __forceinline__ constexpr unsigned overflow_bits();
template <> __device__ __forceinline__ constexpr unsigned overflow_bits<_Float16>() { return 0x477FF000u; }
template <> __device__ __forceinline__ constexpr unsigned overflow_bits<__bf16>() { return 0x7F7F8000u; }
template <> __device__ __forceinline__ constexpr unsigned overflow_bits<float>() { return 0x7F800000u; }

// CINB: Cin is the caller's bf16 input; each value enters as the fp16 X0 the
// scale pass would store, RNE(x 2^e[g]).
template <typename T, typename TO, bool SYM, bool CIN, int NW, int PITCH, bool CP, bool CINB, typename ACC>
__device__ __forceinline__ void staged_epilogue_t(const GemmArgs &p, const ACC &acc, float *lds, int g,
                                                  int tm, int tn, int wm, int wn, int lane, int tid) {
  static_assert(PITCH % 4 == 0, "16-byte staging writes");
  static_assert(NW == 4, "two 8 x 8 blocks per thread and pass");
  constexpr int SR = CP ? 256 : 128;  // staged rows (a power of two)
  static_assert(PITCH >= SR + 4, "one staged column per PITCH floats");
  constexpr int VT = 16 / (int)sizeof(T);   // elements of T per 16 bytes
  constexpr int VO = 16 / (int)sizeof(TO);  // elements of TO per 16 bytes
  constexpr int NV = 8 / VT;                // 16-byte vectors of T per 8 elements
  typedef typename Vec16<T>::type vt_t;
  typedef typename Vec16<TO>::type vo_t;
  float alpha = p.alpha, beta = p.beta;
  input_scales(p, g, alpha, beta);
  const T *cin = CIN ? reinterpret_cast<const T *>(p.Cin) + (size_t)g * p.sC : nullptr;
  static_assert(!CINB || (CIN && sizeof(T) == 2), "a bf16 Cin replaces a 16-bit one");
  const int cex = CINB ? reinterpret_cast<const int32_t *>(p.gscale + p.batch)[g] : 0;
  auto cin_value = [&](T v) -> float {
    if constexpr (CINB) {
      const float x = __builtin_bit_cast(float, (unsigned)__builtin_bit_cast(unsigned short, v) << 16);
      return (float)(_Float16)ldexpf(x, cex);
    } else {
      return (float)v;
    }
  };
  TO *o0 = p.out0 ? reinterpret_cast<TO *>(p.out0) + (size_t)g * p.s0 : nullptr;
  // the transposed copy and out2: TO for symmetric products (whose outputs
  // all take one dtype), the compute dtype T for general ones
  using TA = std::conditional_t<SYM, TO, T>;
  static_assert(sizeof(TA) == sizeof(T), "16-byte vectors of TA hold VT elements");
  typedef typename Vec16<TA>::type va_t;
  T *o1 = p.out1 ? reinterpret_cast<T *>(p.out1) + (size_t)g * p.s1 : nullptr;
  TA *o2 = (SYM && p.out2) ? reinterpret_cast<TA *>(p.out2) + (size_t)g * p.s2 : nullptr;
  TA *ot = SYM ? reinterpret_cast<TA *>(o0) : reinterpret_cast<TA *>(o1);
  const int64_t ldt = SYM ? p.ld0 : p.ld1;
  const bool pad0 = p.out0_pad != 0;
  const bool chk = p.status != nullptr;
  const bool diag_tile = SYM && (tm == tn);
  // 16-byte row stores need the row pitch and base of out0 to allow them
  const bool vec0 = o0 != nullptr && (p.ld0 % VO) == 0 && ((reinterpret_cast<uintptr_t>(o0) & 15) == 0);
  const int wave = tid >> 6;
  const int rb = lane & 7, cb = lane >> 3;
  bool finite = true;
  vt_t cinv[2][8][NV];  // Cin of the thread's block it of a pass
  // region reg of a pass: rows and columns of the tile it covers
  auto reg_row = [&](int pass, int reg) { return CP ? (reg & 3) * 64 : pass * 128 + (reg & 1) * 64; };
  auto reg_col = [&](int pass, int reg) { return CP ? (reg >> 2) * 128 + pass * 64 : (reg >> 1) * 64; };
  auto load_cin = [&](int pass, int it) {
    const int reg = wave + 4 * it;
    const T *cp = cin + (size_t)(tm * 256 + reg_row(pass, reg) + 8 * rb) * p.ldc + (tn * 256 + reg_col(pass, reg) + 8 * cb);
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int e = 0; e < NV; ++e) cinv[it][r][e] = *reinterpret_cast<const vt_t *>(cp + (size_t)r * p.ldc + e * VT);
  };
  auto run_pass = [&](auto pass_c) {
    const int pass = pass_c;
    if constexpr (CIN) load_cin(pass, 0);
    // ---- A: accumulators -> LDS ----
    if constexpr (CP) {
      stage_acc_cols<PITCH, decltype(pass_c)::value>(acc, lds, wm, wn, lane);
    } else {
      if (wm == pass) stage_acc<PITCH>(acc, lds, wn, lane);
    }
    __syncthreads();
    // ---- B: 8 x 8 blocks ----
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      if constexpr (CIN) { if (it == 0) load_cin(pass, 1); }
      const int reg = wave + 4 * it;
      // staged row rr and column cc of the block, and its place in the output
      const int rr = (CP ? (reg & 3) * 64 : (reg & 1) * 64) + 8 * rb, cc = (reg >> (CP ? 2 : 1)) * 64 + 8 * cb;
      const int grow = tm * 256 + reg_row(pass, reg) + 8 * rb, gcol = tn * 256 + reg_col(pass, reg) + 8 * cb;
      const bool full = grow + 8 <= p.Mv && gcol + 8 <= p.Nv;  // every element of the block is valid
      float v[8][8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float *src = lds + (cc + c) * PITCH;
        const int rot = (cb & 1) ? ((c & 1) ? -4 : 4) : 0;  // stage_rot(cc + c)
        const float4 x0 = *reinterpret_cast<const float4 *>(src + ((rr + rot) & (SR - 1)));
        const float4 x1 = *reinterpret_cast<const float4 *>(src + ((rr + 4 + rot) & (SR - 1)));
        v[0][c] = x0.x; v[1][c] = x0.y; v[2][c] = x0.z; v[3][c] = x0.w;
        v[4][c] = x1.x; v[5][c] = x1.y; v[6][c] = x1.z; v[7][c] = x1.w;
      }
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          // one fixed rounding: fma(beta', Cin, alpha' acc), whatever the
          // compiler would contract
          float x = alpha * v[r][c];
          if constexpr (CIN) x = __builtin_fmaf(beta, cin_value(cinv[it][r][c / VT][c % VT]), x);
          v[r][c] = x;
        }
      if (!full) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int c = 0; c < 8; ++c)
            if (!(grow + r < p.Mv && gcol + c < p.Nv)) v[r][c] = 0.f;
      }
      if (chk) {
        // v is 0 outside the valid corner, so the block's largest |v| decides:
        // cvt<TO>(v) is non-finite iff |v| (as fp32 bits, NaN above +inf)
        // reaches TO's overflow threshold (the first value that rounds to inf)
        unsigned m = 0;
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int c = 0; c < 8; ++c) m = max(m, __builtin_bit_cast(unsigned, v[r][c]) & 0x7FFFFFFFu);
        finite = finite && m < overflow_bits<TO>();
      }
      // 0: off the diagonal or below it; 1: on it; 2: above it
      const int cls = !diag_tile ? 0 : (grow >= gcol + 8 ? 0 : (grow == gcol ? 1 : 2));
      // per-block bases; rows and columns step by uniform pitches
      TO *const b0 = o0 + (size_t)grow * p.ld0 + gcol;
      TA *const bt = ot + (size_t)gcol * ldt + grow;
      TA *const b2r = o2 + (size_t)grow * p.ld2 + gcol;
      TA *const b2c = o2 + (size_t)gcol * p.ld2 + grow;
      if (cls == 0) {
        if (o0 != nullptr) {
          if (vec0 && full) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
              for (int e = 0; e < 8 / VO; ++e) {
                vo_t w;
#pragma unroll
                for (int q = 0; q < VO; ++q) w[q] = cvt<TO>(v[r][e * VO + q]);
                st_out<SYM>(w, reinterpret_cast<vo_t *>(b0 + (size_t)r * p.ld0 + e * VO));
              }
          } else {
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
              for (int c = 0; c < 8; ++c)
                if (pad0 || (grow + r < p.Mv && gcol + c < p.Nv))
                  st_out<SYM>(cvt<TO>(v[r][c]), b0 + (size_t)r * p.ld0 + c);
          }
        }
        if (o2 != nullptr) {
#pragma unroll
          for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int e = 0; e < NV; ++e) {
              va_t w;
#pragma unroll
              for (int q = 0; q < VT; ++q) w[q] = cvt<TA>(v[r][e * VT + q]);
              st_out<SYM>(w, reinterpret_cast<va_t *>(b2r + (size_t)r * p.ld2 + e * VT));
            }
        }
        if (ot != nullptr) {  // columns: the transposed copy (and out2's mirror)
#pragma unroll
          for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int e = 0; e < NV; ++e) {
              va_t w;
#pragma unroll
              for (int q = 0; q < VT; ++q) w[q] = cvt<TA>(v[e * VT + q][c]);
              st_out<SYM>(w, reinterpret_cast<va_t *>(bt + (size_t)c * ldt + e * VT));
              if (o2 != nullptr) st_out<SYM>(w, reinterpret_cast<va_t *>(b2c + (size_t)c * p.ld2 + e * VT));
            }
        }
      } else if (cls == 1) {
        // On the diagonal: the block is made exactly symmetric from its lower
        // half (w[r][c] = v[max(r, c)][min(r, c)]) and stored as 8 rows; its
        // transposed place is itself.  Every element gets the value the lower
        // half holds, as if the lower half were stored to both places, with
        // whole-row stores instead of one store per element.
        float w[8][8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int c = 0; c < 8; ++c) w[r][c] = c <= r ? v[r][c] : v[c][r];
        if (o0 != nullptr) {
          if (vec0 && full) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
              for (int e = 0; e < 8 / VO; ++e) {
                vo_t x;
#pragma unroll
                for (int q = 0; q < VO; ++q) x[q] = cvt<TO>(w[r][e * VO + q]);
                st_out<SYM>(x, reinterpret_cast<vo_t *>(b0 + (size_t)r * p.ld0 + e * VO));
              }
          } else {
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
              for (int c = 0; c < 8; ++c)
                if (pad0 || (grow + r < p.Mv && gcol + c < p.Nv))
                  st_out<SYM>(cvt<TO>(w[r][c]), b0 + (size_t)r * p.ld0 + c);
          }
        }
        if (o2 != nullptr) {  // + diag on the valid diagonal
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            va_t x[NV];
#pragma unroll
            for (int c = 0; c < 8; ++c)
              x[c / VT][c % VT] = cvt<TA>((r == c && grow + r < p.Mv) ? w[r][c] + p.diag : w[r][c]);
#pragma unroll
            for (int e = 0; e < NV; ++e) st_out<SYM>(x[e], reinterpret_cast<va_t *>(b2r + (size_t)r * p.ld2 + e * VT));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (pass == 0) __syncthreads();  // LDS is rewritten by the next pass
  };
  if constexpr (CP) {  // compile-time passes: their staging reads fixed accumulator columns
    run_pass(std::integral_constant<int, 0>{});
    run_pass(std::integral_constant<int, 1>{});
  } else {  // a run-time loop (unrolled, the symmetric epilogues spill)
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) run_pass(pass);
  }
  if (chk && __ballot(!finite) != 0 && lane == 0) p.status[g] = 1;
}

// TS: the dtype of a symmetric product's outputs (the compute dtype, or fp16
// for the bf16-MFMA product of a raw bf16 input)
template <typename T, bool SYM, bool CIN, int NW, int PITCH, bool CP = false, typename TS = T, bool CINB = false,
          typename ACC>
__device__ __forceinline__ void staged_epilogue(const GemmArgs &p, const ACC &acc, float *lds, int g,
                                                int tm, int tn, int wm, int wn, int lane, int tid) {
  if constexpr (SYM) {
    staged_epilogue_t<T, TS, true, CIN, NW, PITCH, CP, CINB>(p, acc, lds, g, tm, tn, wm, wn, lane, tid);
  } else {
    if (p.out0_dtype == NSG_F16)
      staged_epilogue_t<T, _Float16, false, CIN, NW, PITCH, CP, CINB>(p, acc, lds, g, tm, tn, wm, wn, lane, tid);
    else if (p.out0_dtype == NSG_BF16)
      staged_epilogue_t<T, __bf16, false, CIN, NW, PITCH, CP, CINB>(p, acc, lds, g, tm, tn, wm, wn, lane, tid);
    else
      staged_epilogue_t<T, float, false, CIN, NW, PITCH, CP, CINB>(p, acc, lds, g, tm, tn, wm, wn, lane, tid);
  }
}


// Block id -> (matrix, tile) of the 256 x 256 kernels.  Workgroups reach the
// XCDs round-robin (block L on XCD L % 8).  Rounds of 8 x 32 consecutive tiles
// are split so XCD x takes chunk x (32 tiles = the workgroups it runs at once;
// for a general product a 4 x 8 block of the grouped order below): the 8 XCDs
// then work on neighbouring tiles of the same matrix, whose operands stay in
// the shared last-level cache, while each XCD's 32 tiles share operand panels
// in its own L2.  (Giving each XCD whole matrices instead measured slower: the
// shared last-level-cache hits are lost.)  The rem < 256 tiles of a last,
// partial round (all of a launch smaller than one round) are split the same
// way into 8 runs, one per XCD, as long as the XCD's share of those
// workgroups: XCD x has q + (x < r) of them (q = rem / 8, r = rem % 8), so its
// run starts at x q + min(x, r).  Neighbouring tiles then share an XCD's L2 in
// a partial round too (a launch of 42 matrices of 3 x 3 tiles: 252 tiles).
template <bool SYM>
__device__ __forceinline__ void tile_256(const GemmArgs &p, unsigned L, unsigned total, int &g, int &tm, int &tn) {
  constexpr unsigned CH = 32, ROUND = 8 * CH;
  const unsigned full = total / ROUND;
  unsigned V;
  const unsigned xcd = L & 7u, slot = L >> 3;
  if (L < full * ROUND) {
    V = (slot / CH) * ROUND + xcd * CH + (slot % CH);
  } else {
    const unsigned rem = total - full * ROUND, q = rem >> 3, r = rem & 7u;
    V = full * ROUND + xcd * q + min(xcd, r) + (slot % CH);
  }
  const int tiles_m = p.M >> 8, tiles_n = p.N >> 8;
  const int tiles = SYM ? tiles_m * (tiles_m + 1) / 2 : tiles_m * tiles_n;
  g = (int)(V / (unsigned)tiles);
  const int t = (int)(V - (unsigned)g * (unsigned)tiles);
  if constexpr (SYM) {
    // Lower triangle (diagonal included) in 8 x 8-tile super-blocks taken
    // row by row; inside a super-block, column by column (the lower half of
    // a diagonal one).  32 consecutive tiles then share fewer operand panels
    // than rows of the triangle would (L2 hit rate 72.6 -> 74.2% at K = 4096,
    // 68.4 -> 71.9% at K = 11008 on the 7B bucket).
    int u = t, I = 0;
    for (;; ++I) {
      const int R = min(8, tiles_m - 8 * I);
      const int row_tiles = I * 8 * R + R * (R + 1) / 2;
      if (u < row_tiles) break;
      u -= row_tiles;
    }
    const int R = min(8, tiles_m - 8 * I);
    if (u < I * 8 * R) {  // off-diagonal super-block (I, J), R rows x 8 columns
      const int J = u / (8 * R), v = u - J * 8 * R;
      tm = 8 * I + v % R;
      tn = 8 * J + v / R;
    } else {  // diagonal super-block: column c holds R - c tiles
      int v = u - I * 8 * R, c = 0;
      while (v >= R - c) {
        v -= R - c;
        ++c;
      }
      tm = 8 * I + c + v;
      tn = 8 * I + c;
    }
  } else {
    constexpr int GM = 4;
    const int in_group = GM * tiles_n;
    const int first = (t / in_group) * GM;
    const int gsz = min(tiles_m - first, GM);
    const int w = t - (t / in_group) * in_group;
    tm = first + w % gsz;
    tn = w / gsz;
  }
}

template <int DT, bool SYM, int NW>
__global__ void __launch_bounds__(NW * 64, 1) gemm256_kernel(const GemmArgs p) {
  using MF = Mfma<DT>;
  using T = typename MF::T;
  using frag_t = typename MF::frag_t;
  constexpr int ES = (int)sizeof(T);
  constexpr int BK = 128 / ES;       // K elements per stage (128-byte row slices)
  constexpr int CE = 16 / ES;        // elements per 16-byte chunk
  constexpr int SLICE = 256 * 128;   // bytes of one operand slice
  constexpr int STAGE = 2 * SLICE;   // A slice then B slice
  constexpr int NST = kStages256;
  constexpr int S = BK / MF::KPER;   // MFMA K-steps per stage
  constexpr int WGN = NW / 2;        // waves along N (2 along M)
  constexpr int WN = 256 / WGN;      // wave tile: 128 x WN
  constexpr int TN = WN / 32;
  constexpr int NLD = 32 / NW;       // 1 KB direct loads per operand per wave per stage
  static_assert(NLD >= 1 && 32 % NW == 0, "waves");
  constexpr int EPI_PITCH = 132;  // floats per staged column (128 rows + 4)
  constexpr int EPI_BYTES = 256 * EPI_PITCH * 4;
  constexpr int LDS_BYTES = NST * STAGE > EPI_BYTES ? NST * STAGE : EPI_BYTES;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[LDS_BYTES + 256];  // + prefetch sink

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  int g, tm, tn;
  tile_256<SYM>(p, blockIdx.x, gridDim.x, g, tm, tn);

  // ---- direct-load sources: wave w fills the 1 KB blocks b = w + NW i of
  //      each slice (rows 8 b .. 8 b + 7; lane l writes chunk slot l % 8 of
  //      row 8 b + l / 8, i.e. logical chunk (l % 8) ^ f(row)) ----
  const T *gA = reinterpret_cast<const T *>(p.A) + (size_t)g * p.sA + (size_t)tm * 256 * p.lda;
  const T *gB = reinterpret_cast<const T *>(p.B) + (size_t)g * p.sB + (size_t)tn * 256 * p.ldb;
  unsigned offA[NLD], offB[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int b = wave + NW * i;
    const int row = b * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ slice_swz(row);
    offA[i] = (unsigned)((row * (int)p.lda + chunk * CE) * ES);
    offB[i] = (unsigned)((row * (int)p.ldb + chunk * CE) * ES);
  }
  // Cache prefetch (wave 0 only): one 4-byte touch per row for an eighth of
  // the rows of each operand panel, kPrefetchAhead stages ahead of the direct
  // loads.  The tiles that share a panel (neighbours in the grouped order)
  // touch different eighths, so together they bring whole slices from HBM
  // into the last-level cache and L2 before any of them needs them.
  const int nk = p.K / BK;  // >= 2: K is a multiple of 256
  const T *pf_ptr = lane < 32 ? gA + (size_t)((tn & 7) + 8 * lane) * p.lda
                              : gB + (size_t)((tm & 7) + 8 * (lane - 32)) * p.ldb;
  auto prefetch = [&](int kt) {
    if (wave == 0) lds_touch4(pf_ptr + (size_t)(kt < nk ? kt : nk - 1) * BK, lds + LDS_BYTES);
  };

  // ---- fragment reads: lane l reads row (block row + l%32) at K element
  //      ks + (l/32) FE of the stage ----
  const int rA = wm * 128 + (lane & 31), rB = wn * WN + (lane & 31);
  const int h = lane >> 5;
  auto frag_off = [&](int rbase, int i, int s) -> int {
    const int k = s * MF::KPER + h * MF::FE;
    return lds_slice_off(rbase + i * 32, k / CE) + (k % CE) * ES;
  };
  f32x16 acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Pipeline over stages k (slot k % 2).  K-step s of a stage runs its
  // 4 x TN MFMAs while the fragments of K-step s+1 are read, one read next to
  // each of the first 4 + TN MFMAs.  Once every wave holds the last K-step of
  // stage k in registers (barrier A, halfway through K-step S-2), slot k % 2
  // is refilled with stage k+2.  The 2 NLD direct loads of a stage are spread
  // at one per two MFMAs over the rest of stage k and K-step 0 of stage k+1,
  // so the address unit never queues a wave's MFMA issue behind a burst of
  // loads.  Barrier B (after K-step S-2) publishes stage k+1, whose loads all
  // left one stage earlier.
  static_assert(NST == 2, "the pipeline below is a double buffer");
  static_assert(S >= 4 && S % 2 == 0, "K-steps per stage");
  constexpr int NQ = 2 * NLD;                  // direct-load instructions per wave per stage
  constexpr int Q1 = TN, Q2 = 2 * TN, Q3 = NQ - Q1 - Q2;
  static_assert(Q3 >= 0 && Q3 <= 2 * TN, "load spread");
  auto dma_q = [&](int kt, int slot, int q) {  // q-th load: pair q / 2, operand q % 2
    unsigned char *st = lds + slot * STAGE;
    const int i = q >> 1;
    if (q & 1) lds_dma16(gB + (size_t)kt * BK, offB[i], st + SLICE + (wave + NW * i) * 1024);
    else lds_dma16(gA + (size_t)kt * BK, offA[i], st + (wave + NW * i) * 1024);
  };
  frag_t fa[2][4], fb[2][TN];
  const std::integral_constant<bool, true> kRd;
  const std::integral_constant<bool, false> kNoRd;
  // MFMAs of rows i0 .. i1-1 of one K-step; next to MFMA m the m-th fragment
  // read of K-step rs of stage rst (when `reads` is true) and, after every second
  // MFMA, the next of `nq` loads (from q0) of stage dk into slot dslot.
  auto kstep = [&](const frag_t (&f_a)[4], const frag_t (&f_b)[TN], int i0, int i1, auto reads,
                   const unsigned char *rst, int rs, frag_t (&n_a)[4], frag_t (&n_b)[TN],
                   int dk, int dslot, int q0, int nq) {
    constexpr bool RD = decltype(reads)::value;
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int m = (i - i0) * TN + j;
        acc[i][j] = MF::mma(f_a[i], f_b[j], acc[i][j]);
        if (RD && m < 4 + TN) {
          if (m < 4) n_a[m] = *reinterpret_cast<const frag_t *>(rst + frag_off(rA, m, rs));
          else n_b[m - 4] = *reinterpret_cast<const frag_t *>(rst + SLICE + frag_off(rB, m - 4, rs));
        }
        if ((m & 1) && (m >> 1) < nq) dma_q(dk, dslot, q0 + (m >> 1));
        __builtin_amdgcn_sched_barrier(0);
      }
  };
#pragma unroll
  for (int q = 0; q < NQ; ++q) dma_q(0, 0, q);
#pragma unroll
  for (int q = 0; q < Q1 + Q2; ++q) dma_q(1, 1, q);
  wait_vmcnt<Q1 + Q2>();  // stage 0 landed
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[0][i] = *reinterpret_cast<const frag_t *>(lds + frag_off(rA, i, 0));
#pragma unroll
  for (int j = 0; j < TN; ++j) fb[0][j] = *reinterpret_cast<const frag_t *>(lds + SLICE + frag_off(rB, j, 0));
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const unsigned char *st = lds + (kt & 1) * STAGE;
    const unsigned char *nst = lds + ((kt + 1) & 1) * STAGE;
    // past the end: stage nk-1 again, into the slot that is not read any
    // more, so the wait counts stay uniform
    const int kn = kt + 2 < nk ? kt + 2 : nk - 1;
    kstep(fa[0], fb[0], 0, 4, kRd, st, 1, fa[1], fb[1], kt + 1, (kt + 1) & 1, Q1 + Q2, Q3);
    prefetch(kt + 2 + kPrefetchAhead);
#pragma unroll
    for (int s = 1; s + 2 < S; ++s)
      kstep(fa[s & 1], fb[s & 1], 0, 4, kRd, st, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1], 0, 0, 0, 0);
    kstep(fa[(S - 2) & 1], fb[(S - 2) & 1], 0, 2, kRd, st, S - 1, fa[(S - 1) & 1], fb[(S - 1) & 1], 0, 0, 0, 0);
    wait_lgkmcnt0();  // this wave's reads of stage kt are in registers
    raw_barrier();    // A: ... and every other wave's: slot kt % 2 is free
    kstep(fa[(S - 2) & 1], fb[(S - 2) & 1], 2, 4, kNoRd, st, 0, fa[0], fb[0], kn, kt & 1, 0, Q1);
    // this wave's loads of stage kt+1 landed (the first loads of stage kn and
    // wave 0's last prefetch may be in flight)
    if (wave == 0) wait_vmcnt<Q1 + 1>();
    else wait_vmcnt<Q1>();
    raw_barrier();  // B: every wave's loads of stage kt+1 landed
    kstep(fa[(S - 1) & 1], fb[(S - 1) & 1], 0, 4, kRd, nst, 0, fa[0], fb[0], kn, kt & 1, Q1, Q2);
  }
  {  // last stage
    const unsigned char *st = lds + ((nk - 1) & 1) * STAGE;
#pragma unroll
    for (int s = 0; s + 1 < S; ++s)
      kstep(fa[s & 1], fb[s & 1], 0, 4, kRd, st, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1], 0, 0, 0, 0);
    kstep(fa[(S - 1) & 1], fb[(S - 1) & 1], 0, 4, kNoRd, st, 0, fa[0], fb[0], 0, 0, 0, 0);
  }

  // ---- fp32 epilogue (same contract as gemm_nt_kernel), staged in LDS ----
  wait_vmcnt<0>();  // the last (unused) refill has landed
  __syncthreads();  // all waves are done with the operand stages
  if (p.Cin != nullptr)
    staged_epilogue<T, SYM, true, NW, EPI_PITCH>(p, acc, reinterpret_cast<float *>(lds), g, tm, tn, wm, wn, lane, tid);
  else
    staged_epilogue<T, SYM, false, NW, EPI_PITCH>(p, acc, reinterpret_cast<float *>(lds), g, tm, tn, wm, wn, lane, tid);
}


// ---------------------------------------------------------------------------
// 256x256 batched NT GEMM for fp16 / bf16 on 16x16x32 MFMAs.  Same tile,
// operand staging, block order and epilogue as gemm256_kernel; each wave owns
// 128 x 128 as 8 x 8 blocks of 16 x 16 (f32x4 accumulators, 256 per lane).
// A 64-element stage is two 32-element MFMA K-steps, and each block's two
// MFMAs of a stage are issued back to back (the second accumulates onto the
// first's result).  At the shader clock this chip sustains under its power
// limit this order of 16x16x32 MFMAs delivers more fp16 throughput than
// 32x32x16 (measured on random operands: ~2.05 vs ~1.65 PFLOP/s).
//
// All fragments of a stage (8 A and 8 B blocks x 2 K-steps, 128 VGPRs) are
// in registers when its MFMAs start; the next stage's fragments replace them
// as they die: a stage runs columns 0-3 (H0) then columns 4-7 (H1), row by
// row, so B columns 0-3 are free during H1, A row i after H1 row i, and B
// columns 4-7 at the end.  LDS slot use per stage k (slot k % 2):
//   H0 row 0: barrier A (every wave read stage k) -> slot k % 2 takes stage
//             k + 2: 16 direct loads, one per 4 MFMAs over H0 rows 1-4 and
//             H1 rows 1-4;
//   H1 row 0: barrier B (stage k + 1 landed) -> its fragments are read
//             during the rest of H1.
// LDS chunk swizzle: chunk c of row r sits at c ^ ((r >> 1) & 7), so the 16
// rows of a fragment read (one 16-byte chunk per row) hit distinct banks and
// a lane's fragment offsets differ by immediates across its blocks.
// ---------------------------------------------------------------------------
template <int DT> struct Mfma16;
template <> struct Mfma16<NSG_F16> {
  using T = _Float16;
  using frag_t = f16x8;
  static __device__ __forceinline__ f32x4 mma(frag_t a, frag_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma16<NSG_BF16> {
  using T = __bf16;
  using frag_t = bf16x8;
  static __device__ __forceinline__ f32x4 mma(frag_t a, frag_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// Operands in their K-major layout (AT / BT): the operand is stored as
// K x 256-wide rows (the M or N index contiguous, pitch lda / ldb), and a
// stage is 64 K-rows of 512 bytes.  Direct-load instruction i of wave w
// fills K-rows 2 (w + 4 i) and 2 (w + 4 i) + 1; inside a row the 16 blocks
// of 16 columns (32 bytes) are permuted, physical block = logical block ^
// g(row), g(row) = (row & 3) | ((row >> 3) & 1) << 2.  A fragment (16
// columns, 8 consecutive K) is two ds_read_b64_tr_b16: lane j of each group
// of 16 points at K-row kb + j / 4, columns 4 (j % 4) .. + 3 of the block,
// and lane n receives the 4 consecutive K values kb .. kb + 3 of column n.
// The 8 K-rows a group of 32 lanes reads then fall on 8 distinct 32-byte
// block slots: one pass over the 64 banks, no conflict.
__device__ __forceinline__ int trg(int row) { return (row & 3) | (((row >> 3) & 1) << 2); }
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 *lds_s16x4_t;
template <typename F>
__device__ __forceinline__ F tr_frag(const unsigned char *p0, const unsigned char *p1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(p1));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  return __builtin_bit_cast(F, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// bf16 pair -> fp16 pair, each RNE(x 2^e): the value the scale pass stores
// for a bf16 input (bf16 -> fp32 is exact; ldexp and the conversion round once
// each, as there).
__device__ __forceinline__ unsigned bf16x2_to_f16x2(unsigned w, int e) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const float lo = __builtin_bit_cast(float, w << 16), hi = __builtin_bit_cast(float, w & 0xFFFF0000u);
  const h2 h = {(_Float16)ldexpf(lo, e), (_Float16)ldexpf(hi, e)};
  return __builtin_bit_cast(unsigned, h);
}

// SRC (OperandSource): kSrcPlain; kSrcCvtA / kSrcCvtB, an operand converted
// from the bf16 input in LDS (fp16 kernel, general products; a Cin term is
// then that input too, converted in the epilogue); kSrcRaw, the symmetric
// product of the raw bf16 input on bf16 MFMAs with fp16 outputs.
// Converted operand X: its 8 loads of a stage go to a raw area of LDS (one
// slice, after the two stage slots) instead of the stage slot.  In step k,
// the wave reads its own 1 KB block p of stage k + 1 from the raw area at H0
// row p (each lane its own 16 bytes: no other wave touches them), converts
// it into slot (k + 1) % 2 one row later (the read's latency hides behind
// the row's MFMAs) and loads block p of stage k + 2 into the raw area again;
// block 7 is written at H1 row 0, before barrier B.  The other operand's 8
// loads are at H1 rows 1-4.  With 16 loads per stage, 15 were issued after
// the one a read waits for, so every load has one step to land.
template <int DT, bool SYM, bool CIN, bool AT, bool BT, int SRC = kSrcPlain>
__global__ void __launch_bounds__(256, 1) gemm256h_kernel(const GemmArgs p) {
  using MF = Mfma16<DT>;
  using T = typename MF::T;
  using frag_t = typename MF::frag_t;
  constexpr bool CVA = SRC == kSrcCvtA, CVB = SRC == kSrcCvtB, CV = CVA || CVB;
  constexpr bool RAW = SRC == kSrcRaw;
  static_assert(!CV || (DT == NSG_F16 && !SYM), "converted operands: general fp16 products");
  static_assert(!RAW || (DT == NSG_BF16 && SYM && !CIN && AT == BT), "raw input: symmetric bf16 products");
  using TS = std::conditional_t<RAW, _Float16, T>;  // symmetric outputs
  constexpr int NW = 4;
  constexpr int BK = 64;             // K elements per stage (128-byte row slices)
  constexpr int SLICE = 256 * 128;   // bytes of one operand slice
  constexpr int STAGE = 2 * SLICE;   // A slice then B slice
  constexpr int NLD = 8;             // 1 KB direct loads per operand per wave per stage
  // converted operand: raw blocks of the next stage.  The epilogue's staging
  // area reaches into it; no raw load is in flight by then (the last raw
  // blocks are converted in the step before the last stage).
  constexpr int RAW_OFF = 2 * STAGE;
  constexpr int MAIN_BYTES = CV ? 2 * STAGE + SLICE : 2 * STAGE;
  // the epilogue stages 256 columns of 128 rows per pass (symmetric
  // products) or 128 columns of 256 rows (general ones), 4 floats of padding
  // per column
  constexpr int EPI_COLS = SYM ? 256 : 128;
  constexpr int EPI_PITCH = SYM ? 132 : 260;
  constexpr int EPI_BYTES = EPI_COLS * EPI_PITCH * 4;
  constexpr int LDS_BYTES = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[LDS_BYTES];
  static_assert(EPI_PITCH >= 256 * 128 / EPI_COLS + 4 && EPI_BYTES <= LDS_BYTES, "staging fits the LDS array");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // persistent: workgroup b takes tiles b, b + gridDim.x, ... (the launch has
  // one workgroup per CU, so tile L runs on the XCD that block L would have)
  const int tiles_m = p.M >> 8, tiles_n = p.N >> 8;
  const unsigned total = (unsigned)(SYM ? tiles_m * (tiles_m + 1) / 2 : tiles_m * tiles_n) * (unsigned)p.batch;
  for (unsigned L = blockIdx.x; L < total; L += gridDim.x) {
  int g, tm, tn;
  tile_256<SYM>(p, L, total, g, tm, tn);

  // exponent e[g] of the matrix (converted or raw operands)
  const int ex = (CV || RAW) ? reinterpret_cast<const int32_t *>(p.gscale + p.batch)[g] : 0;
  // operand bases and pitches: a raw product reads the input, or the scaled
  // copy of a matrix outside raw_exponent_ok
  const bool from_fb = RAW && !raw_exponent_ok(ex);
  const void *baseA = from_fb ? p.fb : p.A, *baseB = from_fb ? p.fb : p.B;
  const int64_t lda = from_fb ? p.ldfb : p.lda, ldb = from_fb ? p.ldfb : p.ldb;
  const int64_t sA = from_fb ? p.sfb : p.sA, sB = from_fb ? p.sfb : p.sB;
  // direct-load sources: wave w fills the 1 KB blocks b = w + 4 i of each
  // slice (rows 8 b .. 8 b + 7; lane l writes chunk slot l % 8 of row
  // 8 b + l / 8, which holds logical chunk (l % 8) ^ ((row >> 1) & 7))
  const T *gA = reinterpret_cast<const T *>(baseA) + (size_t)g * sA + (AT ? (size_t)tm * 256 : (size_t)tm * 256 * lda);
  const T *gB = reinterpret_cast<const T *>(baseB) + (size_t)g * sB + (BT ? (size_t)tn * 256 : (size_t)tn * 256 * ldb);
  // Per-lane offsets are rederived for every tile from a copy of the lane
  // index the compiler cannot see through, so they are never kept (and
  // spilled) across the epilogue.
  int ln = lane;
  asm volatile("" : "+v"(ln));
  auto dma_off = [&](bool trans, int i, int64_t ld) -> unsigned {
    if (trans) {  // K-row 2 (w + 4 i) + ln / 32, physical 16-byte chunk ln % 32
      const int row = 2 * (wave + NW * i) + (ln >> 5), pc = ln & 31;
      return (unsigned)((row * (int)ld + (((pc >> 1) ^ trg(row)) << 4) + ((pc & 1) << 3)) * 2);
    }
    const int row = (wave + NW * i) * 8 + (ln >> 3);
    return (unsigned)((row * (int)ld + (((ln & 7) ^ ((row >> 1) & 7)) << 3)) * 2);
  };
  unsigned offA[NLD], offB[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    offA[i] = dma_off(AT, i, lda);
    offB[i] = dma_off(BT, i, ldb);
  }
  const int nk = p.K / BK;  // >= 4: K is a multiple of 256
  // stage kt of each operand: 64 K elements of every row, or 64 K-rows
  const size_t stepA = AT ? (size_t)BK * lda : (size_t)BK, stepB = BT ? (size_t)BK * ldb : (size_t)BK;
  auto dma = [&](int kt, int slot, int q) {  // q-th of the 16 loads of a stage: pair q / 2, operand q % 2
    unsigned char *st = lds + slot * STAGE;
    const int i = q >> 1;
    if (q & 1) lds_dma16(gB + (size_t)kt * stepB, offB[i], st + SLICE + (wave + NW * i) * 1024);
    else lds_dma16(gA + (size_t)kt * stepA, offA[i], st + (wave + NW * i) * 1024);
  };
  // converted operand X (CV) and the other one, Y: block i of stage kt
  auto x_load = [&](int kt, int i) {  // raw, into the raw area
    if constexpr (CVA) lds_dma16(gA + (size_t)kt * stepA, offA[i], lds + RAW_OFF + (wave + NW * i) * 1024);
    else lds_dma16(gB + (size_t)kt * stepB, offB[i], lds + RAW_OFF + (wave + NW * i) * 1024);
  };
  auto y_load = [&](int kt, int slot, int i) {
    unsigned char *st = lds + slot * STAGE;
    if constexpr (CVA) lds_dma16(gB + (size_t)kt * stepB, offB[i], st + SLICE + (wave + NW * i) * 1024);
    else lds_dma16(gA + (size_t)kt * stepA, offA[i], st + (wave + NW * i) * 1024);
  };
  // this lane's 16 raw bytes of block i, and their conversion into X's
  // slice of a slot
  auto x_read = [&](int i) { return *reinterpret_cast<const uint4 *>(lds + RAW_OFF + (wave + NW * i) * 1024 + 16 * lane); };
  auto x_write = [&](const uint4 &w, int slot, int i) {
    uint4 r;
    r.x = bf16x2_to_f16x2(w.x, ex);
    r.y = bf16x2_to_f16x2(w.y, ex);
    r.z = bf16x2_to_f16x2(w.z, ex);
    r.w = bf16x2_to_f16x2(w.w, ex);
    *reinterpret_cast<uint4 *>(lds + slot * STAGE + (CVA ? 0 : SLICE) + (wave + NW * i) * 1024 + 16 * lane) = r;
  };

  // fragment reads: lane l reads row (block row + l % 16), K elements
  // 32 s + 8 (l / 16) .. + 7 of the stage; block i adds i * 2048 bytes
  const int r16 = ln & 15, q4 = ln >> 4;
  const int rA = wm * 128 + r16, rB = wn * 128 + r16;
  const int zA = (rA >> 1) & 7, zB = (rB >> 1) & 7;
  const int fA0 = rA * 128 + ((q4 ^ zA) << 4), fA1 = rA * 128 + (((4 + q4) ^ zA) << 4);
  const int fB0 = SLICE + rB * 128 + ((q4 ^ zB) << 4), fB1 = SLICE + rB * 128 + (((4 + q4) ^ zB) << 4);
  // K-major operands: lane (q4, r16) reads K-row kr = 8 q4 + r16 / 4 (+ 4 for
  // the second read, + 32 for the second K half), columns 4 (r16 % 4) of
  // block i: byte (kr * 512 + 256 wq + 8 (r16 % 4)) ^ ((i ^ g(kr)) << 5)
  const int kr = 8 * q4 + (r16 >> 2);
  const int tA = kr * 512 + wm * 256 + (r16 & 3) * 8 + (trg(kr) << 5);
  const int tB = SLICE + kr * 512 + wn * 256 + (r16 & 3) * 8 + (trg(kr) << 5);

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  frag_t a[8][2], b[8][2];
  auto rd_a = [&](const unsigned char *st, int i) {
    if constexpr (AT) {
      const unsigned char *q = st + (tA ^ (i << 5));
      a[i][0] = tr_frag<frag_t>(q, q + 2048);
      a[i][1] = tr_frag<frag_t>(q + 16384, q + 18432);
    } else {
      a[i][0] = *reinterpret_cast<const frag_t *>(st + fA0 + i * 2048);
      a[i][1] = *reinterpret_cast<const frag_t *>(st + fA1 + i * 2048);
    }
  };
  auto rd_b = [&](const unsigned char *st, int j) {
    if constexpr (BT) {
      const unsigned char *q = st + (tB ^ (j << 5));
      b[j][0] = tr_frag<frag_t>(q, q + 2048);
      b[j][1] = tr_frag<frag_t>(q + 16384, q + 18432);
    } else {
      b[j][0] = *reinterpret_cast<const frag_t *>(st + fB0 + j * 2048);
      b[j][1] = *reinterpret_cast<const frag_t *>(st + fB1 + j * 2048);
    }
  };
  auto pair = [&](int i, int j) {
    acc[i][j] = MF::mma(a[i][0], b[j][0], acc[i][j]);
    acc[i][j] = MF::mma(a[i][1], b[j][1], acc[i][j]);
  };

  if constexpr (CV) {
    // stage 0: X raw, Y; convert X (and load stage 1's raw X block by
    // block); then Y of stage 1: the order of loads in a step
#pragma unroll
    for (int i = 0; i < NLD; ++i) x_load(0, i);
#pragma unroll
    for (int i = 0; i < NLD; ++i) y_load(0, 0, i);
    wait_vmcnt<NLD>();  // X of stage 0 landed
    __builtin_amdgcn_sched_barrier(0);
    uint4 xr[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) xr[i] = x_read(i);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      x_write(xr[i], 0, i);
      x_load(1, i);  // after its raw block was read
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) y_load(1, 1, i);
    wait_vmcnt<2 * NLD>();  // Y of stage 0 landed
    wait_lgkmcnt0();        // the converted X of stage 0 is written
  } else {
#pragma unroll
    for (int q = 0; q < 2 * NLD; ++q) dma(0, 0, q);
#pragma unroll
    for (int q = 0; q < 2 * NLD; ++q) dma(1, 1, q);
    wait_vmcnt<2 * NLD>();  // stage 0 landed
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) rd_a(lds, i);
#pragma unroll
  for (int j = 0; j < 8; ++j) rd_b(lds, j);

  // one 64-element stage: compute stage kt from registers, read stage kt+1's
  // fragments, and (REFILL) load stage kt+2 into the slot stage kt leaves
  auto step = [&](int kt, auto refill) {
    constexpr bool REFILL = decltype(refill)::value;
    const unsigned char *nst = lds + ((kt + 1) & 1) * STAGE;
    const int kn = kt + 2;
    const int dslot = kt & 1;
    // CV, at H0 row xi (xi = 0..7) and H1 row 0 (xi = 8): the raw block
    // xi - 1 of X of stage kt+1, read one row earlier, into slot
    // (kt+1) % 2 and (REFILL) stage kt+2's raw block xi - 1 loaded; then
    // block xi of stage kt+1 (15 loads were issued after it, stage kt+2's
    // blocks 0 .. xi-1 among them with REFILL) read for the next row
    uint4 xt;
    auto x_step = [&](auto xi_c) {
      constexpr int xi = decltype(xi_c)::value;
      if constexpr (xi >= 1) {
        x_write(xt, (kt + 1) & 1, xi - 1);
        if (REFILL) x_load(kn, xi - 1);
      }
      if constexpr (xi < NLD) {
        wait_vmcnt<REFILL ? 2 * NLD - 1 : 2 * NLD - 1 - xi>();
        __builtin_amdgcn_sched_barrier(0);
        xt = x_read(xi);
      }
    };
    // ---- H0: columns 0-3 ----
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pair(i, j);
        if constexpr (CV) {
          if (j == 1) {
            if (i == 0) x_step(std::integral_constant<int, 0>{});
            if (i == 1) x_step(std::integral_constant<int, 1>{});
            if (i == 2) x_step(std::integral_constant<int, 2>{});
            if (i == 3) x_step(std::integral_constant<int, 3>{});
            if (i == 4) x_step(std::integral_constant<int, 4>{});
            if (i == 5) x_step(std::integral_constant<int, 5>{});
            if (i == 6) x_step(std::integral_constant<int, 6>{});
            if (i == 7) x_step(std::integral_constant<int, 7>{});
          }
        } else {
          if (REFILL && i >= 1 && i <= 4 && (j & 1)) dma(kn, dslot, 2 * (i - 1) + (j >> 1));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (REFILL && i == 0) {
        wait_lgkmcnt0();  // this wave's reads of stage kt are in registers
        raw_barrier();    // A: ... and every other wave's: slot kt % 2 is free
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- H1: columns 4-7; the fragments of stage kt+1 replace those that
    //      died (B columns 0-3 during row 1, A row i after row i) ----
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 4; j < 8; ++j) {
        pair(i, j);
        if constexpr (CV) {
          if (i == 0 && j == 5) x_step(std::integral_constant<int, 8>{});
          if (REFILL && i >= 1 && i <= 4 && (j & 1)) y_load(kn, dslot, 2 * (i - 1) + ((j - 4) >> 1));
        } else {
          if (REFILL && i >= 1 && i <= 4 && (j & 1)) dma(kn, dslot, 8 + 2 * (i - 1) + ((j - 4) >> 1));
        }
        if (i == 1) rd_b(nst, j - 4);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i == 0) {
        // this wave's loads of stage kt+1 landed (with REFILL, the 8 loads
        // of stage kt+2 issued in the first half may be in flight)
        if (REFILL) wait_vmcnt<8>();
        else wait_vmcnt<0>();
        if constexpr (CV) wait_lgkmcnt0();  // the converted blocks of stage kt+1 are written
        raw_barrier();  // B: every wave's loads of stage kt+1 landed
        __builtin_amdgcn_sched_barrier(0);
      }
      rd_a(nst, i);
    }
#pragma unroll
    for (int j = 4; j < 8; ++j) rd_b(nst, j);
  };
  for (int kt = 0; kt + 2 < nk; ++kt) step(kt, std::true_type{});
  step(nk - 2, std::false_type{});  // no stage nk to load
  // last stage
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pair(i, j);
      __builtin_amdgcn_sched_barrier(0);
    }

  __syncthreads();  // all waves are done with the operand stages
  // general products stage column halves (all four waves at once), symmetric
  // ones row halves (measured: -0.5 to -3% per general launch, while column
  // passes slowed the symmetric ones)
  // with a converted operand, a Cin term is the same input (X = a X + B X)
  staged_epilogue<T, SYM, CIN, NW, EPI_PITCH, !SYM, TS, CV && CIN>(p, acc, reinterpret_cast<float *>(lds), g, tm,
                                                                    tn, wm, wn, lane, tid);
  __syncthreads();  // the staging area is read before the next tile's loads overwrite it
  }
}

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

constexpr int kWaves256 = 4;

// Compute units of the current device (cached per device; 0 on error).
static unsigned cu_count() {
  static unsigned cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev]) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
  if (dev < 64) cached[dev] = (unsigned)n;
  return (unsigned)n;
}

template <int DT, bool SYM>
static hipError_t launch_256(const GemmArgs &a, hipStream_t s) {
  const unsigned tm = (unsigned)(a.M / 256), tn = (unsigned)(a.N / 256);
  const unsigned tiles = SYM ? tm * (tm + 1) / 2 : tm * tn;
  const unsigned long long blocks = (unsigned long long)tiles * (unsigned)a.batch;
  if (blocks == 0 || blocks > 0xFFFFFFFFull) return hipErrorInvalidValue;
  if constexpr (DT == NSG_F32) {
    hipLaunchKernelGGL((gemm256_kernel<DT, SYM, kWaves256>), dim3((unsigned)blocks), dim3(kWaves256 * 64), 0, s, a);
  } else {
    const unsigned ncu = cu_count();
    if (ncu == 0) return hipErrorInvalidDevice;
    const unsigned grid = blocks < ncu ? (unsigned)blocks : ncu;
    // operand layouts: both row-major (NT), both K-major (the Gram product
    // of a K-major X), or a K-major B (general products Q X of a row-major X)
    if (a.a_trans != a.b_trans && (SYM || a.a_trans)) return hipErrorInvalidValue;
    const int mode = a.a_trans ? 2 : (a.b_trans ? 1 : 0);
#define NSG_H(C, AT_, BT_) hipLaunchKernelGGL((gemm256h_kernel<DT, SYM, C, AT_, BT_>), dim3(grid), dim3(256), 0, s, a)
#define NSG_HS(C, AT_, BT_, S_) \
  hipLaunchKernelGGL((gemm256h_kernel<DT, SYM, C, AT_, BT_, S_>), dim3(grid), dim3(256), 0, s, a)
    if (a.src != kSrcPlain) {
      // an operand from the caller's bf16 input: converted (general fp16
      // products, X0 as A of a row-major pair or as the K-major B, and as
      // the Cin of X = a X + B X) or raw (symmetric bf16 products)
      if (a.gscale == nullptr) return hipErrorInvalidValue;
      if constexpr (DT == NSG_F16 && !SYM) {
        const void *x0 = a.src == kSrcCvtA ? a.A : a.B;
        if (a.Cin != nullptr && a.Cin != x0) return hipErrorInvalidValue;
        const bool c = a.Cin != nullptr;
        if (a.src == kSrcCvtA && mode == 0) {
          if (c) NSG_HS(true, false, false, kSrcCvtA);
          else NSG_HS(false, false, false, kSrcCvtA);
        } else if (a.src == kSrcCvtB && mode == 1) {
          if (c) NSG_HS(true, false, true, kSrcCvtB);
          else NSG_HS(false, false, true, kSrcCvtB);
        } else {
          return hipErrorInvalidValue;
        }
      } else if constexpr (DT == NSG_BF16 && SYM) {
        if (a.src != kSrcRaw || a.Cin != nullptr || a.fb == nullptr || a.A != a.B || a.lda != a.ldb)
          return hipErrorInvalidValue;
        if (mode == 0) NSG_HS(false, false, false, kSrcRaw);
        else NSG_HS(false, true, true, kSrcRaw);
      } else {
        return hipErrorInvalidValue;
      }
    } else if (a.Cin != nullptr) {
      if (mode == 0) NSG_H(true, false, false);
      else if (mode == 1) NSG_H(true, false, true);
      else NSG_H(true, true, true);
    } else {
      if (mode == 0) NSG_H(false, false, false);
      else if (mode == 1) NSG_H(false, false, true);
      else NSG_H(false, true, true);
    }
#undef NSG_H
#undef NSG_HS
  }
  return hipGetLastError();
}

template <int DT, bool SYM>
static hipError_t launch_cfg(int cfg, const GemmArgs &a, hipStream_t s) {
  // K-major operands exist only on the 16-bit 256 x 256 kernel
  if ((a.a_trans || a.b_trans) && (cfg != kTile256 || DT == NSG_F32)) return hipErrorInvalidValue;
  if (cfg == kTile256) return launch_256<DT, SYM>(a, s);
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

// Each thread owns elements start + 256 V k + V t + v (v < V, V = 16 bytes of
// input); it sums their squares in that order whether it reads them with one
// 16-byte load (aligned input) or V scalar loads, so the result never depends
// on the input's alignment.
template <typename TI, bool VEC>
__global__ void __launch_bounds__(256) norm_reduce_kernel(const NormReduceArgs p) {
  constexpr int V = 16 / (int)sizeof(TI);
  typedef TI vec_t __attribute__((ext_vector_type(V)));
  __shared__ float red[4];
  const int g = blockIdx.y;
  const int64_t start = (int64_t)blockIdx.x * kNormChunk;
  int64_t end = start + kNormChunk;
  if (end > p.elems) end = p.elems;
  const TI *in = reinterpret_cast<const TI *>(p.in) + (size_t)g * p.elems;
  float s = 0.f;
  for (int64_t i = start + (int64_t)threadIdx.x * V; i < end; i += 256 * V) {
    if (VEC && i + V <= end) {
      const vec_t x = *reinterpret_cast<const vec_t *>(in + i);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const float f = to_f32(x[v]);
        s = fmaf(f, f, s);
      }
    } else {
      for (int v = 0; v < V && i + v < end; ++v) {
        const float f = to_f32(in[i + v]);
        s = fmaf(f, f, s);
      }
    }
  }
  s = block_sum_256(s, red);
  if (threadIdx.x == 0) p.partials[(size_t)g * p.nchunks + blockIdx.x] = s;
}

hipError_t launch_norm_reduce(const NormReduceArgs &a, hipStream_t s) {
  if (a.batch == 0 || a.elems == 0) return hipSuccess;
  dim3 grid((unsigned)a.nchunks, (unsigned)a.batch), block(256);
  const size_t es = a.in_dtype == NSG_F32 ? 4 : 2;
  const bool vec = (reinterpret_cast<uintptr_t>(a.in) % 16 == 0) && ((size_t)a.elems * es) % 16 == 0;
#define NSG_RED(TI) \
  if (vec) hipLaunchKernelGGL((norm_reduce_kernel<TI, true>), grid, block, 0, s, a); \
  else hipLaunchKernelGGL((norm_reduce_kernel<TI, false>), grid, block, 0, s, a)
  switch (a.in_dtype) {
    case NSG_F16: NSG_RED(_Float16); break;
    case NSG_BF16: NSG_RED(__bf16); break;
    default: NSG_RED(float); break;
  }
#undef NSG_RED
  return hipGetLastError();
}

// Per matrix: nu = sqrt(sum of the partial sums, fixed tree), kappa =
// 1 / (s (nu + eps)), kappa 2^f = r 2^e with r in [0.5, 1): gscale[g] = r,
// gscale[G + g] = e (int32), status[g] = 0.
__global__ void __launch_bounds__(256) scale_finalize_kernel(const ScaleArgs p) {
  __shared__ float red[4];
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  float s = 0.f;
  for (int i = tid; i < p.nchunks; i += 256) s += p.partials[(size_t)g * p.nchunks + i];
  s = block_sum_256(s, red);
  if (tid == 0) {
    const float nu = sqrtf(s);
    const float kappa = 1.f / (p.safety * (nu + p.eps));
    int e = 0;
    const float r = frexpf(ldexpf(kappa, p.fexp), &e);
    p.gscale[g] = r;
    reinterpret_cast<int32_t *>(p.gscale + p.batch)[g] = e;
    if (p.status != nullptr) p.status[g] = 0;
  }
}

// Scale by the exact power of two 2^e, cast, and write both layouts through a
// 64x64 LDS tile.  Each thread moves 16 consecutive elements of a row: one or
// two 16-byte loads when the input rows allow it (VEC), else scalar loads; the
// same values either way.  Outputs (workspace, 128-byte-aligned pitches) use
// 16-byte stores.
template <typename TI, typename TO, bool VEC>
__global__ void __launch_bounds__(256) scale_cast_transpose_kernel(const ScaleArgs p) {
  __shared__ float tile[64][65];
  constexpr int VI = 16 / (int)sizeof(TI);
  constexpr int VO = 16 / (int)sizeof(TO);
  typedef TI vin_t __attribute__((ext_vector_type(VI)));
  typedef TO vout_t __attribute__((ext_vector_type(VO)));
  const int g = blockIdx.z;
  const int tid = threadIdx.x;
  const int e = reinterpret_cast<const int32_t *>(p.gscale + p.batch)[g];
  const int a0 = blockIdx.y * 64, b0 = blockIdx.x * 64;
  const TI *in = reinterpret_cast<const TI *>(p.in) + (size_t)g * (size_t)(p.R * p.C);
  // load: thread -> row tid / 4, columns 16 (tid % 4) .. + 15
  {
    const int a = tid >> 2, bb = (tid & 3) * 16;
    const int row = a0 + a, col = b0 + bb;
    float v[16];
    if (VEC && row < p.R && col + 16 <= p.C) {
      const TI *src = in + (size_t)row * p.C + col;
#pragma unroll
      for (int u = 0; u < 16 / VI; ++u) {
        const vin_t x = *reinterpret_cast<const vin_t *>(src + u * VI);
#pragma unroll
        for (int q = 0; q < VI; ++q) v[u * VI + q] = to_f32(x[q]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q)
        v[q] = (row < p.R && col + q < p.C) ? to_f32(in[(size_t)row * p.C + col + q]) : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) tile[a][bb + q] = ldexpf(v[q], e);
  }
  __syncthreads();
  TO *same = reinterpret_cast<TO *>(p.same) + (size_t)g * p.s_same;
  TO *swp = reinterpret_cast<TO *>(p.swap) + (size_t)g * p.s_swap;
  {
    const int a = tid >> 2, bb = (tid & 3) * 16;
    // same layout: row a, columns bb .. bb + 15
    TO *dst = same + (size_t)(a0 + a) * p.ld_same + (b0 + bb);
#pragma unroll
    for (int u = 0; u < 16 / VO; ++u) {
      vout_t w;
#pragma unroll
      for (int q = 0; q < VO; ++q) w[q] = cvt<TO>(tile[a][bb + u * VO + q]);
      *reinterpret_cast<vout_t *>(dst + u * VO) = w;
    }
    // transposed: output row (b0 + a) = input column a, input rows bb .. bb + 15
    TO *dst2 = swp + (size_t)(b0 + a) * p.ld_swap + (a0 + bb);
#pragma unroll
    for (int u = 0; u < 16 / VO; ++u) {
      vout_t w;
#pragma unroll
      for (int q = 0; q < VO; ++q) w[q] = cvt<TO>(tile[bb + u * VO + q][a]);
      *reinterpret_cast<vout_t *>(dst2 + u * VO) = w;
    }
  }
}

// The same scale, cast and transpose for 16-bit outputs, on 64 x 128 input
// tiles: each thread loads 8 consecutive inputs of 4 rows (16 lanes cover a
// 128-element row segment), writes them in the input layout straight from
// registers, and parks the converted values in LDS (row pitch 65 words:
// conflict-free 4-byte writes and column reads).  The transposed copy is then
// written as 128-byte rows: a thread takes two adjacent input columns (one
// 4-byte LDS word per row) and 8 input rows.  Every output element is
// cvt(ldexp(x, e)), as in the kernel above.
template <typename TI, typename TO, bool VEC, bool SWAP>
__global__ void __launch_bounds__(256) scale_cast_transpose16_kernel(const ScaleArgs p) {
  static_assert(sizeof(TO) == 2, "16-bit outputs");
  constexpr int PW = 65;  // LDS row pitch in 32-bit words (two outputs each)
  __shared__ uint32_t tile[64 * PW];
  constexpr int VI = 16 / (int)sizeof(TI);
  typedef TI vin_t __attribute__((ext_vector_type(VI)));
  typedef TO vout_t __attribute__((ext_vector_type(8)));
  typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
  const int g = blockIdx.z;
  const int tid = threadIdx.x;
  const int e = reinterpret_cast<const int32_t *>(p.gscale + p.batch)[g];
  if (p.raw_fallback && raw_exponent_ok(e)) return;  // the product reads this matrix raw
  const int a0 = blockIdx.y * 64, b0 = blockIdx.x * 128;
  const TI *in = reinterpret_cast<const TI *>(p.in) + (size_t)g * (size_t)(p.R * p.C);
  TO *same = reinterpret_cast<TO *>(p.same) + (size_t)g * p.s_same;
  TO *swp = reinterpret_cast<TO *>(p.swap) + (size_t)g * p.s_swap;
  const int cl = (tid & 15) * 8;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int a = (tid >> 4) + 16 * k, row = a0 + a, col = b0 + cl;
    float v[8];
    if (VEC && row < p.R && col + 8 <= p.C) {
      const TI *src = in + (size_t)row * p.C + col;
#pragma unroll
      for (int u = 0; u < 8 / VI; ++u) {
        const vin_t x = *reinterpret_cast<const vin_t *>(src + u * VI);
#pragma unroll
        for (int q = 0; q < VI; ++q) v[u * VI + q] = to_f32(x[q]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        v[q] = (row < p.R && col + q < p.C) ? to_f32(in[(size_t)row * p.C + col + q]) : 0.f;
    }
    vout_t w;
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = cvt<TO>(ldexpf(v[q], e));
    *reinterpret_cast<vout_t *>(same + (size_t)row * p.ld_same + col) = w;
    if constexpr (!SWAP) continue;
    const u16x8 bits = __builtin_bit_cast(u16x8, w);
    uint32_t *t = tile + a * PW + (cl >> 1);
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = (uint32_t)bits[2 * u] | ((uint32_t)bits[2 * u + 1] << 16);
  }
  if constexpr (!SWAP) return;  // one layout only
  __syncthreads();
  const int ac = 8 * (tid & 7);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int bp = 2 * (tid >> 3) + 64 * h;  // input columns bp, bp + 1 of the tile
    u16x8 lo, hi;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t x = tile[(ac + q) * PW + (bp >> 1)];
      lo[q] = (unsigned short)(x & 0xFFFFu);
      hi[q] = (unsigned short)(x >> 16);
    }
    *reinterpret_cast<vout_t *>(swp + (size_t)(b0 + bp) * p.ld_swap + (a0 + ac)) = __builtin_bit_cast(vout_t, lo);
    *reinterpret_cast<vout_t *>(swp + (size_t)(b0 + bp + 1) * p.ld_swap + (a0 + ac)) = __builtin_bit_cast(vout_t, hi);
  }
}

template <typename TI, bool VEC>
static void launch_scale_in(const ScaleArgs &a, dim3 grid, hipStream_t s) {
  // 16-bit outputs: 64 x 128 tiles (the padded column count is a multiple of 256)
  const dim3 grid16(grid.x / 2, grid.y, grid.z);
  const bool swap = a.swap != nullptr;
  switch (a.cdtype) {
    case NSG_F16:
      if (swap) hipLaunchKernelGGL((scale_cast_transpose16_kernel<TI, _Float16, VEC, true>), grid16, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((scale_cast_transpose16_kernel<TI, _Float16, VEC, false>), grid16, dim3(256), 0, s, a);
      break;
    case NSG_BF16:
      if (swap) hipLaunchKernelGGL((scale_cast_transpose16_kernel<TI, __bf16, VEC, true>), grid16, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((scale_cast_transpose16_kernel<TI, __bf16, VEC, false>), grid16, dim3(256), 0, s, a);
      break;
    default: hipLaunchKernelGGL((scale_cast_transpose_kernel<TI, float, VEC>), grid, dim3(256), 0, s, a); break;
  }
}

hipError_t launch_scale(const ScaleArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(scale_finalize_kernel, dim3((unsigned)a.batch), dim3(256), 0, s, a);
  if (a.same == nullptr) return hipGetLastError();  // the products read the input in place
  dim3 grid((unsigned)(a.cols_p / 64), (unsigned)(a.rows_p / 64), (unsigned)a.batch);
  const size_t es = a.in_dtype == NSG_F32 ? 4 : 2;
  const bool vec = (reinterpret_cast<uintptr_t>(a.in) % 16 == 0) && ((size_t)a.C * es) % 16 == 0;
  switch (a.in_dtype) {
    case NSG_F16: vec ? launch_scale_in<_Float16, true>(a, grid, s) : launch_scale_in<_Float16, false>(a, grid, s); break;
    case NSG_BF16: vec ? launch_scale_in<__bf16, true>(a, grid, s) : launch_scale_in<__bf16, false>(a, grid, s); break;
    default: vec ? launch_scale_in<float, true>(a, grid, s) : launch_scale_in<float, false>(a, grid, s); break;
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
