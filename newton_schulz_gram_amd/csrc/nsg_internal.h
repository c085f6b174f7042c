// Internal interface between the host runtime (nsg_api.cpp) and the gfx950
// kernels (nsg_kernels.hip).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "nsg.h"

namespace nsg {

// Every matrix the library keeps in its workspace has both dimensions padded
// to a multiple of kPad, with zeros in the padding, so that GEMM tiles and
// K-steps never need bounds checks on their loads.
constexpr int kPad = 256;
// Elements of the input summed by one block of the norm reduction.  Fixed, so
// the reduction order of a matrix never depends on the bucket size.
constexpr int64_t kNormChunk = 16384;

// kInUser: the caller's input read in place (16-bit input, both sides
// multiples of kPad; in the compute dtype, or bf16 under fp16 compute with the
// operand sources below)
enum BufferKind : int { kInUser = -3, kOutUser = -2, kNone = -1 };

// Operand sources of the 16-bit 256 x 256 GEMM kernel.
//   kSrcPlain: A and B in the kernel's dtype.
//   kSrcCvtA / kSrcCvtB (fp16 kernel, general products): A (or B) is the
//     caller's bf16 input; its K-slices are loaded raw into LDS and each wave
//     converts the blocks it loaded to X_stored = RNE_fp16(x 2^e[b]), the
//     value the scale pass would have stored, before the MFMAs read them.  A
//     Cin, if given, is that input too and is converted in the epilogue.
//   kSrcRaw (bf16 kernel, symmetric products, fp16 outputs): A = B = the
//     caller's bf16 input G, whose products are exact in fp32, with alpha'
//     times 2^(gpow e[b]), for every matrix whose exponent passes
//     raw_exponent_ok(e[b]); any other matrix reads the bf16 copy G 2^e[b]
//     at `fb` (ld `ldfb`, `sfb` elements per matrix) without that factor.
enum OperandSource : int { kSrcPlain = 0, kSrcCvtA = 1, kSrcCvtB = 2, kSrcRaw = 3 };

// Exponents e (X_stored = G 2^e) for which the symmetric product of the raw
// bf16 input is safe: |G|_F ~ 2^(f - e) with f <= 8 then lies in
// [2^-24, 2^49], so sums of products stay finite in fp32, every product of
// entries above 2^-40 |G|_F stays a normal fp32 number, and 2^(2e) is one.
__host__ __device__ constexpr bool raw_exponent_ok(int e) { return e >= -40 && e <= 24; }

// One batched GEMM launch: V = alpha' A B^T + beta' Cin, with
// alpha' = alpha * gscale[b]^gpow and beta' = beta * gscale[b]^gpow, both
// times 2^(gpow e[b]) when gexp is set (e[b]: the int32 exponent stored after
// the G scales; the operands are then the unscaled input G, and G 2^e is the
// stored X0).
// A is M x K (lda), B is N x K (ldb), Cin is M x N (ldc), all in the compute
// dtype, batches `s*` elements apart.  M, N, K are padded sizes (multiples of
// the tile); Mv x Nv is the valid corner.  a_trans / b_trans: the operand is
// stored K-major instead, as K x M (lda >= M) or K x N (ldb >= N) (16-bit
// 256 x 256 kernel only: both for symmetric products, b_trans alone for
// general ones).
struct GemmArgs {
  const void *A = nullptr;
  int64_t lda = 0, sA = 0;
  const void *B = nullptr;
  int64_t ldb = 0, sB = 0;
  int32_t a_trans = 0, b_trans = 0;
  const void *Cin = nullptr;
  int64_t ldc = 0, sC = 0;
  // out0: V (row-major, mirrored for symmetric launches).  Its dtype may be
  // the caller's output dtype.  out0_pad = 1 writes zeros outside the valid
  // corner (workspace outputs); 0 writes nothing there (the caller's buffer).
  void *out0 = nullptr;
  int64_t ld0 = 0, s0 = 0;
  int32_t out0_dtype = NSG_F16;
  int32_t out0_pad = 1;
  // out1: V^T (general launches only), compute dtype, zero padding.
  void *out1 = nullptr;
  int64_t ld1 = 0, s1 = 0;
  // out2: V + diag * I (symmetric launches only, mirrored), compute dtype.
  void *out2 = nullptr;
  int64_t ld2 = 0, s2 = 0;
  float diag = 0.f;
  int32_t M = 0, N = 0, K = 0;
  int32_t Mv = 0, Nv = 0;
  float alpha = 1.f, beta = 0.f;
  const float *gscale = nullptr;
  int32_t gpow = 0;
  int32_t gexp = 0;
  int32_t src = kSrcPlain;  // OperandSource
  const void *fb = nullptr;  // kSrcRaw: bf16 G 2^e of the matrices that fail raw_exponent_ok
  int64_t ldfb = 0, sfb = 0;
  int32_t *status = nullptr;  // set to 1 for a batch with a non-finite out0 value
  int32_t batch = 0;
};

struct NormReduceArgs {
  const void *in = nullptr;
  int32_t in_dtype = NSG_F16;
  int64_t elems = 0;  // R * C
  int32_t nchunks = 0;
  float *partials = nullptr;  // [G][nchunks]
  int32_t batch = 0;
};

// X_stored = RNE(G * 2^e) where kappa 2^f = r 2^e, kappa = 1/(s(nu+eps)),
// r in [0.5, 1); so X0 = r 2^-f X_stored, and gscale[b] = r.
struct ScaleArgs {
  const void *in = nullptr;
  int32_t in_dtype = NSG_F16;
  int64_t R = 0, C = 0;
  const float *partials = nullptr;
  int32_t nchunks = 0;
  float safety = 1.f, eps = 1e-7f;
  int32_t fexp = 0;
  int32_t tr = 0;  // 1: input is m x n (R > C)
  int32_t rows_p = 0, cols_p = 0;  // padded dims of the input's own layout
  void *same = nullptr;  // rows_p x cols_p, the input's layout (null: scales only)
  void *swap = nullptr;  // cols_p x rows_p, transposed
  int64_t ld_same = 0, ld_swap = 0;  // row pitches (elements)
  int64_t s_same = 0, s_swap = 0;    // elements per matrix
  int32_t cdtype = NSG_F16;  // dtype of the copies
  // 1: `same` (bf16 here) is written only for the matrices whose e fails
  // raw_exponent_ok: the fallback operand of a kSrcRaw product
  int32_t raw_fallback = 0;
  float *gscale = nullptr;   // [G] r, followed by [G] int32 e
  int32_t *status = nullptr;
  int32_t batch = 0;
};

// Tile configurations of the GEMM kernels.
enum TileCfg : int { kTile128 = 0, kTile256 = 1 };
int tile_m(int cfg);

hipError_t launch_gemm(int dtype, bool symmetric, int cfg, const GemmArgs &a, hipStream_t s);
hipError_t launch_norm_reduce(const NormReduceArgs &a, hipStream_t s);
hipError_t launch_scale(const ScaleArgs &a, hipStream_t s);
hipError_t launch_copy(const void *src, void *dst, size_t bytes, hipStream_t s);

// Muon step (nsg_muon.hip)
hipError_t launch_muon_momentum(void *M, int m_dtype, const void *G, int g_dtype, int64_t n, float mu,
                                hipStream_t s);
hipError_t launch_muon_update(void *W, int w_dtype, const void *O, int o_dtype, int64_t n, float c1, float c2,
                              int stochastic, uint64_t seed, uint64_t step, hipStream_t s);

// selection front-end (nsg_select.hip)
int64_t l1_cols_chunks(int64_t R);
hipError_t launch_l1_norms(const void *in, int dtype, int64_t G, int64_t R, int64_t C, int dim, double *keys,
                           double *part, hipStream_t s);
hipError_t launch_topk(const double *keys, int64_t G, int64_t n, int64_t k, int32_t *idx, int32_t *pos,
                       hipStream_t s);
hipError_t launch_gather(const void *in, int dtype, int64_t G, int64_t R, int64_t C, int dim, const int32_t *idx,
                         int64_t k, void *out, hipStream_t s);
hipError_t launch_scatter(const void *O, int dtype, int64_t G, int64_t R, int64_t C, int dim, const int32_t *pos,
                          int64_t k, void *out, hipStream_t s);

}  // namespace nsg
