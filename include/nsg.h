/*
 * nsg.h — batched Newton–Schulz / Gram Newton–Schulz orthogonalization on
 * AMD Instinct MI355X (gfx950).  C ABI of libnsg.so.
 *
 * What is computed (the pages' notation: n <= m, alpha = m / n):
 *   For every matrix G_g of a bucket [G, R, C]:
 *     X  = G_g       if R <= C,   X = G_g^T  otherwise (short side leads;
 *          "muon" kernel card, "How it works")
 *     X0 = X / (s (||X||_F + eps))            (Dion3 paper, Alg. 1 / Alg. 3 step 2;
 *                                              safety factor s, App. B.2.2)
 *     NSG_STANDARD: T steps of  A = X X^T,  B = b_t A + c_t A^2,  X = a_t X + B X
 *                   (Dion3 paper, Section 2.2, Algorithm 1)
 *     NSG_GRAM:     R = X0 X0^T, Q = I, T steps of
 *                     Z = b_t R + c_t R^2,  Q = Q Z + a_t Q,
 *                     RZ = R Z + a_t R,     R = Z RZ + a_t RZ
 *                   with one restart (X = Q X, R = X X^T, Q = I) at the top of
 *                   step restart_after + 1, output Q X
 *                   (Dion3 paper, Section 4.2, Algorithm 3; the a*I terms are
 *                   applied in fp32 epilogues, never stored: Appendix B.2.3).
 *                   A square matrix (m == n) runs NSG_STANDARD instead
 *                   (Dion3 paper, Section 4.1, last paragraph).
 *     out_g = result (transposed back when R > C).
 *
 * Arithmetic: GEMM operands and every intermediate matrix are stored in the
 * compute dtype (fp16 by default, Alg. 3 step 3; bf16; or fp32 for the debug
 * path); products accumulate in fp32 and every epilogue (scales, a*X, a*Q,
 * a*R, a*RZ, the +a*I of a fresh Q) runs in fp32, rounding once to the
 * storage dtype (round to nearest even).  The Frobenius norm is a fixed-order
 * fp32 sum of squares.  Results depend only on (matrix, shape, parameters),
 * never on G or on the other matrices of the bucket.
 *
 * Conventions for every call below:
 *   - Memory: every pointer marked "device" is device memory owned by the
 *     caller; the library allocates nothing, frees nothing and never blocks
 *     the host.  ns_orthogonalize only enqueues work on `stream`.
 *   - Errors: argument problems are reported before anything is enqueued and
 *     leave `out` untouched.  A failed kernel launch returns NSG_ERR_HIP.
 *     Numerical blow-up is not an error: it is reported per matrix in
 *     `status` (when given).
 *   - Thread safety: calls are reentrant; concurrent calls need distinct
 *     workspaces.  The optional launch timing (ns_timing_*) is process-global.
 */
#ifndef NSG_H_
#define NSG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NSG_OK = 0,
  NSG_ERR_INVALID_ARG = 1,         /* null pointer, bad enum, bad steps/coeffs/safety */
  NSG_ERR_UNSUPPORTED_DTYPE = 2,   /* dtype code outside nsg_dtype_t */
  NSG_ERR_SHAPE = 3,               /* negative size, or a side above NSG_MAX_SIDE */
  NSG_ERR_WORKSPACE_TOO_SMALL = 4, /* workspace null, misaligned or too small */
  NSG_ERR_HIP = 5,                 /* a HIP runtime call or kernel launch failed */
  NSG_ERR_SCRATCH_TOO_SMALL = 6    /* ns_orthogonalize_noalloc: the bucket's workspace
                                      exceeds NSG_NOALLOC_MAX_BYTES */
} nsg_status_t;

typedef enum { NSG_F16 = 0, NSG_BF16 = 1, NSG_F32 = 2 } nsg_dtype_t;

typedef enum {
  NSG_STANDARD = 0, /* Algorithm 1 */
  NSG_GRAM = 1      /* Algorithm 3; square matrices fall back to Algorithm 1 */
} nsg_mode_t;

#define NSG_MAX_SIDE 65536 /* largest R or C accepted */
#define NSG_MAX_STEPS 64
#define NSG_WORKSPACE_ALIGN 256

typedef struct {
  int32_t steps;          /* T >= 1 (Muon: 5) */
  const double *coeffs;   /* host: 3 values (a, b, c) used at every step, or
                             3*steps values a_1,b_1,c_1,...; read during the
                             call only.  "muon" kernel card: (3.4445, -4.7750,
                             2.0315) */
  int32_t n_coeffs;       /* 3 or 3*steps */
  int32_t mode;           /* nsg_mode_t */
  int32_t restart_after;  /* NSG_GRAM: restart at the top of step
                             restart_after + 1 (Alg. 3: 2); 0, or >= steps,
                             means no restart (Alg. 2) */
  float safety;           /* s > 0 in X / (s (||X||_F + eps)); App. B.2.2
                             recommends 1.05 for Gram NS */
  float eps;              /* >= 0; Alg. 1: 1e-7 */
  int32_t compute_dtype;  /* nsg_dtype_t: F16 (Alg. 3), BF16 (Alg. 1), or F32
                             (debug path) */
  int32_t sym_updates;    /* NSG_GRAM only.  1: the products Q Z + a Q and
                             R Z + a R run on the symmetric kernel (lower
                             triangle computed, mirrored), as the Dion3 paper's
                             FLOP count in Section 4.1 assumes; Q, RZ and R are
                             then exactly symmetric.  0: both run as general
                             products.  Other values are an argument error. */
  uint64_t restart_mask;  /* NSG_GRAM only.  0: restart_after decides (one
                             restart).  Otherwise bit t-1 set restarts at the
                             top of step t (2 <= t <= steps): X <- Q X,
                             R <- X X^T, Q <- I, as often as the mask says
                             (Dion3 paper, Appendix B.2: repeated restarts;
                             B.2.1: multi-restart schedules).  Bit 0 or a bit
                             beyond `steps` is an argument error. */
} nsg_params_t;

/* Fills *p with the defaults: steps 5, the Muon triple, NSG_GRAM,
 * restart_after 2, safety 1.05, eps 1e-7, fp16 compute, sym_updates 1,
 * restart_mask 0.  The coefficient pointer refers to static storage inside
 * the library. */
void ns_default_params(nsg_params_t *p);

/* Bytes of device workspace ns_orthogonalize needs for a bucket of G
 * matrices of R x C with parameters *p.  Host only; no GPU needed.
 * Returns NSG_OK and writes *bytes (0 for an empty bucket), or an argument
 * error as ns_orthogonalize would. */
nsg_status_t ns_workspace_size(int64_t G, int64_t R, int64_t C,
                               const nsg_params_t *p, size_t *bytes);

/* Orthogonalize a bucket.
 *   in      device, [G, R, C] row-major contiguous, dtype in_dtype; read only.
 *           When in_dtype is the 16-bit compute dtype, R and C are multiples
 *           of 256, `in` is 16-byte aligned and `out` does not overlap it,
 *           the products read X0 = G 2^e straight from `in` (the exact power
 *           of two rides in their fp32 epilogue scale) and no scaled copy is
 *           written; the results are the same either way.
 *           Under the same conditions a bf16 input with fp16 compute and
 *           256 <= min(R, C) < 2048 is read in place too (larger buckets are
 *           bound by the MFMAs and keep the copy, which is then faster): the
 *           products that read X0 convert the bf16 values to the fp16 X0 the
 *           copy would hold, and the first X0 X0^T (Gram R0, or the standard
 *           step's A) multiplies the bf16 values themselves (their products
 *           are exact in fp32, so it is at least as accurate as from the fp16
 *           copy; entries of X0 below fp16's normal range keep their bits).  A matrix with |G|_F outside about [2^-20, 2^45] (where
 *           fp32 sums of raw products could overflow or small products
 *           flush) takes a scaled bf16 copy for that product instead.
 *   out     device, [G, R, C] row-major contiguous, dtype out_dtype; may be
 *           the same memory as `in` (the input is then fully consumed into
 *           the workspace before the first output write); any other overlap
 *           with `in` is an error the library does not detect.
 *   workspace  device, at least ns_workspace_size bytes, aligned to
 *           NSG_WORKSPACE_ALIGN; contents on entry are ignored and on exit
 *           undefined.
 *   status  device, G int32 values, or NULL.  Set to 0 for a matrix whose
 *           output is all finite, 1 otherwise.
 *   stream  hipStream_t to enqueue on (NULL = the default stream).
 * G == 0, R == 0 or C == 0 returns NSG_OK and enqueues nothing. */
nsg_status_t ns_orthogonalize(const void *in, int32_t in_dtype,
                              void *out, int32_t out_dtype,
                              int64_t G, int64_t R, int64_t C,
                              const nsg_params_t *p,
                              void *workspace, size_t workspace_bytes,
                              int32_t *status, void *stream);

/* ns_orthogonalize without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing and calls no
 * allocating routine.  Its workspace is a fixed array of
 * NSG_NOALLOC_MAX_BYTES inside the library: one copy per GPU, held from the
 * library's first use of that GPU until the process ends.
 *   in, out, G, R, C, p, status, stream: as for ns_orthogonalize (in, out and
 *           status are the caller's device memory).
 * A bucket whose ns_workspace_size exceeds NSG_NOALLOC_MAX_BYTES returns
 * NSG_ERR_SCRATCH_TOO_SMALL before anything is enqueued; other argument
 * errors as for ns_orthogonalize.  The array is looked up on the device
 * current on the calling thread, which must be the device of `stream`.
 * Every call on one GPU uses that GPU's single array: two calls that may
 * overlap on one GPU (different streams, or different host threads without
 * stream ordering between them) race on it.  Calls ordered on one stream are
 * safe; no call depends on what an earlier call left in the array.
 * Results are bit for bit those of ns_orthogonalize. */
#define NSG_NOALLOC_MAX_BYTES (128u << 20) /* 128 MiB */
nsg_status_t ns_orthogonalize_noalloc(const void *in, int32_t in_dtype,
                                      void *out, int32_t out_dtype,
                                      int64_t G, int64_t R, int64_t C,
                                      const nsg_params_t *p, int32_t *status,
                                      void *stream);

/* Static text for a status code. */
const char *ns_status_string(nsg_status_t s);

/* FLOPs per matrix of an R x C bucket, host only.
 *   credited: the pages' formula for the algorithm that runs —
 *             2T(2 alpha + 1) n^3 for standard NS (Dion3 paper, Section 2.2),
 *             (4T + 6 alpha - 6) n^3 for Gram NS with one restart
 *             (Section 4.1 plus 3(alpha - 1) n^3, Section 4.2), and
 *             (4T + 3 alpha - 3) n^3 without a restart (Section 4.1);
 *   executed: 2 M N K summed over the tiles the launch plan actually runs
 *             (symmetric products count only their lower-triangle tiles;
 *             padding to whole tiles included). */
nsg_status_t ns_flops(int64_t R, int64_t C, const nsg_params_t *p,
                      double *credited, double *executed);

/* One entry of the launch plan (host only): what each kernel launch of a
 * call does, per matrix. */
typedef struct {
  int32_t kind;     /* 0 norm reduce, 1 scale/cast/transpose (scales only
                       when the input is read in place), 2 general GEMM,
                       3 symmetric GEMM */
  int32_t step;     /* NS step t (1..T); 0 before the loop, T+1 for the output */
  int64_t M, N, K;  /* GEMM logical sizes (0 for the normalize kernels) */
  double flops;     /* executed FLOPs per matrix (tiles run, 2MNK per tile) */
  double bytes;     /* algorithmic HBM bytes per matrix (16-bit output
                       assumed): every distinct matrix the launch
                       reads, once (an operand that is also the added term,
                       or a matrix and its transposed copy, count once), and
                       every matrix of the method it writes, once (transposed
                       copies and mirrored halves are not counted) */
  char label[24];   /* e.g. "R0=XXt", "Z", "Q=QZ+aQ", "RZ", "R=Z.RZ", "Y=QX" */
  int32_t a_kmajor; /* 1: A is read from a K-major buffer (K x M), else M x K */
  int32_t b_kmajor; /* 1: B is read from a K-major buffer (K x N), else N x K */
  int32_t source;   /* where a GEMM's operands come from: 0 the compute dtype
                       (workspace, or the input in place); for a bf16 input
                       under fp16 compute read in place, 1 (2): A (B) is the
                       input, converted to fp16 X0 = RNE(G 2^e) on its way to
                       LDS; 3: a symmetric product of the raw bf16 input on
                       bf16 MFMAs (fp32 accumulation) with fp16 outputs */
} nsg_launch_info_t;

/* Writes up to max_entries launch descriptions for one call on an R x C
 * bucket with input dtype in_dtype and the total count to *count (host
 * only).  The list is that of an aligned input that the output does not
 * overlap; the number of launches never depends on the input. */
nsg_status_t ns_plan(int64_t R, int64_t C, int32_t in_dtype, const nsg_params_t *p,
                     nsg_launch_info_t *entries, int32_t max_entries,
                     int32_t *count);

/* Optional per-launch timing with HIP events, for the benchmark's roofline.
 * ns_timing_enable(1) makes every later ns_orthogonalize call record a
 * hipEvent before and after each of its kernel launches, on the stream the
 * kernels run on.  ns_timing_collect waits for the recorded events, writes up
 * to max_entries (kind, milliseconds) pairs in launch order, sets *count to
 * the number recorded since the last collect or enable, and clears them.
 * Timing is process-global and meant for single-threaded benchmarking. */
nsg_status_t ns_timing_enable(int32_t on);
nsg_status_t ns_timing_collect(int32_t *kinds, float *ms, int32_t max_entries,
                               int32_t *count);

/* Plain device-to-device copy kernel (16-byte vector loads/stores), used to
 * calibrate hardware byte counters against a known traffic.  src and dst are
 * device pointers of `bytes` bytes each, 16-byte aligned, not overlapping. */
nsg_status_t nsg_copy(const void *src, void *dst, size_t bytes, void *stream);


/* Building block, exposed for testing the GEMM kernels on their own.
 * For b in [0, batch):  V = alpha * A_b B_b^T + beta * Cin_b   (fp32), then
 *   out_b   = V           (row-major M x N, ld ldo)       if out   != NULL
 *   out_t_b = V^T         (row-major N x M, ld ldt)       if out_t != NULL
 *   out_d_b = V + diag*I  (row-major M x N, ld ldo)       if out_d != NULL
 * A_b is M x K (ld lda), B_b is N x K (ld ldb), Cin_b is M x N (ld ldc);
 * with a_trans = 1 A_b is stored K-major instead (K x M, ld lda >= M), with
 * b_trans = 1 likewise B_b (K x N, ld ldb >= N): fp16 / bf16 with the
 * 256 x 256 kernel only, both for a symmetric product, b_trans alone or
 * both for a general one (anything else is NSG_ERR_INVALID_ARG);
 * operands, Cin and outputs are in `dtype`; batches are contiguous
 * ([batch][rows][ld]).  symmetric != 0 computes only the tiles on or below
 * the diagonal and mirrors them (requires M == N and out_t == NULL); the
 * result is then exactly symmetric (the symmetric GEMM of the Dion3 paper,
 * Section 5 and Appendix C.1).  M, N and K must be multiples of 256.
 * tile selects the kernel: 128 or 256 (output tile edge), 0 = as
 * ns_orthogonalize would choose.  status (device, batch int32, or NULL):
 * set to 1 for a batch whose out contains a non-finite value after rounding
 * to `dtype` (entries of the others are left as they are).  All pointers are
 * device memory, 16-byte aligned. */
nsg_status_t nsg_gemm_nt(int32_t dtype, int32_t symmetric, int64_t batch,
                         int64_t M, int64_t N, int64_t K,
                         const void *A, int64_t lda, int32_t a_trans,
                         const void *B, int64_t ldb, int32_t b_trans,
                         float alpha, float beta, const void *Cin, int64_t ldc,
                         void *out, int64_t ldo, void *out_t, int64_t ldt,
                         void *out_d, float diag, int32_t tile, int32_t *status,
                         void *stream);

/* ---- Dion3 selection front-end --------------------------------------------
 * Dion3 paper, Section 6 ("Selection", "Orthogonalization") and Algorithm 4,
 * steps 3-4: for every matrix M of the bucket, S = the k rows (or columns)
 * with the largest l1 norm, O = Newton-Schulz(M[S, :]) (or M[:, S]).  The
 * update and error-feedback steps of Algorithm 4 are not part of it. */
#define NSG_SELECT_ROWS 0
#define NSG_SELECT_COLS 1
#define NSG_SELECT_SMALLER (-1) /* rows if R <= C, else columns (the pages'
                                   choice when the weight is not sharded) */

/* The selection size rule of the Dion3 paper, Section 6 ("Selection") and
 * Algorithm 4, step 3, host only: k = ceil(f n) lines (at least 1, at most
 * n) of the dimension `dim` resolves to, n = R for rows, C for columns.
 * NSG_SELECT_SMALLER resolves to columns when C < R, else rows (the pages'
 * choice for an unsharded weight: whichever dimension is smaller).
 *   fraction  f in (0, 1]; anything else is NSG_ERR_INVALID_ARG
 *   dim_out   resolved NSG_SELECT_ROWS or NSG_SELECT_COLS
 *   k_out     lines to select (0 when n == 0)
 * Negative or oversized R, C: NSG_ERR_SHAPE; a null output pointer or a bad
 * dim: NSG_ERR_INVALID_ARG. */
nsg_status_t ns_select_count(int64_t R, int64_t C, int32_t dim, double fraction,
                             int32_t *dim_out, int64_t *k_out);

/* Bytes of device workspace ns_orthogonalize_selected needs (host only).
 * Same argument rules as ns_orthogonalize_selected. */
nsg_status_t ns_select_workspace_size(int64_t G, int64_t R, int64_t C, int64_t k,
                                      int32_t dim, int32_t in_dtype, int32_t out_dtype,
                                      const nsg_params_t *p, size_t *bytes);

/* Selection + orthogonalization of a bucket.
 *   in   [G, R, C] row-major, contiguous, in_dtype (device)
 *   out  [G, R, C] out_dtype (device; may alias in): O in the selected rows
 *        (columns), zeros in the others
 *   k    lines to select per matrix, 1 <= k <= n, with n = R for rows and
 *        n = C for columns (the pages: k = ceil(f n) for a fraction f)
 *   dim  NSG_SELECT_ROWS, NSG_SELECT_COLS or NSG_SELECT_SMALLER
 *   idx  device [G][k] int32 or NULL: the selected indices, ascending
 *   status  as for ns_orthogonalize (per matrix, may be NULL)
 * Norms are fp64 sums of |M_ij| in a fixed order; equal norms go to the lower
 * index.  O is exactly what ns_orthogonalize returns for the gathered k x C
 * (R x k) submatrix with *p.  Errors as for ns_orthogonalize; k out of range
 * or a bad dim is NSG_ERR_INVALID_ARG.  An empty bucket (G = 0) is a no-op. */
nsg_status_t ns_orthogonalize_selected(const void *in, int32_t in_dtype, void *out,
                                       int32_t out_dtype, int64_t G, int64_t R, int64_t C,
                                       int64_t k, int32_t dim, const nsg_params_t *p,
                                       void *workspace, size_t workspace_bytes,
                                       int32_t *idx, int32_t *status, void *stream);

/* Building blocks of the selection, exposed for tests.
 * nsg_l1_norms: keys[g][i] = sum_j |M_g[i, j]| (dim 0) or sum_j |M_g[j, i]|
 * (dim 1) in fp64, fixed order; keys is device [G][n].  Column norms need
 * nsg_l1_workspace_size bytes of device workspace (0 for rows).
 * nsg_topk: per matrix the k largest of keys[g][0..n) (equal keys: lower
 * index first), written ascending to idx[g][0..k); pos[g][i] = rank of i
 * among them, -1 if not selected (pos may not be NULL). */
nsg_status_t nsg_l1_workspace_size(int64_t G, int64_t R, int64_t C, int32_t dim,
                                   size_t *bytes);
nsg_status_t nsg_l1_norms(const void *in, int32_t dtype, int64_t G, int64_t R, int64_t C,
                          int32_t dim, double *keys, void *workspace,
                          size_t workspace_bytes, void *stream);
nsg_status_t nsg_topk(const double *keys, int64_t G, int64_t n, int64_t k, int32_t *idx,
                      int32_t *pos, void *stream);

/* ---- The Muon step around the orthogonalization -------------------------
 * Dion3 paper, Section 2.1, Eq. (1): M <- mu M + G, W <- W - lr polar(M);
 * Algorithm 4, steps 8-9: decoupled weight decay and the update in one
 * pass, W <- (1 - lr wd) W - lr s O; the "muon" kernel card: bf16 W written
 * back with counter-based stochastic rounding keyed by the element's global
 * index.  All arithmetic is fp32, one rounding per operation, no fused
 * multiply-add: t = mu m, m' = t + g; c1 = f32(1 - lr wd), c2 = f32(lr s)
 * (from the double arguments), w' = c1 w - c2 o.  Stochastic rounding adds
 * 16 random bits to the fp32 pattern and truncates (non-finite values round
 * to nearest even); the bits come from Philox-4x32-10 (Salmon et al., SC 2011)
 * with key = seed and counter = (i >> 3, step): element i uses the 16-bit half
 * i & 1 of output word (i & 7) >> 1.  Reproducible bit for bit for a fixed
 * (seed, step). */

/* M [n] (F32 or BF16, rounded to nearest even) <- mu M + G [n] (any dtype).
 * Device pointers; returns before running (stream order). */
nsg_status_t ns_muon_momentum(void *M, int32_t m_dtype, const void *G, int32_t g_dtype,
                              int64_t n, float mu, void *stream);

/* W [n] (F32, or BF16 with stochastic != 0 for stochastic rounding, else
 * nearest even) <- (1 - lr wd) W - lr scale O [n] (any dtype). */
nsg_status_t ns_muon_update(void *W, int32_t w_dtype, const void *O, int32_t o_dtype, int64_t n,
                            double lr, double weight_decay, double scale, int32_t stochastic,
                            uint64_t seed, uint64_t step, void *stream);

/* One Muon step for a bucket of G matrices R x C: ns_muon_momentum, then
 * O = ns_orthogonalize(M) with *p (fp32 output in the workspace), then
 * ns_muon_update(W, O).  W, M, Gr are [G, R, C] contiguous device arrays;
 * status as for ns_orthogonalize.  Workspace: ns_muon_workspace_size. */
nsg_status_t ns_muon_workspace_size(int64_t G, int64_t R, int64_t C, const nsg_params_t *p,
                                    size_t *bytes);
nsg_status_t ns_muon_step(void *W, int32_t w_dtype, void *M, int32_t m_dtype, const void *Gr,
                          int32_t g_dtype, int64_t G, int64_t R, int64_t C, float mu, double lr,
                          double weight_decay, double scale, int32_t stochastic, uint64_t seed,
                          uint64_t step, const nsg_params_t *p, void *workspace,
                          size_t workspace_bytes, int32_t *status, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NSG_H_ */
