// Host runtime of libnsg: argument validation, the bucket planner (transpose,
// mode, tile configuration, workspace layout, launch list, FLOP tally) and the
// sequencer that enqueues the standard or Gram Newton–Schulz launches.
//
// The launch lists follow the Dion3 paper: Algorithm 1 (standard NS) and
// Algorithm 3 (stabilized Gram NS, with the a*I terms moved into fp32
// epilogues as in Appendix B.2.3).  Square matrices run Algorithm 1 in "gram"
// mode (Section 4.1, last paragraph).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "nsg.h"
#include "nsg_internal.h"

namespace nsg {
namespace {

const double kMuon[3] = {3.4445, -4.7750, 2.0315};  // "muon" kernel card, "How it works"

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
size_t dtype_size(int dt) { return dt == NSG_F32 ? 4 : 2; }
bool valid_dtype(int dt) { return dt == NSG_F16 || dt == NSG_BF16 || dt == NSG_F32; }

// Workspace buffers, each [G][rows][cols] in the compute dtype unless noted.
enum Buf : int {
  kPartials = 0,  // fp32 [G][nchunks]
  kGScale,        // fp32 [G] residual scale r, then int32 [G] exponent e
  kX0,            // np x mp   (X0 scaled by 2^e)
  kX0T,           // mp x np
  kX1,            // np x mp   (X after the restart / standard ping-pong)
  kX1T,           // mp x np
  kS0, kS1, kS2, kS3, kS4, kS5,  // np x np
  kNumBufs
};

struct Launch {
  int kind = 0;  // 0 reduce, 1 scale, 2 gen GEMM, 3 sym GEMM
  int step = 0;
  std::string label;
  int A = kNone, B = kNone, Cin = kNone, out0 = kNone, out1 = kNone, out2 = kNone;
  int M = 0, N = 0, K = 0, Mv = 0, Nv = 0;
  int at = 0, bt = 0;  // operand stored K-major (K x M / K x N)
  float alpha = 1.f, beta = 0.f, diag = 0.f;
  int gpow = 0;
  int gexp = 0;  // an operand is the caller's input, read in place
  int src = kSrcPlain;  // OperandSource of the 256 x 256 kernel
  bool final_out = false;
  double flops = 0.0, bytes = 0.0;
};

struct Plan {
  int64_t R = 0, C = 0, n = 0, m = 0, np = 0, mp = 0;
  bool tr = false;
  bool gram = false;
  // one layout of X only (the input's own: X^T for tall inputs, X for wide
  // ones); the products that need the other read it K-major
  bool single = false;
  // the products read the caller's input where they would read X0 (one
  // layout, 16-bit input in the compute dtype, R and C multiples of kPad):
  // the scale pass then only finds the scales and writes no copy
  bool direct = false;
  // the same for a bf16 input under fp16 compute (n < 2048): the first
  // X X^T (R0, or the standard step's A) on bf16 MFMAs from the raw input,
  // the general products that read X0 convert it on its way to LDS (and in
  // their epilogue, where X0 is also the added term of X = a X + B X); the
  // scale pass writes the bf16 copy G 2^e only for matrices whose exponent
  // fails raw_exponent_ok (the first X X^T reads those)
  bool cvt = false;
  int in_dtype = NSG_F16;
  int T = 0;
  uint64_t restarts = 0;  // bit t-1: restart at the top of step t
  bool restart_at(int t) const { return t >= 1 && t <= 64 && ((restarts >> (t - 1)) & 1u); }
  int cdtype = NSG_F16;
  int cfg = kTile128;
  int fexp = 0;
  int nchunks = 0;
  std::vector<double> a, b, c;
  std::vector<Launch> launches;
  // workspace layout: per-buffer byte offset and per-matrix element stride
  size_t off[kNumBufs] = {0};
  // rows x cols padded extent; ld = cols + skew (elements between rows)
  int64_t rows[kNumBufs] = {0}, cols[kNumBufs] = {0}, ld[kNumBufs] = {0};
  bool used[kNumBufs] = {false};
  size_t total = 0;
};

nsg_status_t validate_params(const nsg_params_t *p) {
  if (p == nullptr) return NSG_ERR_INVALID_ARG;
  if (p->steps < 1 || p->steps > NSG_MAX_STEPS) return NSG_ERR_INVALID_ARG;
  if (p->coeffs == nullptr) return NSG_ERR_INVALID_ARG;
  if (p->n_coeffs != 3 && p->n_coeffs != 3 * p->steps) return NSG_ERR_INVALID_ARG;
  for (int i = 0; i < p->n_coeffs; ++i)
    if (!std::isfinite(p->coeffs[i])) return NSG_ERR_INVALID_ARG;
  if (p->mode != NSG_STANDARD && p->mode != NSG_GRAM) return NSG_ERR_INVALID_ARG;
  if (p->restart_after < 0) return NSG_ERR_INVALID_ARG;
  if (!(p->safety > 0.f) || !std::isfinite(p->safety)) return NSG_ERR_INVALID_ARG;
  if (!(p->eps >= 0.f) || !std::isfinite(p->eps)) return NSG_ERR_INVALID_ARG;
  if (!valid_dtype(p->compute_dtype)) return NSG_ERR_UNSUPPORTED_DTYPE;
  if (p->sym_updates != 0 && p->sym_updates != 1) return NSG_ERR_INVALID_ARG;
  if (p->restart_mask != 0) {
    if (p->restart_mask & 1u) return NSG_ERR_INVALID_ARG;  // no restart before step 1
    if (p->steps < 64 && (p->restart_mask >> p->steps) != 0) return NSG_ERR_INVALID_ARG;
  }
  return NSG_OK;
}

nsg_status_t validate_shape(int64_t G, int64_t R, int64_t C) {
  if (G < 0 || R < 0 || C < 0) return NSG_ERR_SHAPE;
  if (R > NSG_MAX_SIDE || C > NSG_MAX_SIDE || G > 65535) return NSG_ERR_SHAPE;
  return NSG_OK;
}

// Tile configuration from (n, m, dtype) only — never from G — so a matrix's
// arithmetic is the same in any bucket.  16-bit matrices with n > 128 take
// the 256 x 256 kernel: whole calls at n = 256 ran 1.1-2.1x faster on it
// than on the 128 x 128 kernel at every bucket size measured (1 to 1024
// matrices).  At n <= 128 the 256 x 256 tile is mostly padding; it won only
// for large buckets (512 matrices of 128 x 512: 1.25 against 1.96 ms) and
// lost for small ones (1 and 8 matrices), so those keep the 128 x 128 kernel.
// NSG_TILE=128|256 in the environment forces a tile configuration (a
// debugging and tuning aid; it applies to every matrix alike).
int choose_cfg(int64_t n, int64_t mp, int dt) {
  (void)mp;
  static const int forced = [] {
    const char *e = std::getenv("NSG_TILE");
    if (e == nullptr) return 0;
    const int v = std::atoi(e);
    return (v == 128 || v == 256) ? v : 0;
  }();
  if (forced == 128) return kTile128;
  if (forced == 256) return kTile256;
  if (dt == NSG_F32) return kTile128;  // debug path
  return n > 128 ? kTile256 : kTile128;
}

double sym_tiles(int64_t M, int bm) {
  const double t = (double)(M / bm);
  return t * (t + 1.0) / 2.0;
}

void add_gemm(Plan &P, bool sym, int step, const char *label, int A, int B, int Cin, int out0,
              int out1, int out2, int64_t M, int64_t N, int64_t K, int64_t Mv, int64_t Nv, double alpha,
              double beta, double diag, int gpow, bool final_out) {
  Launch L;
  L.kind = sym ? 3 : 2;
  L.step = step;
  L.label = label;
  L.A = A; L.B = B; L.Cin = Cin; L.out0 = out0; L.out1 = out1; L.out2 = out2;
  L.M = (int)M; L.N = (int)N; L.K = (int)K; L.Mv = (int)Mv; L.Nv = (int)Nv;
  L.alpha = (float)alpha; L.beta = (float)beta; L.diag = (float)diag;
  L.gpow = gpow;
  L.gexp = (A == kInUser || B == kInUser || Cin == kInUser) ? 1 : 0;
  L.final_out = final_out;
  const int bm = tile_m(P.cfg);
  L.flops = sym ? 2.0 * sym_tiles(M, bm) * bm * bm * (double)K : 2.0 * (double)M * N * K;
  // algorithmic bytes: every distinct matrix the product reads, read once,
  // and the matrices it defines, written once.  A buffer and its transposed
  // copy are one matrix (X0 / X0^T, X1 / X1^T, RZ / RZ^T); a Cin that is an
  // operand (Z = b R + c R^2 reads R once) is not counted again; the
  // transposed copy out1 is a layout choice, not an output of the method.
  const double es = (double)dtype_size(P.cdtype);
  // valid K: K of a GEMM over X's long side is m, else n
  const double Kv = (K == P.mp) ? (double)P.m : (double)P.n;
  auto matrix_of = [](int id) {
    if (id == kX0T || id == kInUser) return (int)kX0;
    if (id == kX1T) return (int)kX1;
    if (id == kS5) return (int)kS4;
    return id;
  };
  const int ma = matrix_of(A), mb = matrix_of(B), mc = matrix_of(Cin);
  double bytes = es * (double)Mv * Kv;
  if (mb != ma) bytes += es * (double)Nv * Kv;
  if (Cin != kNone && mc != ma && mc != mb) bytes += es * (double)Mv * Nv;
  bytes += es * ((out0 != kNone) + (out2 != kNone)) * (double)Mv * Nv;
  L.bytes = bytes;
  for (int id : {A, B, Cin, out0, out1, out2})
    if (id >= 0) P.used[id] = true;
  P.launches.push_back(L);
}

// in_dtype: the input's dtype; in_place_ok: the input may be read in place
// (16-byte aligned, no overlap with the output).
nsg_status_t build_plan(int64_t R, int64_t C, const nsg_params_t *p, int64_t G, int out_dtype, int in_dtype,
                        bool in_place_ok, Plan &P) {
  P.R = R; P.C = C;
  P.tr = R > C;
  P.n = std::min(R, C);
  P.m = std::max(R, C);
  P.np = round_up(P.n, kPad);
  P.mp = round_up(P.m, kPad);
  P.T = p->steps;
  P.cdtype = p->compute_dtype;
  P.gram = (p->mode == NSG_GRAM) && (P.n < P.m);
  P.restarts = 0;
  if (P.gram) {
    if (p->restart_mask != 0) P.restarts = p->restart_mask;
    else if (p->restart_after >= 1 && p->restart_after < P.T) P.restarts = 1ull << p->restart_after;
  }
  P.cfg = choose_cfg(P.n, P.mp, P.cdtype);
  P.single = (P.cfg == kTile256) && (P.cdtype != NSG_F32);
  P.in_dtype = in_dtype;
  P.direct = P.single && in_dtype == P.cdtype && in_place_ok && R % kPad == 0 && C % kPad == 0;
  // Measured per Gram call against the copy (bf16 N(0,1) inputs, same data):
  // +3.2% at n = 512, +2.4% at 768, +1.5% at 1024, +0.3% at 1536, -0.4% at
  // 2048, -1.7% at 3072 and 4096.  The conversion's VALU work and raw staging
  // cost the compute-bound X = Q X0 of a large n more than the saved copy.
  P.cvt = P.single && in_dtype == NSG_BF16 && P.cdtype == NSG_F16 && in_place_ok && R % kPad == 0 &&
          C % kPad == 0 && P.n < 2048;
  // power-of-two range shift f ~ log2(sqrt(n)): keeps X0 = X/||X||_F and
  // R0 = X0 X0^T away from fp16 subnormals (X0 entries ~ 1/sqrt(nm)).
  P.fexp = (int)std::floor(std::log2((double)P.n) / 2.0);
  if (P.fexp < 0) P.fexp = 0;
  P.nchunks = (int)((R * C + kNormChunk - 1) / kNormChunk);
  P.a.resize(P.T); P.b.resize(P.T); P.c.resize(P.T);
  for (int t = 0; t < P.T; ++t) {
    const double *cc = (p->n_coeffs == 3) ? p->coeffs : p->coeffs + 3 * t;
    P.a[t] = cc[0]; P.b[t] = cc[1]; P.c[t] = cc[2];
  }
  const int64_t np = P.np, mp = P.mp, n = P.n, m = P.m;
  const double two_f = std::ldexp(1.0, P.fexp);  // 2^f
  const double xs0 = 1.0 / two_f;                  // X0 = r 2^-f X_stored

  for (int i = 0; i < kNumBufs; ++i) { P.rows[i] = 0; P.cols[i] = 0; P.ld[i] = 0; P.used[i] = false; }
  P.rows[kX0] = np; P.cols[kX0] = mp;
  P.rows[kX0T] = mp; P.cols[kX0T] = np;
  P.rows[kX1] = np; P.cols[kX1] = mp;
  P.rows[kX1T] = mp; P.cols[kX1T] = np;
  for (int i = kS0; i <= kS5; ++i) { P.rows[i] = np; P.cols[i] = np; }
  // Row pitch = padded width, plus 128 bytes when the width is a multiple of
  // 4 KB: consecutive rows of an operand tile then start in different L2
  // channels (such a pitch sends every row of a tile slice to the same
  // channel).  Other widths keep their pitch: with the skew the MoE bucket's
  // 1 KB rows (n = 512) became 1152 bytes, which stores more slowly (a store
  // probe on every CU: 13.2K against 12.1K cycles per 256 KB), and the
  // bucket ran 2.4% slower (same box, same bits).
  const int64_t skew = 128 / (int64_t)dtype_size(P.cdtype);
  for (int i = kX0; i < kNumBufs; ++i)
    P.ld[i] = P.cols[i] + ((P.cols[i] * (int64_t)dtype_size(P.cdtype)) % 4096 == 0 ? skew : 0);
  P.used[kPartials] = P.used[kGScale] = true;

  {
    Launch L; L.kind = 0; L.label = "norm_reduce"; L.bytes = (double)R * C * dtype_size(in_dtype);
    P.launches.push_back(L);
    Launch S; S.kind = 1; S.label = (P.direct || P.cvt) ? "scales" : "scale_cast_T"; S.bytes = 0;
    P.launches.push_back(S);
  }
  // the X0 buffers are reserved in every case (ping-pong and restart targets
  // too), so the workspace size does not depend on the input
  if (P.single) P.used[P.tr ? kX0T : kX0] = true;
  else P.used[kX0] = P.used[kX0T] = true;
  // where X0 is read from: the stored copy, or the input in place
  const bool in_place = P.direct || P.cvt;
  const int X0s = in_place && !P.tr ? (int)kInUser : (int)kX0;
  const int X0Ts = in_place && P.tr ? (int)kInUser : (int)kX0T;
  const int last = P.T + 1;
  const int OUT = kOutUser;
  const bool sgl = P.single, tr = P.tr;
  auto kmajor = [&](int a, int b) { P.launches.back().at = a; P.launches.back().bt = b; };

  if (!P.gram) {
    // Algorithm 1: A = X X^T ; B = b A + c A^2 ; X = a X + B X.
    int X = X0s, XT = X0Ts, Xn = kX1, XnT = kX1T;
    double xs = xs0;
    int xpow = 1;
    for (int t = 1; t <= P.T; ++t) {
      const double a = P.a[t - 1], b = P.b[t - 1], c = P.c[t - 1];
      // A_true = xs^2 r^(2 xpow) X_s X_s^T; stored A~ = A_true / xs^2
      if (sgl && tr) {  // A = X X^T from X^T read K-major
        add_gemm(P, true, t, "A=XXt", XT, XT, kNone, kS0, kNone, kNone, np, np, mp, n, n, 1.0, 0.0, 0.0,
                 2 * xpow, false);
        kmajor(1, 1);
      } else {
        add_gemm(P, true, t, "A=XXt", X, X, kNone, kS0, kNone, kNone, np, np, mp, n, n, 1.0, 0.0, 0.0,
                 2 * xpow, false);
      }
      const double as = xs * xs;
      add_gemm(P, true, t, "B=bA+cA2", kS0, kS0, kS0, kS1, kNone, kNone, np, np, np, n, n, c * as * as,
               b * as, 0.0, 0, false);
      if (t < P.T) {
        if (sgl && tr) {  // X'^T = a X^T + X^T B (B exactly symmetric)
          add_gemm(P, false, t, "Xt=aXt+XtB", XT, kS1, XT, XnT, kNone, kNone, mp, np, np, m, n, xs, a * xs, 0.0,
                   xpow, false);
        } else if (sgl) {  // X' = a X + B X with X read K-major
          add_gemm(P, false, t, "X=aX+BX", kS1, X, X, Xn, kNone, kNone, np, mp, np, n, m, xs, a * xs, 0.0,
                   xpow, false);
          kmajor(0, 1);
        } else {
          add_gemm(P, false, t, "X=aX+BX", kS1, XT, X, Xn, XnT, kNone, np, mp, np, n, m, xs, a * xs, 0.0,
                   xpow, false);
        }
        std::swap(X, Xn);
        std::swap(XT, XnT);
        // the input is never written: its ping-pong partner is the X0 buffer
        if (Xn == kInUser) Xn = kX0;
        if (XnT == kInUser) XnT = kX0T;
      } else if (P.tr) {
        // X'^T = a X^T + X^T B (B exactly symmetric): NT with A = X^T, B = B
        add_gemm(P, false, last, "Yt=aXt+XtB", XT, kS1, XT, OUT, kNone, kNone, mp, np, np, m, n, xs,
                 a * xs, 0.0, xpow, true);
      } else if (sgl) {
        add_gemm(P, false, last, "Y=aX+BX", kS1, X, X, OUT, kNone, kNone, np, mp, np, n, m, xs, a * xs,
                 0.0, xpow, true);
        kmajor(0, 1);
      } else {
        add_gemm(P, false, last, "Y=aX+BX", kS1, XT, X, OUT, kNone, kNone, np, mp, np, n, m, xs, a * xs,
                 0.0, xpow, true);
      }
      xs = 1.0;
      xpow = 0;
    }
  } else {
    // Algorithm 3 with the implicit a*I form of Appendix B.2.3.
    int Xb = X0s, XbT = X0Ts;
    double xs = xs0;
    int xpow = 1;
    int Rb = kS0, Zb = kS1, Qcur = kNone, Qfree[2] = {kS2, kS3}, RZb = kS4, RZTb = kS5;
    const bool symu = p->sym_updates != 0;
    bool r_scaled = true;  // R_true = 2^-2f R_stored (only R0)
    if (sgl && tr) {
      add_gemm(P, true, 0, "R0=XXt", XbT, XbT, kNone, Rb, kNone, kNone, np, np, mp, n, n, 1.0, 0.0, 0.0, 2,
               false);
      kmajor(1, 1);
    } else {
      add_gemm(P, true, 0, "R0=XXt", Xb, Xb, kNone, Rb, kNone, kNone, np, np, mp, n, n, 1.0, 0.0, 0.0, 2,
               false);
    }
    for (int t = 1; t <= P.T; ++t) {
      const double a = P.a[t - 1], b = P.b[t - 1], c = P.c[t - 1];
      if (P.restart_at(t)) {
        // X <- Q X ; R <- X X^T ; Q <- I   (Alg. 3, "restart to stabilize");
        // repeated restarts alternate between the two X buffers
        const int Xn = (Xb == kX1 || XbT == kX1T) ? kX0 : kX1, XnT = (Xb == kX1 || XbT == kX1T) ? kX0T : kX1T;
        if (sgl && tr) {  // X^T <- X^T Q^T, and R = X X^T from X^T read K-major
          add_gemm(P, false, t, "Xt=XtQt", XbT, Qcur, kNone, XnT, kNone, kNone, mp, np, np, m, n, xs, 0.0, 0.0,
                   xpow, false);
          Xb = Xn; XbT = XnT; xs = 1.0; xpow = 0;
          add_gemm(P, true, t, "R=XXt", XbT, XbT, kNone, Rb, kNone, kNone, np, np, mp, n, n, 1.0, 0.0, 0.0,
                   0, false);
          kmajor(1, 1);
        } else {
          if (sgl) {  // X <- Q X with X read K-major
            add_gemm(P, false, t, "X=QX", Qcur, Xb, kNone, Xn, kNone, kNone, np, mp, np, n, m, xs, 0.0, 0.0,
                     xpow, false);
            kmajor(0, 1);
          } else {
            add_gemm(P, false, t, "X=QX", Qcur, XbT, kNone, Xn, XnT, kNone, np, mp, np, n, m, xs, 0.0, 0.0,
                     xpow, false);
          }
          Xb = Xn; XbT = XnT; xs = 1.0; xpow = 0;
          add_gemm(P, true, t, "R=XXt", Xb, Xb, kNone, Rb, kNone, kNone, np, np, mp, n, n, 1.0, 0.0, 0.0,
                   0, false);
        }
        r_scaled = false;
        Qcur = kNone;
      }
      const double rs = r_scaled ? 1.0 / (two_f * two_f) : 1.0;
      // Z = b R + c R^2 ; with Q = I the new Q = Z + a I comes from the same
      // fp32 accumulator (second store).
      const int qnew = (Qcur == kNone) ? Qfree[0] : kNone;
      add_gemm(P, true, t, qnew != kNone ? "Z (+Q=Z+aI)" : "Z=bR+cR2", Rb, Rb, Rb, Zb, kNone, qnew, np, np,
               np, n, n, c * rs * rs, b * rs, a, 0, false);
      if (Qcur == kNone) {
        Qcur = Qfree[0];
      } else {
        const int qn = (Qcur == Qfree[0]) ? Qfree[1] : Qfree[0];
        // Q Z = Q Z^T (Z is exactly symmetric); on the symmetric kernel the
        // lower triangle is computed and mirrored
        add_gemm(P, symu, t, "Q=QZ+aQ", Qcur, Zb, Qcur, qn, kNone, kNone, np, np, np, n, n, 1.0, a, 0.0, 0,
                 false);
        Qcur = qn;
      }
      const bool need_r = (t < P.T) && !P.restart_at(t + 1);
      if (need_r) {
        // RZ = R Z + a R (stored with R's scale); as a general product it is
        // also written transposed, as a symmetric one RZ^T = RZ exactly
        add_gemm(P, symu, t, "RZ=RZ+aR", Rb, Zb, Rb, RZb, symu ? kNone : RZTb, kNone, np, np, np, n, n, 1.0,
                 a, 0.0, 0, false);
        // R = Z RZ + a RZ : NT with B = RZ^T
        add_gemm(P, true, t, "R=Z.RZ+aRZ", Zb, symu ? RZb : RZTb, RZb, Rb, kNone, kNone, np, np, np, n, n, rs,
                 a * rs, 0.0, 0, false);
        r_scaled = false;
      }
    }
    if (P.tr) {
      // Y^T = X^T Q^T : NT with A = X^T (m x n), B = Q
      add_gemm(P, false, last, "Yt=XtQt", XbT, Qcur, kNone, OUT, kNone, kNone, mp, np, np, m, n, xs, 0.0,
               0.0, xpow, true);
    } else if (sgl) {
      add_gemm(P, false, last, "Y=QX", Qcur, Xb, kNone, OUT, kNone, kNone, np, mp, np, n, m, xs, 0.0, 0.0,
               xpow, true);
      kmajor(0, 1);
    } else {
      add_gemm(P, false, last, "Y=QX", Qcur, XbT, kNone, OUT, kNone, kNone, np, mp, np, n, m, xs, 0.0, 0.0,
               xpow, true);
    }
  }
  // the scale pass reads the input once and writes X0 once (its transposed
  // copy is a layout choice); reading the input in place, it moves nothing
  P.launches[1].bytes =
      in_place ? 0.0 : (double)R * C * dtype_size(in_dtype) + (double)n * m * dtype_size(P.cdtype);
  if (P.cvt) {
    // operand sources of the products that read the bf16 input: R0 raw
    // (its 2^e factor in the epilogue), the others converted (already
    // scaled)
    for (Launch &L : P.launches) {
      if (L.kind < 2 || (L.A != kInUser && L.B != kInUser)) continue;
      if (L.kind == 3) {
        L.src = kSrcRaw;
        L.gexp = 1;
      } else {
        L.src = L.A == kInUser ? kSrcCvtA : kSrcCvtB;
        L.gexp = 0;
      }
    }
  }

  // workspace layout
  size_t off = 0;
  for (int i = 0; i < kNumBufs; ++i) {
    if (!P.used[i]) { P.off[i] = 0; continue; }
    size_t per;
    if (i == kPartials) per = (size_t)P.nchunks * 4;
    else if (i == kGScale) per = 8;  // r (fp32), then e (int32) in a second [G] array
    else per = (size_t)P.rows[i] * P.ld[i] * dtype_size(P.cdtype);
    P.off[i] = off;
    off = align_up(off + per * (size_t)G, NSG_WORKSPACE_ALIGN);
  }
  P.total = off;
  (void)out_dtype;
  return NSG_OK;
}

int64_t elem_stride(const Plan &P, int id) {
  if (id == kPartials) return P.nchunks;
  if (id == kGScale) return 1;
  return P.rows[id] * P.ld[id];
}

// ---- optional launch timing (process-global) ----
struct TimingRec {
  int kind;
  hipEvent_t start, stop;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// ---- fixed scratch for the entry point that allocates nothing ----
// The workspace of ns_orthogonalize_noalloc: one array per GPU, held by the
// library from its first use on that GPU until the process ends.  Host code
// never passes `scratch` itself (in host code the name is a host-side
// stand-in, not a device address): it uses the address hipGetSymbolAddress
// returns for the current device, looked up once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace
}  // namespace nsg

static __device__ __align__(256) unsigned char scratch[NSG_NOALLOC_MAX_BYTES];

namespace nsg {
namespace {

// Device address of this device's scratch array (the device current on the
// calling thread), looked up on the first call per device.
nsg_status_t scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NSG_ERR_HIP;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return NSG_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NSG_OK;
}

}  // namespace
}  // namespace nsg

using namespace nsg;

extern "C" {

void ns_default_params(nsg_params_t *p) {
  if (p == nullptr) return;
  p->steps = 5;
  p->coeffs = kMuon;
  p->n_coeffs = 3;
  p->mode = NSG_GRAM;
  p->restart_after = 2;
  p->safety = 1.05f;
  p->eps = 1e-7f;
  p->compute_dtype = NSG_F16;
  p->sym_updates = 1;
  p->restart_mask = 0;
}

const char *ns_status_string(nsg_status_t s) {
  // a C caller may pass any int: read it as one (an out-of-range value held in
  // the enum type would be undefined in C++)
  int v = 0;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case NSG_OK: return "ok";
    case NSG_ERR_INVALID_ARG: return "invalid argument";
    case NSG_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case NSG_ERR_SHAPE: return "unsupported shape";
    case NSG_ERR_WORKSPACE_TOO_SMALL: return "workspace missing, misaligned or too small";
    case NSG_ERR_HIP: return "HIP runtime error";
    case NSG_ERR_SCRATCH_TOO_SMALL: return "bucket needs more than the fixed no-allocation scratch";
  }
  return "unknown status";
}

nsg_status_t ns_workspace_size(int64_t G, int64_t R, int64_t C, const nsg_params_t *p, size_t *bytes) {
  if (bytes == nullptr) return NSG_ERR_INVALID_ARG;
  nsg_status_t st = validate_params(p);
  if (st != NSG_OK) return st;
  st = validate_shape(G, R, C);
  if (st != NSG_OK) return st;
  if (G == 0 || R == 0 || C == 0) {
    *bytes = 0;
    return NSG_OK;
  }
  Plan P;
  st = build_plan(R, C, p, G, NSG_F16, p->compute_dtype, true, P);
  if (st != NSG_OK) return st;
  *bytes = P.total;
  return NSG_OK;
}

nsg_status_t ns_flops(int64_t R, int64_t C, const nsg_params_t *p, double *credited, double *executed) {
  nsg_status_t st = validate_params(p);
  if (st != NSG_OK) return st;
  st = validate_shape(1, R, C);
  if (st != NSG_OK) return st;
  if (R == 0 || C == 0) {
    if (credited) *credited = 0.0;
    if (executed) *executed = 0.0;
    return NSG_OK;
  }
  Plan P;
  st = build_plan(R, C, p, 1, NSG_F16, p->compute_dtype, true, P);
  if (st != NSG_OK) return st;
  const double n = (double)P.n, m = (double)P.m, T = (double)P.T;
  double cr;
  if (!P.gram) {
    cr = 2.0 * T * (2.0 * m * n * n + n * n * n);  // 2T(2 alpha + 1) n^3
  } else {
    cr = 4.0 * T * n * n * n + 3.0 * m * n * n - 3.0 * n * n * n;  // (4T + 3 alpha - 3) n^3
    int nr = 0;
    for (int t = 2; t <= P.T; ++t) nr += P.restart_at(t) ? 1 : 0;
    cr += 3.0 * nr * (m * n * n - n * n * n);  // + 3(alpha - 1) n^3 per restart
  }
  double ex = 0.0;
  for (const Launch &L : P.launches) ex += L.flops;
  if (credited) *credited = cr;
  if (executed) *executed = ex;
  return NSG_OK;
}

nsg_status_t ns_plan(int64_t R, int64_t C, int32_t in_dtype, const nsg_params_t *p, nsg_launch_info_t *entries,
                     int32_t max_entries, int32_t *count) {
  if (count == nullptr || max_entries < 0 || (max_entries > 0 && entries == nullptr)) return NSG_ERR_INVALID_ARG;
  nsg_status_t st = validate_params(p);
  if (st != NSG_OK) return st;
  if (!valid_dtype(in_dtype)) return NSG_ERR_UNSUPPORTED_DTYPE;
  st = validate_shape(1, R, C);
  if (st != NSG_OK) return st;
  if (R == 0 || C == 0) {
    *count = 0;
    return NSG_OK;
  }
  Plan P;
  st = build_plan(R, C, p, 1, NSG_F16, in_dtype, true, P);
  if (st != NSG_OK) return st;
  *count = (int32_t)P.launches.size();
  for (int i = 0; i < (int)P.launches.size() && i < max_entries; ++i) {
    const Launch &L = P.launches[i];
    nsg_launch_info_t &e = entries[i];
    e.kind = L.kind;
    e.step = L.step;
    e.M = L.Mv; e.N = L.Nv;
    e.K = (L.kind >= 2) ? ((L.K == P.mp) ? P.m : P.n) : 0;
    e.flops = L.flops;
    e.bytes = L.bytes;
    std::memset(e.label, 0, sizeof(e.label));
    std::strncpy(e.label, L.label.c_str(), sizeof(e.label) - 1);
    e.a_kmajor = L.at;
    e.b_kmajor = L.bt;
    e.source = L.src;
  }
  return NSG_OK;
}

nsg_status_t ns_orthogonalize(const void *in, int32_t in_dtype, void *out, int32_t out_dtype, int64_t G,
                              int64_t R, int64_t C, const nsg_params_t *p, void *workspace,
                              size_t workspace_bytes, int32_t *status, void *stream) {
  nsg_status_t st = validate_params(p);
  if (st != NSG_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return NSG_ERR_UNSUPPORTED_DTYPE;
  st = validate_shape(G, R, C);
  if (st != NSG_OK) return st;
  if (G == 0 || R == 0 || C == 0) return NSG_OK;
  if (in == nullptr || out == nullptr) return NSG_ERR_INVALID_ARG;
  Plan P;
  // the input is read in place only if it is 16-byte aligned and the output
  // does not overlap it (out == in is allowed and then takes the copy)
  const uintptr_t i0 = reinterpret_cast<uintptr_t>(in), o0 = reinterpret_cast<uintptr_t>(out);
  const uintptr_t i1 = i0 + (uintptr_t)(G * R * C) * dtype_size(in_dtype);
  const uintptr_t o1 = o0 + (uintptr_t)(G * R * C) * dtype_size(out_dtype);
  const bool in_place_ok = i0 % 16 == 0 && (o1 <= i0 || i1 <= o0);
  st = build_plan(R, C, p, G, out_dtype, in_dtype, in_place_ok, P);
  if (st != NSG_OK) return st;
  if (workspace == nullptr || workspace_bytes < P.total ||
      (reinterpret_cast<uintptr_t>(workspace) % NSG_WORKSPACE_ALIGN) != 0)
    return NSG_ERR_WORKSPACE_TOO_SMALL;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char *ws = reinterpret_cast<char *>(workspace);
  auto ptr = [&](int id) -> void * { return id >= 0 ? ws + P.off[id] : nullptr; };
  // operand addresses, row pitches and matrix strides; the input in place is
  // [G][R][C], dense
  auto src = [&](int id) -> const void * { return id == kInUser ? in : ptr(id); };
  auto ld_of = [&](int id) -> int64_t { return id == kInUser ? C : P.ld[id]; };
  auto stride_of = [&](int id) -> int64_t { return id == kInUser ? R * C : elem_stride(P, id); };
  const size_t es = dtype_size(P.cdtype);
  (void)es;

  std::unique_lock<std::mutex> lk(g_tmu, std::defer_lock);
  bool timing = false;
  {
    std::lock_guard<std::mutex> g(g_tmu);
    timing = g_timing;
  }

  for (const Launch &L : P.launches) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (timing) {
      std::lock_guard<std::mutex> g(g_tmu);
      e0 = take_event();
      e1 = take_event();
      if (e0 && hipEventRecord(e0, s) != hipSuccess) return NSG_ERR_HIP;
    }
    hipError_t err = hipSuccess;
    if (L.kind == 0) {
      NormReduceArgs a;
      a.in = in; a.in_dtype = in_dtype; a.elems = R * C; a.nchunks = P.nchunks;
      a.partials = reinterpret_cast<float *>(ptr(kPartials));
      a.batch = (int32_t)G;
      err = launch_norm_reduce(a, s);
    } else if (L.kind == 1) {
      ScaleArgs a;
      a.in = in; a.in_dtype = in_dtype; a.R = R; a.C = C;
      a.partials = reinterpret_cast<const float *>(ptr(kPartials));
      a.nchunks = P.nchunks;
      a.safety = p->safety; a.eps = p->eps; a.fexp = P.fexp;
      a.tr = P.tr ? 1 : 0;
      a.rows_p = (int32_t)(P.tr ? P.mp : P.np);
      a.cols_p = (int32_t)(P.tr ? P.np : P.mp);
      // reading the input in place: no copy, or (bf16 under fp16) the bf16
      // copy of the matrices the raw product cannot take
      a.same = P.direct ? nullptr : (P.tr ? ptr(kX0T) : ptr(kX0));
      a.raw_fallback = P.cvt ? 1 : 0;
      a.swap = P.single ? nullptr : (P.tr ? ptr(kX0) : ptr(kX0T));
      a.ld_same = P.tr ? P.ld[kX0T] : P.ld[kX0];
      a.s_same = elem_stride(P, P.tr ? kX0T : kX0);
      if (!P.single) {
        a.ld_swap = P.tr ? P.ld[kX0] : P.ld[kX0T];
        a.s_swap = elem_stride(P, P.tr ? kX0 : kX0T);
      }
      a.cdtype = P.cvt ? NSG_BF16 : P.cdtype;
      a.gscale = reinterpret_cast<float *>(ptr(kGScale));
      a.status = status;
      a.batch = (int32_t)G;
      err = launch_scale(a, s);
    } else {
      GemmArgs a;
      a.A = src(L.A); a.lda = ld_of(L.A); a.sA = stride_of(L.A);
      a.B = src(L.B); a.ldb = ld_of(L.B); a.sB = stride_of(L.B);
      a.a_trans = L.at; a.b_trans = L.bt;
      if (L.Cin != kNone) { a.Cin = src(L.Cin); a.ldc = ld_of(L.Cin); a.sC = stride_of(L.Cin); }
      if (L.out0 == kOutUser) {
        a.out0 = out;
        a.ld0 = C;  // the caller's [R, C] layout; final launches produce exactly that
        a.s0 = R * C;
        a.out0_dtype = out_dtype;
        a.out0_pad = 0;
        a.status = status;
      } else if (L.out0 >= 0) {
        a.out0 = ptr(L.out0); a.ld0 = P.ld[L.out0]; a.s0 = elem_stride(P, L.out0);
        a.out0_dtype = P.cdtype; a.out0_pad = 1;
      }
      if (L.out1 >= 0) { a.out1 = ptr(L.out1); a.ld1 = P.ld[L.out1]; a.s1 = elem_stride(P, L.out1); }
      if (L.out2 >= 0) { a.out2 = ptr(L.out2); a.ld2 = P.ld[L.out2]; a.s2 = elem_stride(P, L.out2); }
      a.diag = L.diag;
      a.M = L.M; a.N = L.N; a.K = L.K; a.Mv = L.Mv; a.Nv = L.Nv;
      a.alpha = L.alpha; a.beta = L.beta;
      a.gscale = reinterpret_cast<const float *>(ptr(kGScale));
      a.gpow = L.gpow;
      a.gexp = L.gexp;
      a.src = L.src;
      if (L.src == kSrcRaw) {  // matrices outside raw_exponent_ok: the scale pass's bf16 copy
        const int fb = P.tr ? kX0T : kX0;
        a.fb = ptr(fb); a.ldfb = P.ld[fb]; a.sfb = elem_stride(P, fb);
      }
      a.batch = (int32_t)G;
      err = launch_gemm(L.src == kSrcRaw ? NSG_BF16 : P.cdtype, L.kind == 3, P.cfg, a, s);
    }
    if (err != hipSuccess) return NSG_ERR_HIP;
    if (timing) {
      std::lock_guard<std::mutex> g(g_tmu);
      if (e1 && hipEventRecord(e1, s) != hipSuccess) return NSG_ERR_HIP;
      if (e0 && e1) g_recs.push_back({L.kind, e0, e1});
    }
  }
  return NSG_OK;
}

nsg_status_t ns_orthogonalize_noalloc(const void *in, int32_t in_dtype, void *out, int32_t out_dtype, int64_t G,
                                      int64_t R, int64_t C, const nsg_params_t *p, int32_t *status, void *stream) {
  size_t need = 0;
  nsg_status_t st = ns_workspace_size(G, R, C, p, &need);
  if (st != NSG_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return NSG_ERR_UNSUPPORTED_DTYPE;
  if (G == 0 || R == 0 || C == 0) return NSG_OK;
  if (in == nullptr || out == nullptr) return NSG_ERR_INVALID_ARG;
  if (need > (size_t)NSG_NOALLOC_MAX_BYTES) return NSG_ERR_SCRATCH_TOO_SMALL;
  void *ws = nullptr;
  st = scratch_address(&ws);
  if (st != NSG_OK) return st;
  // Every buffer the kernels read from the workspace is written first in
  // the same call (partial sums, scales, X0 with its zero padding, every
  // product with its padding), so the previous call's contents never matter.
  return ns_orthogonalize(in, in_dtype, out, out_dtype, G, R, C, p, ws, (size_t)NSG_NOALLOC_MAX_BYTES, status,
                          stream);
}

nsg_status_t ns_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> g(g_tmu);
  g_timing = on != 0;
  for (auto &r : g_recs) {
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_recs.clear();
  return NSG_OK;
}

nsg_status_t ns_timing_collect(int32_t *kinds, float *ms, int32_t max_entries, int32_t *count) {
  if (count == nullptr || max_entries < 0) return NSG_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(g_tmu);
  nsg_status_t st = NSG_OK;
  int i = 0;
  for (auto &r : g_recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) st = NSG_ERR_HIP;
    float t = 0.f;
    if (st == NSG_OK && hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) st = NSG_ERR_HIP;
    if (i < max_entries) {
      if (kinds) kinds[i] = r.kind;
      if (ms) ms[i] = t;
    }
    ++i;
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  *count = i;
  g_recs.clear();
  return st;
}

nsg_status_t nsg_copy(const void *src, void *dst, size_t bytes, void *stream) {
  if (bytes == 0) return NSG_OK;
  if (src == nullptr || dst == nullptr || bytes % 16 != 0) return NSG_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0) return NSG_ERR_INVALID_ARG;
  return launch_copy(src, dst, bytes, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? NSG_OK : NSG_ERR_HIP;
}

nsg_status_t nsg_gemm_nt(int32_t dtype, int32_t symmetric, int64_t batch, int64_t M, int64_t N, int64_t K,
                         const void *A, int64_t lda, int32_t a_trans, const void *B, int64_t ldb, int32_t b_trans,
                         float alpha, float beta, const void *Cin, int64_t ldc, void *out, int64_t ldo, void *out_t,
                         int64_t ldt, void *out_d, float diag, int32_t tile, int32_t *status, void *stream) {
  if (!valid_dtype(dtype)) return NSG_ERR_UNSUPPORTED_DTYPE;
  if (tile != 0 && tile != 128 && tile != 256) return NSG_ERR_INVALID_ARG;
  if (batch < 0 || M < 0 || N < 0 || K < 0) return NSG_ERR_SHAPE;
  if (batch == 0 || M == 0 || N == 0) return NSG_OK;
  if (M % kPad || N % kPad || K % kPad || K == 0 || batch > 65535 || M > NSG_MAX_SIDE || N > NSG_MAX_SIDE ||
      K > NSG_MAX_SIDE)
    return NSG_ERR_SHAPE;
  if (A == nullptr || B == nullptr) return NSG_ERR_INVALID_ARG;
  if ((a_trans != 0 && a_trans != 1) || (b_trans != 0 && b_trans != 1)) return NSG_ERR_INVALID_ARG;
  // K-major operands: 16-bit 256 x 256 kernel; both (symmetric or general)
  // or B alone (general)
  if ((a_trans || b_trans) &&
      (dtype == NSG_F32 || tile == 128 || (a_trans && !b_trans) || (symmetric && a_trans != b_trans)))
    return NSG_ERR_INVALID_ARG;
  if (lda < (a_trans ? M : K) || ldb < (b_trans ? N : K)) return NSG_ERR_SHAPE;
  if (symmetric && (M != N || out_t != nullptr)) return NSG_ERR_INVALID_ARG;
  if (!symmetric && out_d != nullptr) return NSG_ERR_INVALID_ARG;
  if (Cin != nullptr && ldc < N) return NSG_ERR_SHAPE;
  if ((out != nullptr || out_d != nullptr) && ldo < N) return NSG_ERR_SHAPE;
  if (out_t != nullptr && ldt < M) return NSG_ERR_SHAPE;
  const size_t es = dtype_size(dtype);
  if ((lda * (int64_t)es) % 16 || (ldb * (int64_t)es) % 16) return NSG_ERR_SHAPE;
  GemmArgs a;
  a.A = A; a.lda = lda; a.sA = (a_trans ? K : M) * lda;
  a.B = B; a.ldb = ldb; a.sB = (b_trans ? K : N) * ldb;
  a.a_trans = a_trans; a.b_trans = b_trans;
  if (Cin) { a.Cin = Cin; a.ldc = ldc; a.sC = M * ldc; }
  a.out0 = out; a.ld0 = ldo; a.s0 = M * ldo; a.out0_dtype = dtype; a.out0_pad = 1;
  if (out_t) { a.out1 = out_t; a.ld1 = ldt; a.s1 = N * ldt; }
  if (out_d) { a.out2 = out_d; a.ld2 = ldo; a.s2 = M * ldo; a.diag = diag; }
  a.M = (int32_t)M; a.N = (int32_t)N; a.K = (int32_t)K; a.Mv = (int32_t)M; a.Nv = (int32_t)N;
  a.alpha = alpha; a.beta = beta;
  a.batch = (int32_t)batch;
  a.status = status;
  const int cfg = tile == 0 ? choose_cfg(M, N, dtype) : (tile == 256 ? kTile256 : kTile128);
  if ((a_trans || b_trans) && cfg != kTile256) return NSG_ERR_INVALID_ARG;
  return launch_gemm(dtype, symmetric != 0, cfg, a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? NSG_OK
             : NSG_ERR_HIP;
}


}  // extern "C"

// ---- selection front-end ------------------------------------------------------

namespace {

struct SelectLayout {
  int dim = 0;
  int64_t n = 0;              // lines to choose from
  int64_t sub_R = 0, sub_C = 0;  // gathered submatrix
  size_t keys = 0, part = 0, idx = 0, pos = 0, sub = 0, o = 0, inner = 0, total = 0;
};

nsg_status_t select_layout(int64_t G, int64_t R, int64_t C, int64_t k, int32_t dim, int32_t in_dtype,
                           int32_t out_dtype, const nsg_params_t *p, SelectLayout &L) {
  nsg_status_t st = validate_params(p);
  if (st != NSG_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return NSG_ERR_UNSUPPORTED_DTYPE;
  st = validate_shape(G, R, C);
  if (st != NSG_OK) return st;
  if (dim != NSG_SELECT_ROWS && dim != NSG_SELECT_COLS && dim != NSG_SELECT_SMALLER) return NSG_ERR_INVALID_ARG;
  L.dim = dim == NSG_SELECT_SMALLER ? (C < R ? 1 : 0) : dim;
  L.n = L.dim == 0 ? R : C;
  if (k < 0 || k > L.n || (k == 0 && L.n > 0)) return NSG_ERR_INVALID_ARG;
  L.sub_R = L.dim == 0 ? k : R;
  L.sub_C = L.dim == 0 ? C : k;
  size_t inner = 0;
  st = ns_workspace_size(G, L.sub_R, L.sub_C, p, &inner);
  if (st != NSG_OK) return st;
  const size_t A = NSG_WORKSPACE_ALIGN;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, A);
    return o;
  };
  const size_t g = (size_t)G;
  L.keys = take(8 * g * (size_t)L.n);
  L.part = take(L.dim == 1 ? 8 * g * (size_t)l1_cols_chunks(R) * (size_t)C : 0);
  L.idx = take(4 * g * (size_t)k);
  L.pos = take(4 * g * (size_t)L.n);
  L.sub = take(g * (size_t)L.sub_R * L.sub_C * dtype_size(in_dtype));
  L.o = take(g * (size_t)L.sub_R * L.sub_C * dtype_size(out_dtype));
  L.inner = take(inner);
  L.total = off;
  return NSG_OK;
}

}  // namespace

extern "C" {

nsg_status_t ns_select_count(int64_t R, int64_t C, int32_t dim, double fraction, int32_t *dim_out,
                             int64_t *k_out) {
  if (dim_out == nullptr || k_out == nullptr) return NSG_ERR_INVALID_ARG;
  if (R < 0 || C < 0 || R > NSG_MAX_SIDE || C > NSG_MAX_SIDE) return NSG_ERR_SHAPE;
  if (dim != NSG_SELECT_ROWS && dim != NSG_SELECT_COLS && dim != NSG_SELECT_SMALLER) return NSG_ERR_INVALID_ARG;
  if (!(fraction > 0.0 && fraction <= 1.0)) return NSG_ERR_INVALID_ARG;
  // without sharding the smaller dimension is selected; rows on a tie
  const int32_t d = dim == NSG_SELECT_SMALLER ? (C < R ? NSG_SELECT_COLS : NSG_SELECT_ROWS) : dim;
  const int64_t n = d == NSG_SELECT_ROWS ? R : C;
  int64_t k = 0;
  if (n > 0) {
    // k = ceil(f n), at least one line; the product is rounded up only when
    // it is not already an integer in double precision
    const double fk = std::ceil(fraction * (double)n);
    k = (int64_t)fk;
    if (k < 1) k = 1;
    if (k > n) k = n;
  }
  *dim_out = d;
  *k_out = k;
  return NSG_OK;
}

nsg_status_t ns_select_workspace_size(int64_t G, int64_t R, int64_t C, int64_t k, int32_t dim, int32_t in_dtype,
                                      int32_t out_dtype, const nsg_params_t *p, size_t *bytes) {
  if (bytes == nullptr) return NSG_ERR_INVALID_ARG;
  SelectLayout L;
  nsg_status_t st = select_layout(G, R, C, k, dim, in_dtype, out_dtype, p, L);
  if (st != NSG_OK) return st;
  *bytes = (G == 0 || R == 0 || C == 0) ? 0 : L.total;
  return NSG_OK;
}

nsg_status_t ns_orthogonalize_selected(const void *in, int32_t in_dtype, void *out, int32_t out_dtype, int64_t G,
                                       int64_t R, int64_t C, int64_t k, int32_t dim, const nsg_params_t *p,
                                       void *workspace, size_t workspace_bytes, int32_t *idx, int32_t *status,
                                       void *stream) {
  SelectLayout L;
  nsg_status_t st = select_layout(G, R, C, k, dim, in_dtype, out_dtype, p, L);
  if (st != NSG_OK) return st;
  if (G == 0 || R == 0 || C == 0) return NSG_OK;
  if (in == nullptr || out == nullptr) return NSG_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < L.total ||
      (reinterpret_cast<uintptr_t>(workspace) % NSG_WORKSPACE_ALIGN) != 0)
    return NSG_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char *ws = reinterpret_cast<char *>(workspace);
  double *keys = reinterpret_cast<double *>(ws + L.keys);
  double *part = reinterpret_cast<double *>(ws + L.part);
  int32_t *ix = idx != nullptr ? idx : reinterpret_cast<int32_t *>(ws + L.idx);
  int32_t *pos = reinterpret_cast<int32_t *>(ws + L.pos);
  void *sub = ws + L.sub, *O = ws + L.o;
  if (launch_l1_norms(in, in_dtype, G, R, C, L.dim, keys, part, s) != hipSuccess) return NSG_ERR_HIP;
  if (launch_topk(keys, G, L.n, k, ix, pos, s) != hipSuccess) return NSG_ERR_HIP;
  if (launch_gather(in, in_dtype, G, R, C, L.dim, ix, k, sub, s) != hipSuccess) return NSG_ERR_HIP;
  st = ns_orthogonalize(sub, in_dtype, O, out_dtype, G, L.sub_R, L.sub_C, p, ws + L.inner, workspace_bytes - L.inner,
                        status, stream);
  if (st != NSG_OK) return st;
  if (launch_scatter(O, out_dtype, G, R, C, L.dim, pos, k, out, s) != hipSuccess) return NSG_ERR_HIP;
  return NSG_OK;
}

nsg_status_t nsg_l1_workspace_size(int64_t G, int64_t R, int64_t C, int32_t dim, size_t *bytes) {
  if (bytes == nullptr) return NSG_ERR_INVALID_ARG;
  nsg_status_t st = validate_shape(G, R, C);
  if (st != NSG_OK) return st;
  if (dim != NSG_SELECT_ROWS && dim != NSG_SELECT_COLS) return NSG_ERR_INVALID_ARG;
  *bytes = dim == NSG_SELECT_COLS ? 8 * (size_t)G * (size_t)l1_cols_chunks(R) * (size_t)C : 0;
  return NSG_OK;
}

nsg_status_t nsg_l1_norms(const void *in, int32_t dtype, int64_t G, int64_t R, int64_t C, int32_t dim, double *keys,
                          void *workspace, size_t workspace_bytes, void *stream) {
  size_t need = 0;
  nsg_status_t st = nsg_l1_workspace_size(G, R, C, dim, &need);
  if (st != NSG_OK) return st;
  if (!valid_dtype(dtype)) return NSG_ERR_UNSUPPORTED_DTYPE;
  if (G == 0 || R == 0 || C == 0) return NSG_OK;
  if (in == nullptr || keys == nullptr) return NSG_ERR_INVALID_ARG;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return NSG_ERR_WORKSPACE_TOO_SMALL;
  return launch_l1_norms(in, dtype, G, R, C, dim, keys, reinterpret_cast<double *>(workspace),
                         reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? NSG_OK
             : NSG_ERR_HIP;
}

nsg_status_t nsg_topk(const double *keys, int64_t G, int64_t n, int64_t k, int32_t *idx, int32_t *pos, void *stream) {
  if (G < 0 || G > 65535 || n < 0 || n > NSG_MAX_SIDE || k < 0 || k > n) return NSG_ERR_INVALID_ARG;
  if (G == 0 || n == 0 || k == 0) return NSG_OK;
  if (keys == nullptr || idx == nullptr || pos == nullptr) return NSG_ERR_INVALID_ARG;
  return launch_topk(keys, G, n, k, idx, pos, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? NSG_OK
                                                                                                  : NSG_ERR_HIP;
}


// ---- Muon step ------------------------------------------------------------------

nsg_status_t ns_muon_momentum(void *M, int32_t m_dtype, const void *G, int32_t g_dtype, int64_t n, float mu,
                              void *stream) {
  if (m_dtype != NSG_F32 && m_dtype != NSG_BF16) return NSG_ERR_UNSUPPORTED_DTYPE;
  if (!valid_dtype(g_dtype)) return NSG_ERR_UNSUPPORTED_DTYPE;
  if (n < 0 || !std::isfinite(mu)) return NSG_ERR_INVALID_ARG;
  if (n == 0) return NSG_OK;
  if (M == nullptr || G == nullptr) return NSG_ERR_INVALID_ARG;
  return launch_muon_momentum(M, m_dtype, G, g_dtype, n, mu, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? NSG_OK
             : NSG_ERR_HIP;
}

nsg_status_t ns_muon_update(void *W, int32_t w_dtype, const void *O, int32_t o_dtype, int64_t n, double lr,
                            double weight_decay, double scale, int32_t stochastic, uint64_t seed, uint64_t step,
                            void *stream) {
  if (w_dtype != NSG_F32 && w_dtype != NSG_BF16) return NSG_ERR_UNSUPPORTED_DTYPE;
  if (!valid_dtype(o_dtype)) return NSG_ERR_UNSUPPORTED_DTYPE;
  if (n < 0 || !std::isfinite(lr) || !std::isfinite(weight_decay) || !std::isfinite(scale)) return NSG_ERR_INVALID_ARG;
  if (n == 0) return NSG_OK;
  if (W == nullptr || O == nullptr) return NSG_ERR_INVALID_ARG;
  const float c1 = (float)(1.0 - lr * weight_decay), c2 = (float)(lr * scale);
  return launch_muon_update(W, w_dtype, O, o_dtype, n, c1, c2, stochastic ? 1 : 0, seed, step,
                            reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? NSG_OK
             : NSG_ERR_HIP;
}

nsg_status_t ns_muon_workspace_size(int64_t G, int64_t R, int64_t C, const nsg_params_t *p, size_t *bytes) {
  if (bytes == nullptr) return NSG_ERR_INVALID_ARG;
  size_t inner = 0;
  nsg_status_t st = ns_workspace_size(G, R, C, p, &inner);
  if (st != NSG_OK) return st;
  *bytes = inner == 0 ? 0 : align_up((size_t)G * R * C * 4, NSG_WORKSPACE_ALIGN) + inner;
  return NSG_OK;
}

nsg_status_t ns_muon_step(void *W, int32_t w_dtype, void *M, int32_t m_dtype, const void *Gr, int32_t g_dtype,
                          int64_t G, int64_t R, int64_t C, float mu, double lr, double weight_decay, double scale,
                          int32_t stochastic, uint64_t seed, uint64_t step, const nsg_params_t *p, void *workspace,
                          size_t workspace_bytes, int32_t *status, void *stream) {
  size_t need = 0;
  nsg_status_t st = ns_muon_workspace_size(G, R, C, p, &need);
  if (st != NSG_OK) return st;
  if ((w_dtype != NSG_F32 && w_dtype != NSG_BF16) || (m_dtype != NSG_F32 && m_dtype != NSG_BF16) ||
      !valid_dtype(g_dtype))
    return NSG_ERR_UNSUPPORTED_DTYPE;
  if (G == 0 || R == 0 || C == 0) return NSG_OK;
  if (W == nullptr || M == nullptr || Gr == nullptr) return NSG_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < need ||
      (reinterpret_cast<uintptr_t>(workspace) % NSG_WORKSPACE_ALIGN) != 0)
    return NSG_ERR_WORKSPACE_TOO_SMALL;
  const int64_t n = G * R * C;
  st = ns_muon_momentum(M, m_dtype, Gr, g_dtype, n, mu, stream);
  if (st != NSG_OK) return st;
  char *ws = reinterpret_cast<char *>(workspace);
  const size_t o_bytes = align_up((size_t)n * 4, NSG_WORKSPACE_ALIGN);
  st = ns_orthogonalize(M, m_dtype, ws, NSG_F32, G, R, C, p, ws + o_bytes, workspace_bytes - o_bytes, status, stream);
  if (st != NSG_OK) return st;
  return ns_muon_update(W, w_dtype, ws, NSG_F32, n, lr, weight_decay, scale, stochastic, seed, step, stream);
}

}  // extern "C"
