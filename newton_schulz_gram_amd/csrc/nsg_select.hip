// Dion3 selection front-end on gfx950 (Dion3 paper, Section 6 "Selection";
// Algorithm 4, steps 3-4): l1 norms of the rows or columns of every matrix,
// the k largest per matrix, gather of the selected lines into a k x m bucket
// for the Gram Newton-Schulz path, and scatter of the result back.
//
// Every kernel here is HBM-bound (one pass over the input or the output) except
// the per-matrix top-k, which touches G x n keys.  Norms are fp64 sums in a
// fixed order, so the keys, and with them the selection, never depend on the
// bucket size or on other matrices.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "nsg_internal.h"

namespace nsg {

// |v| in fp64 (fabs also clears the sign of -0, so every key is >= +0)
template <typename TI> __device__ __forceinline__ double absd(TI v) { return __builtin_fabs((double)(float)v); }

// ---------------------------------------------------------------------------
// Row norms: one wave per row.  Lane l sums the 16-byte chunks l, l + 64, ...
// of the row (each chunk's elements in order), then the 64 lane sums are added
// by a fixed xor tree.  An unaligned row reads the same chunks element-wise,
// in the same order.
// ---------------------------------------------------------------------------
template <typename TI, bool VEC>
__global__ void __launch_bounds__(256) l1_rows_kernel(const TI *__restrict__ in, int64_t R, int64_t C,
                                                      double *__restrict__ keys) {
  constexpr int V = 16 / (int)sizeof(TI);
  typedef TI vec_t __attribute__((ext_vector_type(V)));
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int g = blockIdx.y;
  if (row >= R) return;
  const TI *src = in + ((size_t)g * R + row) * C;
  const int64_t nch = (C + V - 1) / V;
  double s = 0.0;
  for (int64_t ch = lane; ch < nch; ch += 64) {
    const int64_t e0 = ch * V;
    double cs = 0.0;
    if (VEC && e0 + V <= C) {
      const vec_t x = *reinterpret_cast<const vec_t *>(src + e0);
#pragma unroll
      for (int v = 0; v < V; ++v) cs += absd<TI>(x[v]);
    } else {
      for (int v = 0; v < V && e0 + v < C; ++v) cs += absd<TI>(src[e0 + v]);
    }
    s += cs;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) keys[(size_t)g * R + row] = s;
}

// ---------------------------------------------------------------------------
// Column norms: thread per column over a chunk of kColChunk rows (rows in
// order), partial sums per chunk; then the chunks of a column are added in
// chunk order.
// ---------------------------------------------------------------------------
constexpr int kColChunk = 512;

// Vector form: a thread owns 16 bytes of consecutive columns (same per-column
// order of rows, so the sums equal the scalar kernel's bit for bit).
template <typename TI>
__global__ void __launch_bounds__(256) l1_cols_partial_vec_kernel(const TI *__restrict__ in, int64_t R, int64_t C,
                                                                  int nchunks, double *__restrict__ part) {
  constexpr int V = 16 / (int)sizeof(TI);
  typedef TI vec_t __attribute__((ext_vector_type(V)));
  const int64_t col0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
  const int chunk = blockIdx.y, g = blockIdx.z;
  if (col0 >= C) return;
  const int64_t r0 = (int64_t)chunk * kColChunk;
  int64_t r1 = r0 + kColChunk;
  if (r1 > R) r1 = R;
  const TI *src = in + (size_t)g * R * C + col0;
  double s[V];
#pragma unroll
  for (int v = 0; v < V; ++v) s[v] = 0.0;
  for (int64_t r = r0; r < r1; ++r) {
    const vec_t x = *reinterpret_cast<const vec_t *>(src + (size_t)r * C);
#pragma unroll
    for (int v = 0; v < V; ++v) s[v] += absd<TI>(x[v]);
  }
  double *dst = part + ((size_t)g * nchunks + chunk) * C + col0;
#pragma unroll
  for (int v = 0; v < V; ++v) dst[v] = s[v];
}

template <typename TI>
__global__ void __launch_bounds__(256) l1_cols_partial_kernel(const TI *__restrict__ in, int64_t R, int64_t C,
                                                              int nchunks, double *__restrict__ part) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int chunk = blockIdx.y, g = blockIdx.z;
  if (col >= C) return;
  const int64_t r0 = (int64_t)chunk * kColChunk;
  int64_t r1 = r0 + kColChunk;
  if (r1 > R) r1 = R;
  const TI *src = in + (size_t)g * R * C + col;
  double s = 0.0;
  for (int64_t r = r0; r < r1; ++r) s += absd<TI>(src[(size_t)r * C]);
  part[((size_t)g * nchunks + chunk) * C + col] = s;
}

__global__ void __launch_bounds__(256) l1_cols_combine_kernel(const double *__restrict__ part, int64_t C,
                                                              int nchunks, double *__restrict__ keys) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int g = blockIdx.y;
  if (col >= C) return;
  double s = 0.0;
  for (int ch = 0; ch < nchunks; ++ch) s += part[((size_t)g * nchunks + ch) * C + col];
  keys[(size_t)g * C + col] = s;
}

// ---------------------------------------------------------------------------
// Top-k per matrix (one 1024-thread workgroup each): radix select on the key
// bits (non-negative doubles order like their bit patterns), 8 bits per pass
// from the top, gives the k-th largest key T and how many keys equal to T are
// taken (the ones with the lowest indices).  A block-wide scan in index order
// then writes the selected indices in ascending order, and pos[i] = rank of
// line i among the selected (-1 if not selected).
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;

__device__ __forceinline__ uint64_t key_bits(double d) { return (uint64_t)__double_as_longlong(d); }

// exclusive prefix sum of v over the block (in thread order) and the total
__device__ __forceinline__ int block_scan(int v, int *wsum, int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < kTopkThreads / 64; ++w) {
      const int t = wsum[w];
      wsum[w] = acc;
      acc += t;
    }
    wsum[kTopkThreads / 64] = acc;
  }
  __syncthreads();
  total = wsum[kTopkThreads / 64];
  return wsum[wave] + x - v;
}

__global__ void __launch_bounds__(kTopkThreads) topk_kernel(const double *__restrict__ keys, int64_t n, int64_t k,
                                                            int32_t *__restrict__ idx, int32_t *__restrict__ pos) {
  __shared__ int hist[256];
  __shared__ int wsum[kTopkThreads / 64 + 1];
  __shared__ uint64_t s_prefix;
  __shared__ int s_need;
  const int g = blockIdx.x;
  const double *kg = keys + (size_t)g * n;
  uint64_t prefix = 0;  // top bits of T fixed so far
  int need = (int)k;    // how many of the largest keys matching `prefix` are still to take
#pragma unroll 1
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    const uint64_t hi_mask = pass == 0 ? 0ull : (~0ull << (shift + 8));
    for (int b = threadIdx.x; b < 256; b += kTopkThreads) hist[b] = 0;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += kTopkThreads) {
      const uint64_t kb = key_bits(kg[i]);
      if ((kb & hi_mask) == prefix) atomicAdd(&hist[(kb >> shift) & 255], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int above = 0, b = 255;
      for (; b > 0; --b) {
        if (above + hist[b] >= need) break;
        above += hist[b];
      }
      s_prefix = prefix | ((uint64_t)b << shift);
      s_need = need - above;
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    __syncthreads();
  }
  // prefix == bits of T; `need` keys equal to T are taken, lowest indices first
  const uint64_t T = prefix;
  int taken_eq = 0, written = 0;
  int32_t *ig = idx + (size_t)g * k;
  int32_t *pg = pos + (size_t)g * n;
#pragma unroll 1
  for (int64_t base = 0; base < n; base += kTopkThreads) {
    const int64_t i = base + threadIdx.x;
    uint64_t kb = 0;
    if (i < n) kb = key_bits(kg[i]);
    const int eq = (i < n && kb == T) ? 1 : 0;
    int eq_total;
    const int eq_rank = taken_eq + block_scan(eq, wsum, eq_total);
    const int sel = (i < n && (kb > T || (eq && eq_rank < need))) ? 1 : 0;
    int sel_total;
    const int p = written + block_scan(sel, wsum, sel_total);
    if (i < n) {
      pg[i] = sel ? p : -1;
      if (sel && p < k) ig[p] = (int32_t)i;
    }
    taken_eq += eq_total;
    written += sel_total;
  }
}

// ---------------------------------------------------------------------------
// Gather and scatter.  Row mode: whole rows, 16-byte copies when aligned.
// Column mode: element-wise along each row (selected columns ascending).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) gather_rows_kernel(const T *__restrict__ in, int64_t R, int64_t C,
                                                          const int32_t *__restrict__ idx, int64_t k,
                                                          T *__restrict__ out) {
  const int64_t j = blockIdx.x;
  const int g = blockIdx.y;
  const T *src = in + ((size_t)g * R + idx[(size_t)g * k + j]) * C;
  T *dst = out + ((size_t)g * k + j) * C;
  for (int64_t c = threadIdx.x; c < C; c += 256) dst[c] = src[c];
}

template <typename T>
__global__ void __launch_bounds__(256) gather_cols_kernel(const T *__restrict__ in, int64_t R, int64_t C,
                                                          const int32_t *__restrict__ idx, int64_t k,
                                                          T *__restrict__ out) {
  const int64_t j = (int64_t)blockIdx.y * 256 + threadIdx.x;
  const int64_t r = blockIdx.x;
  const int g = blockIdx.z;
  if (j >= k) return;
  out[((size_t)g * R + r) * k + j] = in[((size_t)g * R + r) * C + idx[(size_t)g * k + j]];
}

template <typename T>
__global__ void __launch_bounds__(256) scatter_rows_kernel(const T *__restrict__ O, int64_t R, int64_t C,
                                                           const int32_t *__restrict__ pos, int64_t k,
                                                           T *__restrict__ out) {
  const int64_t r = blockIdx.x;
  const int g = blockIdx.y;
  const int p = pos[(size_t)g * R + r];
  T *dst = out + ((size_t)g * R + r) * C;
  if (p < 0) {
    for (int64_t c = threadIdx.x; c < C; c += 256) dst[c] = (T)0.f;
  } else {
    const T *src = O + ((size_t)g * k + p) * C;
    for (int64_t c = threadIdx.x; c < C; c += 256) dst[c] = src[c];
  }
}

template <typename T>
__global__ void __launch_bounds__(256) scatter_cols_vec_kernel(const T *__restrict__ O, int64_t R, int64_t C,
                                                               const int32_t *__restrict__ pos, int64_t k,
                                                               T *__restrict__ out) {
  constexpr int V = 16 / (int)sizeof(T);
  typedef T vec_t __attribute__((ext_vector_type(V)));
  const int64_t c0 = ((int64_t)blockIdx.y * 256 + threadIdx.x) * V;
  const int64_t r = blockIdx.x;
  const int g = blockIdx.z;
  if (c0 >= C) return;
  const int32_t *pg = pos + (size_t)g * C + c0;
  const T *orow = O + ((size_t)g * R + r) * k;
  vec_t w;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int p = pg[v];
    w[v] = p < 0 ? (T)0.f : orow[p];
  }
  *reinterpret_cast<vec_t *>(out + ((size_t)g * R + r) * C + c0) = w;
}

template <typename T>
__global__ void __launch_bounds__(256) scatter_cols_kernel(const T *__restrict__ O, int64_t R, int64_t C,
                                                           const int32_t *__restrict__ pos, int64_t k,
                                                           T *__restrict__ out) {
  const int64_t c = (int64_t)blockIdx.y * 256 + threadIdx.x;
  const int64_t r = blockIdx.x;
  const int g = blockIdx.z;
  if (c >= C) return;
  const int p = pos[(size_t)g * C + c];
  out[((size_t)g * R + r) * C + c] = p < 0 ? (T)0.f : O[((size_t)g * R + r) * k + p];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int64_t l1_cols_chunks(int64_t R) { return (R + kColChunk - 1) / kColChunk; }

hipError_t launch_l1_norms(const void *in, int dtype, int64_t G, int64_t R, int64_t C, int dim, double *keys,
                           double *part, hipStream_t s) {
  if (G == 0 || R == 0 || C == 0) return hipSuccess;
  if (dim == 0) {
    dim3 grid((unsigned)((R + 3) / 4), (unsigned)G);
    const size_t es = dtype == NSG_F32 ? 4 : 2;
    const bool vec = (reinterpret_cast<uintptr_t>(in) % 16 == 0) && ((size_t)C * es) % 16 == 0;
#define NSG_L1R(TI)                                                                                          \
  if (vec) hipLaunchKernelGGL((l1_rows_kernel<TI, true>), grid, dim3(256), 0, s, (const TI *)in, R, C, keys); \
  else hipLaunchKernelGGL((l1_rows_kernel<TI, false>), grid, dim3(256), 0, s, (const TI *)in, R, C, keys)
    switch (dtype) {
      case NSG_F16: NSG_L1R(_Float16); break;
      case NSG_BF16: NSG_L1R(__bf16); break;
      default: NSG_L1R(float); break;
    }
#undef NSG_L1R
  } else {
    const int nch = (int)l1_cols_chunks(R);
    const size_t es = dtype == NSG_F32 ? 4 : 2;
    const int64_t V = 16 / (int64_t)es;
    const bool vec = (reinterpret_cast<uintptr_t>(in) % 16 == 0) && (C % V) == 0;
    dim3 grid((unsigned)((C + 255) / 256), (unsigned)nch, (unsigned)G);
    dim3 gridv((unsigned)((C / V + 255) / 256), (unsigned)nch, (unsigned)G);
#define NSG_L1C(TI)                                                                                              \
  if (vec) hipLaunchKernelGGL(l1_cols_partial_vec_kernel<TI>, gridv, dim3(256), 0, s, (const TI *)in, R, C, nch, part); \
  else hipLaunchKernelGGL(l1_cols_partial_kernel<TI>, grid, dim3(256), 0, s, (const TI *)in, R, C, nch, part)
    switch (dtype) {
      case NSG_F16: NSG_L1C(_Float16); break;
      case NSG_BF16: NSG_L1C(__bf16); break;
      default: NSG_L1C(float); break;
    }
#undef NSG_L1C
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(l1_cols_combine_kernel, dim3((unsigned)((C + 255) / 256), (unsigned)G), dim3(256), 0, s,
                       (const double *)part, C, nch, keys);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const double *keys, int64_t G, int64_t n, int64_t k, int32_t *idx, int32_t *pos,
                       hipStream_t s) {
  if (G == 0 || n == 0 || k == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)G), dim3(kTopkThreads), 0, s, keys, n, k, idx, pos);
  return hipGetLastError();
}

template <typename T>
static hipError_t gather_t(const void *in, int64_t G, int64_t R, int64_t C, int dim, const int32_t *idx, int64_t k,
                           void *out, hipStream_t s) {
  if (dim == 0)
    hipLaunchKernelGGL(gather_rows_kernel<T>, dim3((unsigned)k, (unsigned)G), dim3(256), 0, s, (const T *)in, R, C,
                       idx, k, (T *)out);
  else
    hipLaunchKernelGGL(gather_cols_kernel<T>, dim3((unsigned)R, (unsigned)((k + 255) / 256), (unsigned)G), dim3(256),
                       0, s, (const T *)in, R, C, idx, k, (T *)out);
  return hipGetLastError();
}

template <typename T>
static hipError_t scatter_t(const void *O, int64_t G, int64_t R, int64_t C, int dim, const int32_t *pos, int64_t k,
                            void *out, hipStream_t s) {
  if (dim == 0)
    hipLaunchKernelGGL(scatter_rows_kernel<T>, dim3((unsigned)R, (unsigned)G), dim3(256), 0, s, (const T *)O, R, C,
                       pos, k, (T *)out);
  else {
    constexpr int64_t V = 16 / (int64_t)sizeof(T);
    if ((reinterpret_cast<uintptr_t>(out) % 16 == 0) && (C % V) == 0)
      hipLaunchKernelGGL(scatter_cols_vec_kernel<T>, dim3((unsigned)R, (unsigned)((C / V + 255) / 256), (unsigned)G),
                         dim3(256), 0, s, (const T *)O, R, C, pos, k, (T *)out);
    else
      hipLaunchKernelGGL(scatter_cols_kernel<T>, dim3((unsigned)R, (unsigned)((C + 255) / 256), (unsigned)G),
                         dim3(256), 0, s, (const T *)O, R, C, pos, k, (T *)out);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const void *in, int dtype, int64_t G, int64_t R, int64_t C, int dim, const int32_t *idx,
                         int64_t k, void *out, hipStream_t s) {
  if (G == 0 || R == 0 || C == 0 || k == 0) return hipSuccess;
  switch (dtype) {
    case NSG_F16: return gather_t<_Float16>(in, G, R, C, dim, idx, k, out, s);
    case NSG_BF16: return gather_t<__bf16>(in, G, R, C, dim, idx, k, out, s);
    default: return gather_t<float>(in, G, R, C, dim, idx, k, out, s);
  }
}

hipError_t launch_scatter(const void *O, int dtype, int64_t G, int64_t R, int64_t C, int dim, const int32_t *pos,
                          int64_t k, void *out, hipStream_t s) {
  if (G == 0 || R == 0 || C == 0) return hipSuccess;
  switch (dtype) {
    case NSG_F16: return scatter_t<_Float16>(O, G, R, C, dim, pos, k, out, s);
    case NSG_BF16: return scatter_t<__bf16>(O, G, R, C, dim, pos, k, out, s);
    default: return scatter_t<float>(O, G, R, C, dim, pos, k, out, s);
  }
}

}  // namespace nsg
