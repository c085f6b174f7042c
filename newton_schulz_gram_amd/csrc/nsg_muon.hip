// The Muon step around the orthogonalization, on gfx950 (Dion3 paper,
// Section 2.1, Eq. (1); Algorithm 4, steps 8-9; the "muon" kernel card: scaled
// update with decoupled weight decay in one kernel, bf16 write-back rounded
// stochastically with counter-based random bits keyed by the element's global
// index).
//
//   momentum:  M <- mu M + G           t = mu * m ; m' = t + g          (fp32)
//   update:    W <- c1 W - c2 O        t1 = c1 * w ; t2 = c2 * o ; w' = t1 - t2
// Each operation is one fp32 operation rounded to nearest even; nothing is
// contracted into a fused multiply-add, so the results are reproducible bit for
// bit.  Both kernels are streaming passes (HBM-bound), 8 elements per thread.
//
// Stochastic rounding to bf16 of a finite fp32 value: add 16 random bits to its
// bit pattern and drop the low 16 bits.  Random bits: Philox-4x32 with 10
// rounds (Salmon, Moraes, Dror, Shaw, SC 2011), key = the 64-bit seed, counter
// = (i >> 3, step) for element i, which takes the 16-bit half i & 1 of output
// word (i & 7) >> 1.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "nsg_internal.h"

// Built with -ffp-contract=off (hipcc's default contraction ignores pragmas);
// the pragma states the same intent for other builds.
#pragma clang fp contract(off)

namespace nsg {

struct U4 {
  uint32_t x[4];
};

__device__ __forceinline__ U4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u, kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint64_t p0 = (uint64_t)kM0 * c0, p1 = (uint64_t)kM1 * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  U4 o;
  o.x[0] = c0; o.x[1] = c1; o.x[2] = c2; o.x[3] = c3;
  return o;
}

__device__ __forceinline__ uint16_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);  // NaN
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint16_t bf16_sr_bits(float f, uint32_t r16) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return bf16_rne_bits(f);  // inf, NaN
  return (uint16_t)((u + r16) >> 16);
}

template <typename T> __device__ __forceinline__ float to_f(T v) { return (float)v; }
template <> __device__ __forceinline__ float to_f<uint16_t>(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// 8 consecutive elements as floats: one vector load when VEC, else scalar loads
template <bool VEC, typename T>
__device__ __forceinline__ void load8(const T *p, int64_t base, int64_t n, float (&f)[8]) {
  if (VEC) {
    typedef T v8 __attribute__((ext_vector_type(8)));
    const v8 x = *reinterpret_cast<const v8 *>(p + base);
#pragma unroll
    for (int v = 0; v < 8; ++v) f[v] = to_f<T>(x[v]);
  } else {
#pragma unroll
    for (int v = 0; v < 8; ++v) f[v] = base + v < n ? to_f<T>(p[base + v]) : 0.f;
  }
}

// M <- mu M + G.  TM: float or uint16_t (bf16 bits, RNE); TG: float, _Float16 or uint16_t (bf16)
template <bool VEC, typename TM, typename TG>
__global__ void __launch_bounds__(256) muon_momentum_kernel(TM *__restrict__ M, const TG *__restrict__ G,
                                                            int64_t n, float mu) {
  const int64_t base = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (base >= n) return;
  float m[8], g[8];
  load8<VEC>(M, base, n, m);
  load8<VEC>(G, base, n, g);
  TM o[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const float t = __fmul_rn(mu, m[v]);
    const float r = __fadd_rn(t, g[v]);
    if constexpr (sizeof(TM) == 4) o[v] = r;
    else o[v] = bf16_rne_bits(r);
  }
  if (VEC) {
    typedef TM v8 __attribute__((ext_vector_type(8)));
    v8 w;
#pragma unroll
    for (int v = 0; v < 8; ++v) w[v] = o[v];
    *reinterpret_cast<v8 *>(M + base) = w;
  } else {
#pragma unroll
    for (int v = 0; v < 8; ++v)
      if (base + v < n) M[base + v] = o[v];
  }
}

// W <- c1 W - c2 O; TW: float or uint16_t (bf16 bits); TO: float, _Float16 or uint16_t
template <bool VEC, typename TW, typename TO>
__global__ void __launch_bounds__(256) muon_update_kernel(TW *__restrict__ W, const TO *__restrict__ O, int64_t n,
                                                          float c1, float c2, int stochastic, uint64_t seed,
                                                          uint64_t step) {
  const int64_t grp = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t base = grp * 8;
  if (base >= n) return;
  U4 rb = {};
  if (sizeof(TW) == 2 && stochastic)
    rb = philox10((uint32_t)grp, (uint32_t)((uint64_t)grp >> 32), (uint32_t)step, (uint32_t)(step >> 32),
                  (uint32_t)seed, (uint32_t)(seed >> 32));
  float w[8], o[8];
  load8<VEC>(W, base, n, w);
  load8<VEC>(O, base, n, o);
  TW r[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const float t1 = __fmul_rn(c1, w[v]);
    const float t2 = __fmul_rn(c2, o[v]);
    const float x = __fsub_rn(t1, t2);
    if constexpr (sizeof(TW) == 4) {
      r[v] = x;
    } else {
      r[v] = stochastic ? bf16_sr_bits(x, (rb.x[v >> 1] >> ((v & 1) * 16)) & 0xFFFFu) : bf16_rne_bits(x);
    }
  }
  if (VEC) {
    typedef TW v8 __attribute__((ext_vector_type(8)));
    v8 q;
#pragma unroll
    for (int v = 0; v < 8; ++v) q[v] = r[v];
    *reinterpret_cast<v8 *>(W + base) = q;
  } else {
#pragma unroll
    for (int v = 0; v < 8; ++v)
      if (base + v < n) W[base + v] = r[v];
  }
}

static bool vec_ok(const void *p, int dtype, int64_t n) {
  const size_t es = dtype == NSG_F32 ? 4 : 2;
  return n % 8 == 0 && reinterpret_cast<uintptr_t>(p) % (8 * es) == 0;
}

template <bool VEC, typename TM>
static hipError_t momentum_g(void *M, const void *G, int g_dtype, int64_t n, float mu, dim3 grid, hipStream_t s) {
  switch (g_dtype) {
    case NSG_F16:
      hipLaunchKernelGGL((muon_momentum_kernel<VEC, TM, _Float16>), grid, dim3(256), 0, s, (TM *)M, (const _Float16 *)G, n, mu);
      break;
    case NSG_BF16:
      hipLaunchKernelGGL((muon_momentum_kernel<VEC, TM, uint16_t>), grid, dim3(256), 0, s, (TM *)M, (const uint16_t *)G, n, mu);
      break;
    default:
      hipLaunchKernelGGL((muon_momentum_kernel<VEC, TM, float>), grid, dim3(256), 0, s, (TM *)M, (const float *)G, n, mu);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_muon_momentum(void *M, int m_dtype, const void *G, int g_dtype, int64_t n, float mu,
                                hipStream_t s) {
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 2047) / 2048));
  const bool vec = vec_ok(M, m_dtype, n) && vec_ok(G, g_dtype, n);
  if (m_dtype == NSG_BF16)
    return vec ? momentum_g<true, uint16_t>(M, G, g_dtype, n, mu, grid, s) : momentum_g<false, uint16_t>(M, G, g_dtype, n, mu, grid, s);
  return vec ? momentum_g<true, float>(M, G, g_dtype, n, mu, grid, s) : momentum_g<false, float>(M, G, g_dtype, n, mu, grid, s);
}

template <bool VEC, typename TW>
static hipError_t update_o(void *W, const void *O, int o_dtype, int64_t n, float c1, float c2, int stochastic,
                           uint64_t seed, uint64_t step, dim3 grid, hipStream_t s) {
  switch (o_dtype) {
    case NSG_F16:
      hipLaunchKernelGGL((muon_update_kernel<VEC, TW, _Float16>), grid, dim3(256), 0, s, (TW *)W, (const _Float16 *)O, n,
                         c1, c2, stochastic, seed, step);
      break;
    case NSG_BF16:
      hipLaunchKernelGGL((muon_update_kernel<VEC, TW, uint16_t>), grid, dim3(256), 0, s, (TW *)W, (const uint16_t *)O, n,
                         c1, c2, stochastic, seed, step);
      break;
    default:
      hipLaunchKernelGGL((muon_update_kernel<VEC, TW, float>), grid, dim3(256), 0, s, (TW *)W, (const float *)O, n, c1,
                         c2, stochastic, seed, step);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_muon_update(void *W, int w_dtype, const void *O, int o_dtype, int64_t n, float c1, float c2,
                              int stochastic, uint64_t seed, uint64_t step, hipStream_t s) {
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 2047) / 2048));
  const bool vec = vec_ok(W, w_dtype, n) && vec_ok(O, o_dtype, n);
  if (w_dtype == NSG_BF16)
    return vec ? update_o<true, uint16_t>(W, O, o_dtype, n, c1, c2, stochastic, seed, step, grid, s)
               : update_o<false, uint16_t>(W, O, o_dtype, n, c1, c2, stochastic, seed, step, grid, s);
  return vec ? update_o<true, float>(W, O, o_dtype, n, c1, c2, stochastic, seed, step, grid, s)
             : update_o<false, float>(W, O, o_dtype, n, c1, c2, stochastic, seed, step, grid, s);
}

}  // namespace nsg
