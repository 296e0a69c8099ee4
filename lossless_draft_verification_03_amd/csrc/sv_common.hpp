// Device-side building blocks shared by the libspecverify kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kBlock = 256;        // 4 waves per workgroup
constexpr float kLn2f = 0.693147180559945309f;
constexpr double kLn2 = 0.6931471805599453094;

enum : int { DT_F32 = 0, DT_BF16 = 1 };

// Raw buffer resource over [base, base + bytes): loads past `bytes` return 0
// instead of touching memory; every kernel still predicates its loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

typedef int v4i __attribute__((ext_vector_type(4)));

// Cache-policy bits of a buffer load: 2 marks the access non-temporal.
// Logits are read once per call, and on MI355X non-temporal 16-byte loads
// stream from HBM about 10% faster than default-policy ones.
constexpr int kStreamAux = 2;

__device__ __forceinline__ v4i load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamAux);
}

// bf16 bit patterns packed two per dword: element 0 in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DT>
__device__ __forceinline__ float load_elem(const void* base, long long e) {
  if constexpr (DT == DT_BF16) {
    const uint16_t h = reinterpret_cast<const uint16_t*>(base)[e];
    return __uint_as_float((uint32_t)h << 16);
  } else {
    return reinterpret_cast<const float*>(base)[e];
  }
}

// Unpack one 16-byte vector into EPV floats (8 bf16 or 4 fp32).
template <int DT>
__device__ __forceinline__ void unpack(const v4i& v, float* out) {
  if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      out[2 * q] = bf16_lo((uint32_t)v[q]);
      out[2 * q + 1] = bf16_hi((uint32_t)v[q]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = __int_as_float(v[q]);
  }
}

// ------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}
__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, kWave));
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, kWave));
  return x;
}
// Fixed butterfly: the result depends only on the lane values, never on timing.
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}
// Inclusive prefix sum over the 64 lanes (Hillis-Steele, fixed order).
__device__ __forceinline__ double wave_incl_scan(double x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  return x;
}

// ------------------------------------------------------------------ fp64 exp2
// 2^a to ~1 ulp: a = n + f with n = rint(a), |f| <= 1/2, then 2^f = e^(f ln 2)
// by its Taylor series through degree 13 (truncation below 2e-17 relative
// for |f ln 2| <= 0.347), scaled by 2^n.  Textbook range reduction.
__device__ __forceinline__ double exp2_f64(double a) {
  if (!(a > -1076.0)) return (a != a) ? a : 0.0;
  if (a >= 1024.0) return __builtin_huge_val();
  const double n = __builtin_rint(a);
  const double x = (a - n) * kLn2;
  double p = 1.0 / 6227020800.0;            // 1/13!
  p = fma(p, x, 1.0 / 479001600.0);         // 1/12!
  p = fma(p, x, 1.0 / 39916800.0);
  p = fma(p, x, 1.0 / 3628800.0);
  p = fma(p, x, 1.0 / 362880.0);
  p = fma(p, x, 1.0 / 40320.0);
  p = fma(p, x, 1.0 / 5040.0);
  p = fma(p, x, 1.0 / 720.0);
  p = fma(p, x, 1.0 / 120.0);
  p = fma(p, x, 1.0 / 24.0);
  p = fma(p, x, 1.0 / 6.0);
  p = fma(p, x, 0.5);
  p = fma(p, x, 1.0);
  p = fma(p, x, 1.0);
  return __builtin_ldexp(p, (int)n);
}

// ------------------------------------------------ temperature constants
// c = log2(e) / T split as c_hi + c_lo with c_lo > 0, so -inf logits map to
// exponent -inf without producing NaN; d_min clamps differences whose
// exponent underflows anyway.
struct TempConst {
  float c_hi;
  float c_lo;
  float d_min;
  float pad_;
  double c64;
};

// 2^((z - M) * c) in fp32 with the exponent carried as a double-float pair,
// so the only rounding left is that of the final exp2 and one fma.  Used by
// the final draw (and by the probe that reports what the draw sees).
template <int DT>
__device__ __forceinline__ float exp_rel(float z, float M, const TempConst& tc) {
  if constexpr (DT == DT_BF16) {
    // z and M are bf16 values, so z - M is exact in fp32.
    const float d = fmaxf(z - M, tc.d_min);
    const float ah = d * tc.c_hi;
    float al = fmaf(d, tc.c_hi, -ah);
    al = fmaf(d, tc.c_lo, al);
    const float e = __builtin_amdgcn_exp2f(ah);
    return fmaf(e, al * kLn2f, e);
  } else {
    // fp32 logits: form the exponent in fp64, where z - M is exact.
    double a = ((double)z - (double)M) * tc.c64;
    a = a > -200.0 ? a : -200.0;
    const float ah = (float)a;
    const float al = (float)(a - (double)ah);
    const float e = __builtin_amdgcn_exp2f(ah);
    return fmaf(e, al * kLn2f, e);
  }
}

// Sequence-level result of the accept scan, handed to the draw kernels.
struct DrawInfo {
  int j;        // accepted drafts (0..gamma), or -1 for an invalid draft token
  float Mt;     // max of target row j
  float Md;     // max of draft row j (j < gamma)
  float pad_;
  double rho;   // S_t / S_d of row j (j < gamma)
};

// Per-row statistics handed between kernels.
struct Partial {
  float m;      // max of the segment (or -inf)
  int arg;      // lowest row-local index holding m (INT_MAX if none)
  double s;     // sum of 2^((z - m) c) over the segment, exact reference m
};

}  // namespace sv
