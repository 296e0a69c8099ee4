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
// Within each 16-lane row: DPP quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror and row_mirror pair every lane with partners that cover
// the row, so after four steps all 16 lanes hold the same row value (each
// step combines a and b as op(a, b) with a commutative op, so partners get
// bitwise-equal results).  The four row values are then read with readlane
// and combined in a fixed order; the result is wave-uniform.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const int lo = dpp_i<CTRL>(__double2loint(x));
  const int hi = dpp_i<CTRL>(__double2hiint(x));
  return __hiloint2double(hi, lo);
}
constexpr int kDppXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ double readlane_d(double x, int l) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), l);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), l);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kDppXor1>(x));
  x = fmaxf(x, dpp_f<kDppXor2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_f<kDppMirror>(x));
  return fmaxf(fmaxf(readlane_f(x, 0), readlane_f(x, 16)), fmaxf(readlane_f(x, 32), readlane_f(x, 48)));
}
__device__ __forceinline__ int wave_min(int x) {
  x = min(x, dpp_i<kDppXor1>(x));
  x = min(x, dpp_i<kDppXor2>(x));
  x = min(x, dpp_i<kDppHalfMirror>(x));
  x = min(x, dpp_i<kDppMirror>(x));
  return min(min(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             min(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
__device__ __forceinline__ int wave_max_i(int x) {
  x = max(x, dpp_i<kDppXor1>(x));
  x = max(x, dpp_i<kDppXor2>(x));
  x = max(x, dpp_i<kDppHalfMirror>(x));
  x = max(x, dpp_i<kDppMirror>(x));
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
// Fixed combination order: the result depends only on the lane values.
__device__ __forceinline__ double wave_sum(double x) {
  x += dpp_d<kDppXor1>(x);
  x += dpp_d<kDppXor2>(x);
  x += dpp_d<kDppHalfMirror>(x);
  x += dpp_d<kDppMirror>(x);
  return (readlane_d(x, 0) + readlane_d(x, 16)) + (readlane_d(x, 32) + readlane_d(x, 48));
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

// Reductions inside aligned groups of G lanes (G a power of two <= 64); every
// lane of a group gets the group's value.
template <int G>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (G >= 2) x = fmaxf(x, dpp_f<kDppXor1>(x));
  if constexpr (G >= 4) x = fmaxf(x, dpp_f<kDppXor2>(x));
  if constexpr (G >= 8) x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  if constexpr (G >= 16) x = fmaxf(x, dpp_f<kDppMirror>(x));
  if constexpr (G >= 32) x = fmaxf(x, __shfl_xor(x, 16, kWave));
  if constexpr (G >= 64) x = fmaxf(x, __shfl_xor(x, 32, kWave));
  return x;
}
template <int G>
__device__ __forceinline__ int group_min(int x) {
  if constexpr (G >= 2) x = min(x, dpp_i<kDppXor1>(x));
  if constexpr (G >= 4) x = min(x, dpp_i<kDppXor2>(x));
  if constexpr (G >= 8) x = min(x, dpp_i<kDppHalfMirror>(x));
  if constexpr (G >= 16) x = min(x, dpp_i<kDppMirror>(x));
  if constexpr (G >= 32) x = min(x, __shfl_xor(x, 16, kWave));
  if constexpr (G >= 64) x = min(x, __shfl_xor(x, 32, kWave));
  return x;
}
template <int G>
__device__ __forceinline__ double group_sum(double x) {
  if constexpr (G >= 2) x += dpp_d<kDppXor1>(x);
  if constexpr (G >= 4) x += dpp_d<kDppXor2>(x);
  if constexpr (G >= 8) x += dpp_d<kDppHalfMirror>(x);
  if constexpr (G >= 16) x += dpp_d<kDppMirror>(x);
  if constexpr (G >= 32) x += __shfl_xor(x, 16, kWave);
  if constexpr (G >= 64) x += __shfl_xor(x, 32, kWave);
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

// The same exponential as exp_rel, returned in fp64: the head 2^ah from the
// hardware exp2 and the tail factor (1 + al ln 2) applied in fp64, so neither
// the tail nor a later difference of two such values is rounded to fp32.
template <int DT>
__device__ __forceinline__ double exp_rel_f64(float z, float M, const TempConst& tc) {
  float ah, al;
  if constexpr (DT == DT_BF16) {
    const float d = fmaxf(z - M, tc.d_min);
    ah = d * tc.c_hi;
    al = fmaf(d, tc.c_hi, -ah);
    al = fmaf(d, tc.c_lo, al);
  } else {
    double a = ((double)z - (double)M) * tc.c64;
    a = a > -200.0 ? a : -200.0;
    ah = (float)a;
    al = (float)(a - (double)ah);
  }
  const double e = (double)__builtin_amdgcn_exp2f(ah);
  return fma(e, (double)al * kLn2, e);
}

// The row a final draw samples from: the target row alone (weights
// e_t = 2^((z_t - M_t) c), proportional to p), or a residual row with weights
// max(0, e_t - rho e_d) proportional to max(0, p - (rho S_d / S_t) q); rho is
// carried as the float pair rho_hi + rho_lo.
struct DrawRow {
  const char* t;      // target row base (element 0 of the row)
  const char* d;      // draft row base (resid only)
  float Mt, Md;       // row maxima (exp_rel weights)
  float Kt, Kd;       // exponent offsets (exp_koff weights)
  float rho_hi, rho_lo;
  double rho;         // rho_hi + rho_lo, unsplit (draw_weight_f64)
  bool resid;
};

// 2^(z c - K) in the row sweep's K-offset form: a = fl(z c_lo + fl(z c_hi - K))
// carries both halves of c = log2(e)/T, and K (a row's fl(M c_hi)) is the only
// per-row constant.  One fp32 rounding of the exponent (|a| ulp / 2), then the
// hardware exp2; -inf logits give 0 (c_lo > 0).  The linear draw's weights:
// measured in emulation on the large workload's rows (bf16 N(0, 2), draft
// noise 0.8, T = 0.7), the expected share of draws whose token moves,
// sum_v |F(v) - F_exact(v)|, is about 2.0e-4 for residual draws and 2.3e-4
// for bonus draws, against 1.5e-4 and 0.8e-4 with exp_rel's double-float
// exponent: the hardware exp2's own rounding dominates the residual draws.
__device__ __forceinline__ float exp_koff(float z, float K, const TempConst& tc) {
  return __builtin_amdgcn_exp2f(fmaf(z, tc.c_lo, fmaf(z, tc.c_hi, -K)));
}

// Draw weight of the linear draw: the bonus row's 2^(z_t c - K_t), or the
// residual row's max(0, 2^(z_t c - K_t) - rho 2^(z_d c - K_d)) (rho carried as
// rho_hi + rho_lo); both proportional to the row's p or max(0, p - q).
template <bool RESID>
__device__ __forceinline__ float draw_weight_k(const DrawRow& R, float zt, float zd, const TempConst& tc) {
  const float et = exp_koff(zt, R.Kt, tc);
  if constexpr (!RESID) {
    return et;
  } else {
    const float ed = exp_koff(zd, R.Kd, tc);
    float w = fmaf(-ed, R.rho_hi, et);
    w = fmaf(-ed, R.rho_lo, w);
    return fmaxf(w, 0.f);
  }
}
__device__ __forceinline__ float draw_weight_k(const DrawRow& R, float zt, float zd, const TempConst& tc) {
  return R.resid ? draw_weight_k<true>(R, zt, zd, tc) : draw_weight_k<false>(R, zt, zd, tc);
}

// Exponent offset K = fl(M c_hi) of a row with max M, and the fp64 factor
// 2^(K - M c) between 2^(z c - K) and 2^((z - M) c).
__device__ __forceinline__ float koff_of(float M, const TempConst& tc) { return M * tc.c_hi; }

template <int DT, bool RESID>
__device__ __forceinline__ float draw_weight_r(const DrawRow& R, float zt, float zd, const TempConst& tc) {
  const float et = exp_rel<DT>(zt, R.Mt, tc);
  if constexpr (!RESID) {
    return et;
  } else {
    const float ed = exp_rel<DT>(zd, R.Md, tc);
    float w = fmaf(-ed, R.rho_hi, et);
    w = fmaf(-ed, R.rho_lo, w);
    return fmaxf(w, 0.f);
  }
}
// The same weight with R.resid read at run time.
template <int DT>
__device__ __forceinline__ float draw_weight(const DrawRow& R, float zt, float zd, const TempConst& tc) {
  return R.resid ? draw_weight_r<DT, true>(R, zt, zd, tc) : draw_weight_r<DT, false>(R, zt, zd, tc);
}
// The same weight formed in fp64 from exp_rel_f64 values and the unsplit
// rho: max(0, e_t - rho e_d) with one fp64 rounding.  Its only error left is
// that of the two hardware exp2 heads.
template <int DT>
__device__ __forceinline__ double draw_weight_f64(const DrawRow& R, float zt, float zd, const TempConst& tc) {
  const double et = exp_rel_f64<DT>(zt, R.Mt, tc);
  if (!R.resid) return et;
  const double ed = exp_rel_f64<DT>(zd, R.Md, tc);
  return fmax(fma(-R.rho, ed, et), 0.0);
}

// Wave-parallel location of the segment holding thr: lanes scan the segment
// masses in chunks of 64 (fp64 inclusive scans, fixed order).  Returns the
// segment index and the mass before it; if rounding leaves no crossing, the
// last segment with positive mass and fallback = 1.
// first0 is the caller's copy of the first chunk (lane < nseg ? seg[lane] :
// 0), already in registers, so that chunk is not read again.
__device__ __forceinline__ int locate_segment(const double* seg, int nseg, double thr, int lane, double* base,
                                             int* fallback, double first0) {
  double carry = 0.0;
  int last = 0;
  double lastbase = 0.0;
  for (int c0 = 0; c0 < nseg; c0 += kWave) {
    const int t = c0 + lane;
    const double m = c0 == 0 ? first0 : (t < nseg ? seg[t] : 0.0);
    const double incl = carry + wave_incl_scan(m, lane);
    const unsigned long long mc = __ballot(m > 0.0 && incl > thr);
    const unsigned long long mp = __ballot(m > 0.0);
    if (mc) {
      const int l = (int)__ffsll((long long)mc) - 1;
      *base = readlane_d(incl, l) - readlane_d(m, l);
      *fallback = 0;
      return c0 + l;
    }
    if (mp) {
      const int l = 63 - (int)__clzll((long long)mp);
      last = c0 + l;
      lastbase = readlane_d(incl, l) - readlane_d(m, l);
    }
    carry = readlane_d(incl, kWave - 1);
  }
  *base = lastbase;
  *fallback = 1;
  return last;
}

__device__ __forceinline__ int locate_segment(const double* seg, int nseg, double thr, int lane, double* base,
                                             int* fallback) {
  return locate_segment(seg, nseg, thr, lane, base, fallback, lane < nseg ? seg[lane] : 0.0);
}

// Sequence-level result of the accept scan, handed to the draw kernels.
struct DrawInfo {
  int j;        // accepted drafts (0..gamma), or -1 for an invalid draft token
  float Kt;     // exponent offset of target row j: fl(M_t c_hi)
  float Kd;     // exponent offset of draft row j (j < gamma): fl(M_d c_hi)
  float pad_;
  double rho;   // (S_t / S_d) 2^((K_d - M_d c) - (K_t - M_t c)) of row j (j < gamma)
};

// Per-segment statistics handed from the row sweep to its consumers.
struct Partial {
  float m;      // max of the segment (or -inf)
  int arg;      // lowest row-local index holding m (INT_MAX if none)
  float K;      // exponent offset of s: s = sum 2^(z c - K) over the segment
  float pad_;
  double s;
};

// Merge a row's segment partials within a group of GROUP consecutive lanes
// (GROUP a power of two dividing 64; gl = lane index inside the group).  The
// row max M is the group max of the partial maxima; the row sum relative to
// it is sum_s s_s 2^(K_s - M c), formed in fp64 with the group's lanes
// adding their partials in segment order and the group combining them in a
// fixed order.  Returns M, the sum (WANT & 1) and the lowest index holding
// M (WANT & 2; 0 for a row of -inf).
// The same merge when every lane holds at most one partial (nseg <= GROUP):
// pp is lane gl's partial, loaded by the caller (valid = gl < nseg), so the
// partials are read once and callers can issue several rows' loads together.
// Same operations in the same order as merge_partials, so the same bits.
template <int WANT, int GROUP>
__device__ __forceinline__ void merge_loaded(const Partial& pp, bool valid, const TempConst& tc, float* M_out,
                                             double* S_out, int* A_out) {
  const float NEG_INF = -__builtin_huge_valf();
  float m = NEG_INF;
  int a = 0x7fffffff;
  if (valid) {
    if (pp.m > m) {
      m = pp.m;
      a = pp.arg;
    } else if (pp.m == m) {
      a = min(a, pp.arg);
    }
  }
  const float M = group_max<GROUP>(m);
  double sv = 0.0;
  if constexpr ((WANT & 1) != 0) {
    if (M != NEG_INF) {
      const double Mc = (double)M * tc.c64;
      if (valid && pp.m != NEG_INF) sv += pp.s * exp2_f64((double)pp.K - Mc);
    }
    sv = group_sum<GROUP>(sv);
  }
  int aa = (m == M && M != NEG_INF) ? a : 0x7fffffff;
  if constexpr ((WANT & 2) != 0) aa = group_min<GROUP>(aa);
  *M_out = M;
  *S_out = sv;
  *A_out = aa == 0x7fffffff ? 0 : aa;
}

__device__ __forceinline__ Partial load_partial(const Partial* part, int nseg, int gl) {
  Partial pp;
  if (gl < nseg) {
    pp = part[gl];
  } else {
    pp.m = -__builtin_huge_valf();
    pp.arg = 0x7fffffff;
    pp.K = 0.f;
    pp.pad_ = 0.f;
    pp.s = 0.0;
  }
  return pp;
}

template <int WANT, int GROUP>
__device__ __forceinline__ void merge_partials(const Partial* part, int nseg, const TempConst& tc, int gl,
                                               float* M_out, double* S_out, int* A_out) {
  if (nseg <= GROUP) {                        // uniform: one partial per lane at most, read once
    merge_loaded<WANT, GROUP>(load_partial(part, nseg, gl), gl < nseg, tc, M_out, S_out, A_out);
    return;
  }
  const float NEG_INF = -__builtin_huge_valf();
  float m = NEG_INF;
  int a = 0x7fffffff;
  for (int t = gl; t < nseg; t += GROUP) {
    const Partial pp = part[t];
    if (pp.m > m) {
      m = pp.m;
      a = pp.arg;
    } else if (pp.m == m) {
      a = min(a, pp.arg);
    }
  }
  const float M = group_max<GROUP>(m);
  double sv = 0.0;
  if constexpr ((WANT & 1) != 0) {
    if (M != NEG_INF) {
      const double Mc = (double)M * tc.c64;
      for (int t = gl; t < nseg; t += GROUP) {
        const Partial pp = part[t];
        if (pp.m != NEG_INF) sv += pp.s * exp2_f64((double)pp.K - Mc);
      }
    }
    sv = group_sum<GROUP>(sv);
  }
  int aa = (m == M && M != NEG_INF) ? a : 0x7fffffff;
  if constexpr ((WANT & 2) != 0) aa = group_min<GROUP>(aa);
  *M_out = M;
  *S_out = sv;
  *A_out = aa == 0x7fffffff ? 0 : aa;
}

// Lane-group width for merging nseg partials: the next power of two, at most 64.
// The accept test of one drafted position rejects unless
// u < p(x)/q(x) = 2^((z_t(x) - M_t) c - (z_d(x) - M_d) c) * S_d / S_t, the
// ratio formed from one fp64 exponent; q(x) = 0 < p(x) accepts, p(x) = 0
// rejects.  Shared by the draw and the early-exit sweep, so both take the
// same decision from the same merged row statistics.
__device__ __forceinline__ bool sample_rejects(float zt, float zd, float Mt, double St, float Md, double Sd,
                                               float u, const TempConst& tc) {
  const double et = ((double)zt - (double)Mt) * tc.c64;
  const double ed = ((double)zd - (double)Md) * tc.c64;
  double r;
  if (!(et > -__builtin_huge_val())) r = 0.0;                          // p(x) = 0
  else if (!(ed > -__builtin_huge_val())) r = __builtin_huge_val();    // q(x) = 0 < p(x)
  else r = exp2_f64(et - ed) * (Sd / St);
  return !((double)u < r);
}

inline int merge_group(int nseg) {
  int g = 1;
  while (g < nseg && g < 64) g <<= 1;
  return g;
}

}  // namespace sv
