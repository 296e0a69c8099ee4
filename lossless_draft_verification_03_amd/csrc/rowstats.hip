// Row sweep: max, sum of 2^((z - max) log2(e) / T) and lowest-index argmax of
// every logit row, in one HBM pass per row.
//
// Pages: "EAGLE-3 speculative decoding review", "EAGLE: Predict Features, Not
// Tokens" (logits -> softmax -> next-token distribution) and "Does Using a
// Small Model's Answer Reduce Quality?" (greedy takes the target's argmax).
//
// Work split: a row is cut into `nseg` segments of whole 16-byte vectors and
// each wavefront reduces one segment; a workgroup is four independent waves.
// A lane loads VPT vectors (coalesced: vector q of the segment goes to lane
// q % 64) before it computes anything, so every lane keeps VPT 16-byte loads
// in flight.  Elements of a row that do not fill a whole aligned vector (row
// head / tail when V is not a multiple of the vector width) are loaded one by
// one by the wave of segment 0.
//
// Numerics of the sum: per wave, with m the wave max, K = fl(m c_hi) and
// a = fl(z c_lo + fl(z c_hi - K)) the exponent of every element carries both
// halves of c = log2(e)/T, so no temperature bias enters; the constant
// offset kappa = m c - K is removed in fp64 at the end.  Four fp32
// accumulators per lane, fp64 from the lane level up.  Every wave writes one
// partial (m, sum, argmax) and exits: there is no handoff between waves
// inside the kernel (an agent-scope release/acquire per wave costs an L2
// write-back and invalidate on this part).  A second, small kernel merges a
// row's partials in segment order in fp64 after the kernel boundary.
#include "sv_kernels.hpp"

#include <limits.h>

namespace sv {

namespace {

constexpr int kVPT = 8;   // 16-byte vectors per lane per segment

template <int DT, int WANT>
__global__ __launch_bounds__(kBlock) void k_row_stats(RowStatsParams P) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  const float NEG_INF = -__builtin_huge_valf();
  const int lane = threadIdx.x & (kWave - 1);
  // the wave index is uniform across the wave; say so, so that everything
  // derived from it (row, segment, buffer descriptor) lives in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const long long unit = (long long)blockIdx.x * (kBlock / kWave) + wave;
  const long long rows = P.rows0 + P.rows1;
  if (unit >= rows * P.nseg) return;
  const long long r = unit / P.nseg;
  const int s = (int)(unit - r * P.nseg);
  const bool second = r >= P.rows0;
  const char* base = static_cast<const char*>(second ? P.src1 : P.src0);
  const long long rr = second ? r - P.rows0 : r;
  const long long V = P.V;
  const long long e0 = rr * V, e1 = e0 + V;
  const long long vfirst = (e0 + EPV - 1) / EPV;   // first whole vector of the row
  const long long vlast = e1 / EPV;                // one past the last whole vector
  const long long vs = vfirst + (long long)s * P.seg_vecs;
  long long ve = vs + P.seg_vecs;
  if (ve > vlast) ve = vlast;
  const int nv = ve > vs ? (int)(ve - vs) : 0;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(base + vs * 16, (uint32_t)nv * 16u);

  // Issue every load before using any: the offset is clamped into the
  // segment (never past it), and vectors beyond the segment are masked to
  // -inf afterwards, so a lane always has kVPT loads in flight.
  v4i raw[kVPT];
  if (nv > 0) {
#pragma unroll
    for (int k = 0; k < kVPT; ++k) {
      const int q = min(k * kWave + lane, nv - 1);
      raw[k] = load16(rsrc, (uint32_t)q * 16u);
    }
  }
  const int neg_pat = DT == DT_BF16 ? (int)0xff80ff80u : (int)0xff800000u;
  float z[kVPT][EPV];
#pragma unroll
  for (int k = 0; k < kVPT; ++k) {
    if ((k + 1) * kWave > nv) {             // wave-uniform: only the tail vectors
      const bool valid = k * kWave + lane < nv;
#pragma unroll
      for (int q = 0; q < 4; ++q) raw[k][q] = valid ? raw[k][q] : neg_pat;
    }
    unpack<DT>(raw[k], z[k]);
  }
  // Row head / tail elements outside whole vectors (segment 0 only).
  float ze = NEG_INF;
  int ie = INT_MAX;
  if (s == 0) {
    const long long he = e1 < vfirst * EPV ? e1 : vfirst * EPV;
    const long long tb = (vlast > vfirst ? vlast : vfirst) * EPV;
    long long e = -1;
    if (lane < EPV) {
      if (e0 + lane < he) e = e0 + lane;
    } else if (lane < 2 * EPV) {
      if (tb + (lane - EPV) < e1) e = tb + (lane - EPV);
    }
    if (e >= 0) {
      ze = load_elem<DT>(base, e);
      ie = (int)(e - e0);
    }
  }

  float m = ze;
#pragma unroll
  for (int k = 0; k < kVPT; ++k)
#pragma unroll
    for (int i = 0; i < EPV; ++i) m = fmaxf(m, z[k][i]);
  const float M = wave_max(m);

  int idx = INT_MAX;
  if constexpr ((WANT & 2) != 0) {
    if (M != NEG_INF) {
      const int lane_base = (int)((vs + lane) * EPV - e0);
#pragma unroll
      for (int k = kVPT - 1; k >= 0; --k)
#pragma unroll
        for (int i = EPV - 1; i >= 0; --i)
          if (z[k][i] == M) idx = lane_base + k * kWave * EPV + i;
      if (ze == M) idx = min(idx, ie);
    }
    idx = wave_min(idx);
  }

  double S = 0.0;
  if constexpr ((WANT & 1) != 0) {
    if (M != NEG_INF) {
      const float c_hi = P.tc.c_hi, c_lo = P.tc.c_lo;
      const float K = M * c_hi;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < kVPT; ++k)
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
          const float a = fmaf(z[k][i], c_lo, fmaf(z[k][i], c_hi, -K));
          acc[i & 3] += __builtin_amdgcn_exp2f(a);
        }
      acc[0] += __builtin_amdgcn_exp2f(fmaf(ze, c_lo, fmaf(ze, c_hi, -K)));
      double t = ((double)acc[0] + (double)acc[1]) + ((double)acc[2] + (double)acc[3]);
      t = wave_sum(t);
      const double kappa = (double)M * P.tc.c64 - (double)K;
      S = t * exp2_f64(-kappa);
    }
  }

  if (lane == 0) {
    Partial pp;
    pp.m = M;
    pp.arg = idx;
    pp.s = S;
    P.part[r * P.nseg + s] = pp;
  }
}

// One wave per row: merge the row's segment partials in segment order.
template <int WANT>
__global__ __launch_bounds__(kBlock) void k_row_merge(RowStatsParams P) {
  const float NEG_INF = -__builtin_huge_valf();
  const int lane = threadIdx.x & (kWave - 1);
  const long long r = (long long)blockIdx.x * (kBlock / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (r >= P.rows0 + P.rows1) return;
  const Partial* part = P.part + r * P.nseg;
  float Mr = NEG_INF;
  for (int t = lane; t < P.nseg; t += kWave) Mr = fmaxf(Mr, part[t].m);
  Mr = wave_max(Mr);
  double Sr = 0.0;
  int ar = INT_MAX;
  for (int t = lane; t < P.nseg; t += kWave) {
    const Partial pp = part[t];
    if constexpr ((WANT & 1) != 0)
      if (pp.m != NEG_INF) Sr += pp.s * exp2_f64(((double)pp.m - (double)Mr) * P.tc.c64);
    if constexpr ((WANT & 2) != 0)
      if (pp.m == Mr) ar = min(ar, pp.arg);
  }
  if constexpr ((WANT & 1) != 0) Sr = wave_sum(Sr);
  if constexpr ((WANT & 2) != 0) ar = wave_min(ar);
  if (lane == 0) {
    P.out_max[r] = Mr;
    if constexpr ((WANT & 1) != 0) P.out_sum[r] = Sr;
    if constexpr ((WANT & 2) != 0) P.out_arg[r] = ar == INT_MAX ? 0 : ar;
  }
}

template <int DT>
hipError_t launch_dt(const RowStatsParams& p, hipStream_t s) {
  const long long rows = p.rows0 + p.rows1;
  const long long units = rows * (long long)p.nseg;
  const long long wpb = kBlock / kWave;
  const long long grid = (units + wpb - 1) / wpb;
  const long long mgrid = (rows + wpb - 1) / wpb;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  switch (p.want) {
    case 1:
      hipLaunchKernelGGL((k_row_stats<DT, 1>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
      hipLaunchKernelGGL((k_row_merge<1>), dim3((unsigned)mgrid), dim3(kBlock), 0, s, p);
      break;
    case 2:
      hipLaunchKernelGGL((k_row_stats<DT, 2>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
      hipLaunchKernelGGL((k_row_merge<2>), dim3((unsigned)mgrid), dim3(kBlock), 0, s, p);
      break;
    case 3:
      hipLaunchKernelGGL((k_row_stats<DT, 3>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
      hipLaunchKernelGGL((k_row_merge<3>), dim3((unsigned)mgrid), dim3(kBlock), 0, s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

RowSweepShape row_sweep_shape(int V, int dt) {
  const long long epv = dt == DT_BF16 ? 8 : 4;
  const long long whole = (long long)V / epv;           // whole vectors per row, at most
  const long long cap = (long long)kVPT * kWave;        // vectors one wave reduces
  long long nseg = (whole + cap - 1) / cap;
  if (nseg < 1) nseg = 1;
  long long seg = (whole + nseg - 1) / nseg;
  if (seg < 1) seg = 1;
  return RowSweepShape{(int)nseg, (int)seg};
}

hipError_t launch_row_stats(const RowStatsParams& p, int dt, hipStream_t s) {
  return dt == DT_BF16 ? launch_dt<DT_BF16>(p, s) : launch_dt<DT_F32>(p, s);
}

hipError_t launch_row_sweep(const RowStatsParams& p, int dt, hipStream_t s) {
  const long long units = (p.rows0 + p.rows1) * (long long)p.nseg;
  const long long wpb = kBlock / kWave;
  const long long grid = (units + wpb - 1) / wpb;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL || p.want != 1) return hipErrorInvalidValue;
  if (dt == DT_BF16) hipLaunchKernelGGL((k_row_stats<DT_BF16, 1>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
  else hipLaunchKernelGGL((k_row_stats<DT_F32, 1>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace sv
