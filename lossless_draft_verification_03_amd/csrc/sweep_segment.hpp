// One segment of the row sweep as a device function: the partial (max,
// lowest-index argmax, exponent offset K, sum of 2^(z c - K)) of segment s of
// row rr of a [*, V] logit tensor, reduced by one group of kBlock threads.
// Shared by the row sweep kernel and by kernels that need the statistics of a
// few rows on the fly (the tree sampler), so both produce the same bits.
//
// Layout: the row is cut into segments of seg_vecs whole 16-byte vectors,
// counted from the tensor base (so a row's head and tail may hold elements
// outside whole vectors; segment 0 loads those one by one).  Lane t of the
// group loads vectors t, t + kBlock, ... (kSweepVPT per lane) before it
// computes anything, offsets clamped into the segment and the excess masked
// afterwards, with the non-temporal cache policy.
//
// Numerics of the sum: with m the segment max, K = fl(m c_hi) and
// a = fl(z c_lo + fl(z c_hi - K)) the exponent of every element carries both
// halves of c = log2(e)/T, so no temperature bias enters.  The partial keeps
// s = sum 2^a together with K; a consumer rescales it to the row max M with
// one fp64 factor 2^(K - M c).  Four fp32 accumulators per lane, fp64 from
// the lane level up, wave reductions by DPP in a fixed order.
#pragma once

#include <limits.h>

#include "sv_common.hpp"

namespace sv {

#ifndef SV_SWEEP_VPT
#define SV_SWEEP_VPT 7
#endif
constexpr int kSweepVPT = SV_SWEEP_VPT;   // 16-byte vectors per lane per segment

// VPT (vectors per lane) sets the segment's capacity, VPT * kBlock vectors;
// seg_vecs must not exceed it.
// tid in [0, kBlock) and wid = tid / kWave index the thread inside its group;
// sh_m, sh_s, sh_a are the group's LDS slots (kBlock / kWave each).  Every
// thread of the workgroup must make the call (two workgroup barriers); the
// returned partial is the same in every lane of the group.  If xtok is not
// null and x = *xtok lies in [0, V), z[rr][x] is stored to *gdst; *xtok is
// read only after the segment's loads are issued, so they do not wait for it.
template <int DT, int WANT, int VPT = kSweepVPT>
__device__ __forceinline__ Partial sweep_segment(const char* base, long long rr, long long V, int s, int seg_vecs,
                                                 const TempConst& tc, int tid, int wid, float* sh_m, double* sh_s,
                                                 int* sh_a, const int* xtok, float* gdst) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int kVPT = VPT;
  const float NEG_INF = -__builtin_huge_valf();
  const int lane = tid & (kWave - 1);
  (void)ES;
  const long long e0 = rr * V, e1 = e0 + V;
  const long long vfirst = (e0 + EPV - 1) / EPV;   // first whole vector of the row
  const long long vlast = e1 / EPV;                // one past the last whole vector
  const long long vs = vfirst + (long long)s * seg_vecs;
  long long ve = vs + seg_vecs;
  if (ve > vlast) ve = vlast;
  const int nv = ve > vs ? (int)(ve - vs) : 0;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(base + vs * 16, (uint32_t)nv * 16u);
  v4i raw[kVPT];
  if (nv > 0) {
#pragma unroll
    for (int k = 0; k < kVPT; ++k) {
      const int q = min(k * kBlock + tid, nv - 1);
      raw[k] = load16(rsrc, (uint32_t)q * 16u);
    }
  }
  long long gx = -1;
  if (xtok != nullptr) {
    const int x = *xtok;
    if (x >= 0 && (long long)x < V) gx = x;
  }
  const int neg_pat = DT == DT_BF16 ? (int)0xff80ff80u : (int)0xff800000u;
#pragma unroll
  for (int k = 0; k < kVPT; ++k) {
    if ((k + 1) * kBlock > nv) {            // uniform: only the tail vectors
      const bool valid = k * kBlock + tid < nv;
#pragma unroll
      for (int q = 0; q < 4; ++q) raw[k][q] = valid ? raw[k][q] : neg_pat;
    }
  }
  // Row head / tail elements outside whole vectors (segment 0, wave 0).
  float ze = NEG_INF;
  int ie = INT_MAX;
  if (s == 0 && tid < 2 * EPV) {
    const long long he = e1 < vfirst * EPV ? e1 : vfirst * EPV;
    const long long tb = (vlast > vfirst ? vlast : vfirst) * EPV;
    long long e = -1;
    if (tid < EPV) {
      if (e0 + tid < he) e = e0 + tid;
    } else {
      if (tb + (tid - EPV) < e1) e = tb + (tid - EPV);
    }
    if (e >= 0) {
      ze = load_elem<DT>(base, e);
      ie = (int)(e - e0);
    }
  }
  // row-local index of element i of this lane's vector k: lane_base + k*kBlock*EPV + i
  const int lane_base = (int)((vs + tid) * EPV - e0);

  // pick out z[x] if x lies in this segment's whole vectors or edge elements
  if (gx >= 0) {
    const long long gv = (e0 + gx) / EPV;    // vector holding element x
    if (gv >= vs && gv < ve) {
      const int q = (int)(gv - vs);
      if ((q & (kBlock - 1)) == tid) {
        const int kk = q / kBlock;
        const int ii = (int)((e0 + gx) - gv * EPV);
        float zz = 0.f;
#pragma unroll
        for (int k = 0; k < kVPT; ++k) {
          if (k == kk) {
            float z[EPV];
            unpack<DT>(raw[k], z);
#pragma unroll
            for (int i = 0; i < EPV; ++i)
              if (i == ii) zz = z[i];
          }
        }
        *gdst = zz;
      }
    }
    if (ie == (int)gx) *gdst = ze;
  }

  // workgroup max: every wave's max through LDS (one barrier)
  float m = ze;
#pragma unroll
  for (int k = 0; k < kVPT; ++k) {
    float z[EPV];
    unpack<DT>(raw[k], z);
#pragma unroll
    for (int i = 0; i < EPV; ++i) m = fmaxf(m, z[i]);
  }
  const float Mw = wave_max(m);
  if (lane == 0) sh_m[wid] = Mw;
  __syncthreads();
  float M = sh_m[0];
#pragma unroll
  for (int w = 1; w < kBlock / kWave; ++w) M = fmaxf(M, sh_m[w]);

  int idx = INT_MAX;
  if constexpr ((WANT & 2) != 0) {
    if (M != NEG_INF && Mw == M) {          // uniform per wave
#pragma unroll
      for (int k = kVPT - 1; k >= 0; --k) {
        float z[EPV];
        unpack<DT>(raw[k], z);
#pragma unroll
        for (int i = EPV - 1; i >= 0; --i)
          if (z[i] == M) idx = lane_base + k * kBlock * EPV + i;
      }
      if (ze == M) idx = min(idx, ie);
      idx = wave_min(idx);
    }
  }

  double S = 0.0;
  float K = 0.f;
  if constexpr ((WANT & 1) != 0) {
    if (M != NEG_INF) {
      const float c_hi = tc.c_hi, c_lo = tc.c_lo;
      K = M * c_hi;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < kVPT; ++k) {
        float z[EPV];
        unpack<DT>(raw[k], z);
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
          const float a = fmaf(z[i], c_lo, fmaf(z[i], c_hi, -K));
          acc[i & 3] += __builtin_amdgcn_exp2f(a);
        }
      }
      acc[0] += __builtin_amdgcn_exp2f(fmaf(ze, c_lo, fmaf(ze, c_hi, -K)));
      S = wave_sum(((double)acc[0] + (double)acc[1]) + ((double)acc[2] + (double)acc[3]));
    }
  }
  if (lane == 0) {
    sh_s[wid] = S;
    sh_a[wid] = idx;
  }
  __syncthreads();
  Partial pp;
  pp.m = M;
  pp.arg = min(min(sh_a[0], sh_a[1]), min(sh_a[2], sh_a[3]));
  pp.K = K;
  pp.pad_ = 0.f;
  pp.s = (sh_s[0] + sh_s[1]) + (sh_s[2] + sh_s[3]);
  return pp;
}

}  // namespace sv
