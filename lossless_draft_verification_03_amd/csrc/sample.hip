// Speculative sampling after the row sweep: accept scan, residual / bonus
// mass and the inverse-CDF draw, for B sequences.
//
// Pages: "EAGLE-3 speculative decoding review", "Speculative Decoding"
// (3. Accept or Reject: walk the drafts left to right, stop at the first
// rejection, resample it, or take one more token if all are accepted) and
// "Does Using a Small Model's Answer Reduce Quality?" (A(x) = min(1,
// p(x)/q(x)); resample from norm(max(0, p - q))); "EAGLE math", "Vanilla
// speculative decoding" ((p - q)_+ and the +1 bonus token); "Speculative
// decoding" wiki, "The mechanism".
//
// Two kernels after the row sweep; the kernel boundaries are the only
// handoffs between workgroups.
//  k_draw_mass  B x nseg workgroups.  Every workgroup of sequence b first
//               merges the row partials of its 2 gamma + 1 rows in fp64
//               (lane groups of NP lanes, one row per group) and runs the
//               accept scan: lane i tests u_i < p_i(x_i)/q_i(x_i) with the
//               ratio formed from one fp64 exponent (z(x_i) was picked out by
//               the sweep); a ballot gives the first rejection j.  All of
//               them reach the same j; workgroup (b, 0) records it.  Then the
//               draw weights of one segment of row j are summed in fp64, each
//               wave over its own contiguous quarter (a sub-segment):
//                 j <  gamma : w = max(0, p_j - q_j)  (as max(0, e_t - rho e_d))
//                 j == gamma : w = p_gamma            (as e_t)
//               with e = 2^(z c - K) per element in the row sweep's K-offset
//               form (exp_koff), K = fl(M c_hi) per row and rho absorbing
//               both rows' normalisers and offsets.
//  k_draw_pick  one workgroup per sequence: wave 0 locates the sub-segment
//               holding u[b][gamma] * total among the B x 4 nseg masses, the
//               block rescans those 2048 bf16 (1024 fp32) elements with one
//               16-byte run per lane (weights kept in registers), block-scans
//               the lane sums in fp64 and the crossing lane walks its run.
// A residual weight costs two exp2 and about seven other VALU instructions
// per element pair; the pick's rescan is VALU-bound on its one CU, and the
// sub-segments cut it to a quarter of a segment.
#include "sv_kernels.hpp"

#include <limits.h>

namespace sv {

namespace {

// Draw segments by element type: the pick's rescan gives each lane one
// 16-byte vector (8 bf16 or 4 fp32 logits), so a sub-segment (one wave's
// share of a mass workgroup) is 2048 bf16 or 1024 fp32 logits, and a segment
// 8192 or 4096: the same 16 KB of each row per mass workgroup either way.
template <int DT>
constexpr int run_elems() { return DT == DT_BF16 ? 8 : 4; }
template <int DT>
constexpr int sub_elems() { return kBlock * run_elems<DT>(); }
template <int DT>
constexpr int seg_elems() { return kDrawSub * sub_elems<DT>(); }
static_assert(kDrawSub * kWave == kBlock, "one sub-segment per wave");


template <int DT>
__device__ DrawRow draw_row(const SampleParams& P, int b, const DrawInfo& di) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  const int g = P.g;
  const long long V = P.V;
  DrawRow R;
  R.resid = di.j < g;
  R.t = static_cast<const char*>(P.tgt) + ((long long)b * (g + 1) + di.j) * V * ES;
  R.d = R.resid ? static_cast<const char*>(P.drf) + ((long long)b * g + di.j) * V * ES : R.t;
  R.Mt = 0.f;
  R.Md = 0.f;
  R.Kt = di.Kt;
  R.Kd = di.Kd;
  R.rho_hi = (float)di.rho;
  R.rho_lo = (float)(di.rho - (double)R.rho_hi);
  R.rho = di.rho;
  return R;
}

// Sum of the draw weights over elements [s0, s1) of the draw row (at most
// sub_elems<DT>()), lane-interleaved over one wave, fp64 accumulation; returns the
// wave's total in every lane (fixed combination order).
template <int DT, bool ALIGNED, bool RESID>
__device__ double sub_partial(const DrawRow& R, long long s0, long long s1, const TempConst& tc, int lane) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  double acc = 0.0;
  if constexpr (ALIGNED) {
    // every lane issues its KV loads (offsets clamped into the range) before
    // computing
    constexpr int KV = sub_elems<DT>() / EPV / kWave;
    const int nvec = (int)((s1 - s0) / EPV);
    if (nvec > 0) {
      const __amdgpu_buffer_rsrc_t rt = make_rsrc(R.t + s0 * ES, (uint32_t)nvec * 16u);
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(R.d + s0 * ES, (uint32_t)nvec * 16u);
      v4i vt[KV], vd[KV];
#pragma unroll
      for (int k = 0; k < KV; ++k) {
        const uint32_t off = (uint32_t)min(k * kWave + lane, nvec - 1) * 16u;
        vt[k] = load16(rt, off);
        if constexpr (RESID) vd[k] = load16(rd, off);
      }
#pragma unroll
      for (int k = 0; k < KV; ++k) {
        if (k * kWave + lane >= nvec) continue;
        float zt[EPV], zd[EPV];
        unpack<DT>(vt[k], zt);
        if constexpr (RESID) unpack<DT>(vd[k], zd);
#pragma unroll
        for (int i = 0; i < EPV; ++i) acc += (double)draw_weight_k<RESID>(R, zt[i], RESID ? zd[i] : 0.f, tc);
      }
    }
  } else {
    for (long long e = s0 + lane; e < s1; e += kWave) {
      const float zt = load_elem<DT>(R.t, e);
      const float zd = RESID ? load_elem<DT>(R.d, e) : 0.f;
      acc += (double)draw_weight_k<RESID>(R, zt, zd, tc);
    }
  }
  return wave_sum(acc);
}

// Sub-segment masses of segment s of the draw row: wave w sums sub-segment
// 4 s + w and lane 0 stores it.
template <int DT, bool ALIGNED>
__device__ void segment_masses(const DrawRow& R, long long V, int s, const TempConst& tc, int wid, int lane,
                               double* sub) {
  const long long s0 = min((long long)s * seg_elems<DT>() + (long long)wid * sub_elems<DT>(), V);
  const long long s1 = min(s0 + sub_elems<DT>(), V);
  const double m = R.resid ? sub_partial<DT, ALIGNED, true>(R, s0, s1, tc, lane)
                           : sub_partial<DT, ALIGNED, false>(R, s0, s1, tc, lane);
  if (lane == 0) sub[s * kDrawSub + wid] = m;
}

template <int DT, bool ALIGNED, int NP>
__global__ __launch_bounds__(kBlock) void k_draw_mass(SampleParams P) {
  __shared__ float sh_M[2 * 64];
  __shared__ double sh_S[2 * 64];
  __shared__ DrawInfo sh_di;
  // wid is wave-uniform; readfirstlane lets the compiler keep what derives
  // from it (buffer descriptors) in scalar registers
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int b = blockIdx.x / P.nseg, s = blockIdx.x - b * P.nseg;
  const int g = P.g;
  const long long V = P.V;
  const long long rt0 = (long long)b * (g + 1);
  const long long rd0 = (long long)b * g;
  const long long rds0 = (long long)P.B * (g + 1) + rd0;
  // inputs of the accept test that do not depend on the merge
  int x = 0;
  float zt = 0.f, zd = 0.f, u = 0.f;
  if (tid < g) {
    x = P.tokens[rd0 + tid];
    zt = P.gathered[rt0 + tid];
    zd = P.gathered[rds0 + tid];
    u = P.unif[rt0 + tid];
  }
  // merge: rows 0..g are target rows, g+1..2g draft rows
  const int nr = 2 * g + 1;
  for (int row = tid / NP; row < nr; row += kBlock / NP) {
    const long long gr = row <= g ? rt0 + row : rds0 + (row - g - 1);
    float M;
    double S;
    int a;
    merge_partials<1, NP>(P.part + gr * P.nseg_rows, P.nseg_rows, P.tc, tid & (NP - 1), &M, &S, &a);
    if ((tid & (NP - 1)) == 0) {
      sh_M[row] = M;
      sh_S[row] = S;
    }
  }
  __syncthreads();
  if (tid < kWave) {
    bool rej = false, bad = false;
    if (tid < g) {
      if (x < 0 || (long long)x >= V) {
        bad = true;
      } else {
        rej = sample_rejects(zt, zd, sh_M[tid], sh_S[tid], sh_M[g + 1 + tid], sh_S[g + 1 + tid], u, P.tc);
      }
    }
    const unsigned long long mb = __ballot(bad);
    const unsigned long long mr = __ballot(rej);
    if (tid == 0) {
      const int j = mb ? -1 : (mr ? (int)__ffsll((long long)mr) - 1 : g);
      // the draw's weights are 2^(z c - K) with K = fl(M c_hi) per row; rho
      // absorbs the two rows' offsets from the exact 2^((z - M) c)
      DrawInfo di;
      di.j = j;
      const float Mt = j >= 0 ? sh_M[j] : 0.f, Md = (j >= 0 && j < g) ? sh_M[g + 1 + j] : 0.f;
      di.Kt = koff_of(Mt, P.tc);
      di.Kd = koff_of(Md, P.tc);
      di.pad_ = 0.f;
      di.rho = (j >= 0 && j < g)
                   ? sh_S[j] / sh_S[g + 1 + j] *
                         exp2_f64(((double)di.Kd - (double)Md * P.tc.c64) - ((double)di.Kt - (double)Mt * P.tc.c64))
                   : 0.0;
      sh_di = di;
      if (s == 0) {
        P.info[b] = di;
        P.accept_len[b] = j;
      }
    }
  }
  __syncthreads();
  const DrawInfo di = sh_di;
  if (s == 0) {
    int* out = P.out_tokens + rt0;
    for (int i = tid; i <= g; i += kBlock) {
      if (di.j < 0 || i > di.j) out[i] = -1;
      else if (i < di.j) out[i] = P.tokens[rd0 + i];
    }
  }
  if (di.j < 0) return;                       // uniform
  const DrawRow R = draw_row<DT>(P, b, di);
  segment_masses<DT, ALIGNED>(R, V, s, P.tc, wid, lane, P.segsum + (long long)b * P.nseg * kDrawSub);
}

template <int DT, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void k_draw_pick(SampleParams P) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int kRun = run_elems<DT>();
  constexpr int kSubElems = sub_elems<DT>();
  __shared__ double sh_wtot[4];
  __shared__ int sh_first[4];
  __shared__ long long sh_y;
  __shared__ double sh_base, sh_thr;
  // sh_zero: the residual of row j has no mass (draw from p_j instead);
  // sh_locfb: rounding left no crossing in the located sub-segment.  Two
  // flags, because waves 1..3 read sh_zero while wave 0 locates.
  __shared__ int sh_k, sh_zero, sh_locfb;
  // wid is wave-uniform; readfirstlane lets the compiler keep what derives
  // from it (buffer descriptors) in scalar registers
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int b = blockIdx.x;
  const int g = P.g;
  const long long V = P.V;
  const long long ubase = (long long)b * (g + 1);
  const int nsub = P.nseg * kDrawSub;
  double* const sub = P.segsum + (long long)b * nsub;
  // everything this kernel reads first, issued together (the masses are
  // read before j is known; they are ignored when j < 0)
  const DrawInfo di = P.info[b];
  const float u = P.unif[ubase + g];
  double m0 = wid == 0 && lane < nsub ? sub[lane] : 0.0;
  if (di.j < 0) return;                       // k_draw_mass (b, 0) wrote the -1s
  DrawRow R = draw_row<DT>(P, b, di);
  if (wid == 0) {
    // total in a fixed order (chunks of 64, the first kept in registers)
    double total = wave_sum(m0);
    for (int c0 = kWave; c0 < nsub; c0 += kWave) total += wave_sum(c0 + lane < nsub ? sub[c0 + lane] : 0.0);
    if (lane == 0) {
      sh_zero = total > 0.0 ? 0 : 1;
      sh_thr = (double)u * total;
    }
  }
  __syncthreads();
  if (sh_zero) {
    // A zero residual cannot follow a rejection in exact arithmetic; if
    // rounding produces one, draw from p_j (this workgroup recomputes the
    // row's sub-segment masses alone, in place; the barrier makes them
    // visible to wave 0).
    R.resid = false;
    R.d = R.t;
    for (int t = 0; t < P.nseg; ++t) segment_masses<DT, ALIGNED>(R, V, t, P.tc, wid, lane, sub);
    __syncthreads();
    if (wid == 0) {
      m0 = lane < nsub ? sub[lane] : 0.0;
      double total = wave_sum(m0);
      for (int c0 = kWave; c0 < nsub; c0 += kWave) total += wave_sum(c0 + lane < nsub ? sub[c0 + lane] : 0.0);
      if (lane == 0) sh_thr = (double)u * total;
    }
    __syncthreads();
  }
  if (wid == 0) {
    double base;
    int fb;
    // the first 64 masses are still in m0
    const int k = locate_segment(sub, nsub, sh_thr, lane, &base, &fb, m0);
    if (lane == 0) {
      sh_k = k;
      sh_base = base;
      sh_locfb = fb;
      sh_y = -1;
    }
  }
  __syncthreads();
  const long long kb = (long long)__builtin_amdgcn_readfirstlane(sh_k) * kSubElems;   // uniform (LDS)
  const long long ke = kb + kSubElems < V ? kb + kSubElems : V;
  // this lane's run [rb, re) inside sub-segment k, weights kept in registers
  const long long rb0 = kb + (long long)tid * kRun;
  const long long rb = rb0 < ke ? rb0 : ke;
  const long long re = rb + kRun < ke ? rb + kRun : ke;
  float w[kRun];
  if constexpr (ALIGNED) {
    // one descriptor for the whole segment (uniform), per-lane offsets
    constexpr int KV = kRun / EPV;
    const int nvec = (int)((re - rb) / EPV);
    const int segvec = (int)((ke - kb) / EPV);
    const int lane_vec0 = (int)((rb - kb) / EPV);
    if (nvec > 0) {
      const __amdgpu_buffer_rsrc_t rt = make_rsrc(R.t + kb * ES, (uint32_t)segvec * 16u);
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(R.d + kb * ES, (uint32_t)segvec * 16u);
      v4i vt[KV], vd[KV];
#pragma unroll
      for (int k = 0; k < KV; ++k) {
        const uint32_t off = (uint32_t)(lane_vec0 + min(k, nvec - 1)) * 16u;
        vt[k] = load16(rt, off);
        if (R.resid) vd[k] = load16(rd, off);
      }
#pragma unroll
      for (int k = 0; k < KV; ++k) {
        float zt[EPV], zd[EPV];
        unpack<DT>(vt[k], zt);
        if (R.resid) unpack<DT>(vd[k], zd);
#pragma unroll
        for (int i = 0; i < EPV; ++i)
          w[k * EPV + i] = k < nvec ? draw_weight_k(R, zt[i], R.resid ? zd[i] : 0.f, P.tc) : 0.f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < kRun; ++e) w[e] = 0.f;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      const long long ee = rb + e;
      float v = 0.f;
      if (ee < re) {
        const float zt = load_elem<DT>(R.t, ee);
        const float zd = R.resid ? load_elem<DT>(R.d, ee) : 0.f;
        v = draw_weight_k(R, zt, zd, P.tc);
      }
      w[e] = v;
    }
  }
  // lane sum in run order through four interleaved fp64 chains
  double T4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int e = 0; e < kRun; ++e) T4[e & 3] += (double)w[e];
  const double T = (T4[0] + T4[1]) + (T4[2] + T4[3]);
  const double incl = wave_incl_scan(T, lane);
  if (lane == kWave - 1) sh_wtot[wid] = incl;
  __syncthreads();
  double wbase = 0.0;
  for (int v = 0; v < wid; ++v) wbase += sh_wtot[v];
  const double excl = sh_base + wbase + (incl - T);
  const double thr = sh_thr;
  const bool cross = !sh_locfb && T > 0.0 && excl + T > thr;
  const unsigned long long mc = __ballot(cross);
  const unsigned long long mp = __ballot(T > 0.0);
  if (lane == 0) sh_first[wid] = mc ? wid * kWave + (int)__ffsll((long long)mc) - 1 : INT_MAX;
  __syncthreads();
  const int first = min(min(sh_first[0], sh_first[1]), min(sh_first[2], sh_first[3]));
  __syncthreads();
  if (lane == 0) sh_first[wid] = mp ? wid * kWave + 63 - (int)__clzll((long long)mp) : -1;
  __syncthreads();
  const int lastpos = max(max(sh_first[0], sh_first[1]), max(sh_first[2], sh_first[3]));
  const int who = first != INT_MAX ? first : lastpos;
  if (tid == who) {
    double acc = excl;
    int y = -1, ylast = -1;
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      if (w[e] > 0.f) {
        acc += (double)w[e];
        ylast = e;
        if (y < 0 && first != INT_MAX && acc > thr) y = e;
      }
    }
    sh_y = rb + (y >= 0 ? y : ylast);
  }
  __syncthreads();
  if (tid == 0) P.out_tokens[ubase + di.j] = (int)sh_y;
}

template <int DT, bool ALIGNED, int NP>
hipError_t launch_sample_np(const SampleParams& p, hipStream_t s) {
  hipLaunchKernelGGL((k_draw_mass<DT, ALIGNED, NP>), dim3((unsigned)((long long)p.B * p.nseg)), dim3(kBlock), 0, s,
                     p);
  hipLaunchKernelGGL((k_draw_pick<DT, ALIGNED>), dim3((unsigned)p.B), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

template <int DT, bool ALIGNED>
hipError_t launch_sample_t(const SampleParams& p, hipStream_t s) {
  switch (merge_group(p.nseg_rows)) {
    case 1: return launch_sample_np<DT, ALIGNED, 1>(p, s);
    case 2: return launch_sample_np<DT, ALIGNED, 2>(p, s);
    case 4: return launch_sample_np<DT, ALIGNED, 4>(p, s);
    case 8: return launch_sample_np<DT, ALIGNED, 8>(p, s);
    case 16: return launch_sample_np<DT, ALIGNED, 16>(p, s);
    case 32: return launch_sample_np<DT, ALIGNED, 32>(p, s);
    default: return launch_sample_np<DT, ALIGNED, 64>(p, s);
  }
}

}  // namespace

int sample_draw_segments(int V, int dt, int* seg_elems_out) {
  const int se = dt == DT_BF16 ? seg_elems<DT_BF16>() : seg_elems<DT_F32>();
  long long n = ((long long)V + se - 1) / se;
  if (n < 1) n = 1;
  *seg_elems_out = se;
  return (int)n;
}

hipError_t launch_sample(const SampleParams& p, int dt, hipStream_t s) {
  if ((long long)p.B * p.nseg > 0x7fffffffLL) return hipErrorInvalidValue;
  const bool aligned = dt == DT_BF16 ? (p.V % 8 == 0) : (p.V % 4 == 0);
  if (dt == DT_BF16) return aligned ? launch_sample_t<DT_BF16, true>(p, s) : launch_sample_t<DT_BF16, false>(p, s);
  return aligned ? launch_sample_t<DT_F32, true>(p, s) : launch_sample_t<DT_F32, false>(p, s);
}

}  // namespace sv
