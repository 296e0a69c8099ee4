// Speculative sampling: accept scan, residual / bonus mass and the final
// inverse-CDF draw, for B sequences, after the row sweep has produced every
// row's (max, sum).
//
// Pages: "EAGLE-3 speculative decoding review", "Speculative Decoding"
// (3. Accept or Reject: walk the drafts left to right, stop at the first
// rejection, resample it, or take one more token if all are accepted) and
// "Does Using a Small Model's Answer Reduce Quality?" (A(x) = min(1,
// p(x)/q(x)); resample from norm(max(0, p - q))); "EAGLE math", "Vanilla
// speculative decoding" ((p - q)_+ and the +1 bonus token); "Speculative
// decoding" wiki, "The mechanism".
//
// Grid: B x nseg workgroups.  Every workgroup of sequence b first runs the
// accept scan (wave 0, one lane per drafted position, fp64 ratio from one
// exponent, ballot for the first rejection j); all of them reach the same j.
// Workgroup (b, s) then sums the draw weights of segment s of row j:
//   j <  gamma : w = max(0, p_j - q_j)   (scaled by S_t: max(0, e_t - rho e_d))
//   j == gamma : w = p_gamma             (scaled by S_t: e_t)
// The last workgroup of b (agent-scope arrival count) locates the segment
// holding u[b][gamma] * total, rescans that segment with one contiguous run
// per lane, block-scans the lane sums in fp64 and walks the one lane's run.
#include "sv_kernels.hpp"

#include <limits.h>

namespace sv {

namespace {

constexpr int kDrawVPT = 4;   // vectors per lane per draw segment

struct DrawRow {
  const char* t;      // target row base (element 0 of the row)
  const char* d;      // draft row base (resid only)
  float Mt, Md;
  float rho_hi, rho_lo;
  bool resid;
};

template <int DT>
__device__ __forceinline__ float weight(const DrawRow& R, float zt, float zd, const TempConst& tc) {
  const float et = exp_rel<DT>(zt, R.Mt, tc);
  if (!R.resid) return et;
  const float ed = exp_rel<DT>(zd, R.Md, tc);
  float w = fmaf(-ed, R.rho_hi, et);
  w = fmaf(-ed, R.rho_lo, w);
  return fmaxf(w, 0.f);
}

// Sum of weights over elements [e_beg, e_end) of the draw row, coalesced
// (lane-interleaved), fp64 accumulation.  Returns the lane's partial.
template <int DT, bool ALIGNED>
__device__ double segment_partial(const DrawRow& R, long long e_beg, long long e_end,
                                  const TempConst& tc, int tid) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  double acc = 0.0;
  if constexpr (ALIGNED) {
    const int nvec = (int)((e_end - e_beg) / EPV);
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(R.t + e_beg * ES, (uint32_t)nvec * 16u);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(R.resid ? R.d + e_beg * ES : R.t + e_beg * ES,
                                                (uint32_t)nvec * 16u);
    for (int q = tid; q < nvec; q += kBlock) {
      float zt[EPV], zd[EPV];
      unpack<DT>(load16(rt, (uint32_t)q * 16u), zt);
      if (R.resid) unpack<DT>(load16(rd, (uint32_t)q * 16u), zd);
#pragma unroll
      for (int i = 0; i < EPV; ++i) acc += (double)weight<DT>(R, zt[i], R.resid ? zd[i] : 0.f, tc);
    }
  } else {
    for (long long e = e_beg + tid; e < e_end; e += kBlock) {
      const float zt = load_elem<DT>(R.t, e);
      const float zd = R.resid ? load_elem<DT>(R.d, e) : 0.f;
      acc += (double)weight<DT>(R, zt, zd, tc);
    }
  }
  return acc;
}

// Block-wide fp64 sum with a fixed combination order.
__device__ double block_sum(double x, double* sh4, int tid) {
  x = wave_sum(x);
  __syncthreads();
  if ((tid & (kWave - 1)) == 0) sh4[tid / kWave] = x;
  __syncthreads();
  const double t = (sh4[0] + sh4[1]) + (sh4[2] + sh4[3]);
  __syncthreads();
  return t;
}

template <int DT, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void k_sample(SampleParams P) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  __shared__ int sh_j;
  __shared__ int sh_last;
  __shared__ double sh4[4];
  __shared__ double sh_wtot[4];
  __shared__ int sh_first[4];
  __shared__ long long sh_y;
  __shared__ double sh_base, sh_thr;
  __shared__ int sh_k, sh_fallback;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int b = blockIdx.x / P.nseg, s = blockIdx.x - b * P.nseg;
  const int g = P.g;
  const long long V = P.V;
  const long long rt0 = (long long)b * (g + 1);              // target rows of b
  const long long rd0s = (long long)P.B * (g + 1) + (long long)b * g;   // draft rows in stats
  const long long rd0 = (long long)b * g;                    // draft rows in the tensor
  const TempConst tc = P.tc;

  // ---- accept scan: lane i tests drafted position i
  if (wid == 0) {
    bool rej = false, bad = false;
    if (lane < g) {
      const int x = P.tokens[rd0 + lane];
      if (x < 0 || (long long)x >= V) {
        bad = true;
      } else {
        const float zt = load_elem<DT>(P.tgt, (rt0 + lane) * V + x);
        const float zd = load_elem<DT>(P.drf, (rd0 + lane) * V + x);
        const double et = ((double)zt - (double)P.row_max[rt0 + lane]) * tc.c64;
        const double ed = ((double)zd - (double)P.row_max[rd0s + lane]) * tc.c64;
        double r;
        if (!(et > -__builtin_huge_val())) r = 0.0;                 // p(x) = 0
        else if (!(ed > -__builtin_huge_val())) r = __builtin_huge_val();  // q(x) = 0
        else r = exp2_f64(et - ed) * (P.row_sum[rd0s + lane] / P.row_sum[rt0 + lane]);
        const double u = (double)P.unif[rt0 + lane];
        rej = !(u < r);
      }
    }
    const unsigned long long mb = __ballot(bad);
    const unsigned long long mr = __ballot(rej);
    if (lane == 0) sh_j = mb ? -1 : (mr ? (int)__ffsll((long long)mr) - 1 : g);
  }
  __syncthreads();
  const int j = sh_j;

  DrawRow R;
  R.resid = false;
  R.t = R.d = nullptr;
  R.Mt = R.Md = 0.f;
  R.rho_hi = R.rho_lo = 0.f;
  if (j >= 0) {
    R.resid = j < g;
    R.t = static_cast<const char*>(P.tgt) + (rt0 + j) * V * ES;
    R.Mt = P.row_max[rt0 + j];
    if (R.resid) {
      R.d = static_cast<const char*>(P.drf) + (rd0 + j) * V * ES;
      R.Md = P.row_max[rd0s + j];
      const double rho = P.row_sum[rt0 + j] / P.row_sum[rd0s + j];
      R.rho_hi = (float)rho;
      R.rho_lo = (float)(rho - (double)R.rho_hi);
    }
  }

  // ---- pass 1: this workgroup's segment mass
  const long long sb = (long long)s * P.seg_elems;
  const long long se = sb + P.seg_elems < V ? sb + P.seg_elems : V;
  double part = 0.0;
  if (j >= 0) part = segment_partial<DT, ALIGNED>(R, sb, se, tc, tid);
  part = block_sum(part, sh4, tid);
  if (tid == 0) {
    P.segsum[(long long)b * P.nseg + s] = part;
    sh_last = count_arrival(P.cnt + b) == (unsigned)(P.nseg - 1);
  }
  __syncthreads();
  if (!sh_last) return;
  acquire_agent();

  int* out = P.out_tokens + rt0;
  if (j < 0) {
    for (int i = tid; i <= g; i += kBlock) out[i] = -1;
    if (tid == 0) {
      P.accept_len[b] = -1;
      P.cnt[b] = 0u;
    }
    return;
  }

  // ---- locate the segment holding u * total (thread 0, segment order)
  const double* seg = P.segsum + (long long)b * P.nseg;
  if (tid == 0) {
    double total = 0.0;
    for (int t = 0; t < P.nseg; ++t) total += seg[t];
    sh_fallback = total > 0.0 ? 0 : 1;
    sh_thr = (double)P.unif[rt0 + g] * total;
  }
  __syncthreads();
  if (sh_fallback) {
    // A zero residual cannot follow a rejection in exact arithmetic; if
    // rounding produces one, draw from p_j (this workgroup recomputes the
    // row's bonus-style segment masses alone).
    R.resid = false;
    for (int t = 0; t < P.nseg; ++t) {
      const long long b0 = (long long)t * P.seg_elems;
      const long long b1 = b0 + P.seg_elems < V ? b0 + P.seg_elems : V;
      const double m = block_sum(segment_partial<DT, ALIGNED>(R, b0, b1, tc, tid), sh4, tid);
      if (tid == 0) P.segsum[(long long)b * P.nseg + t] = m;
    }
    __syncthreads();
    if (tid == 0) {
      double total = 0.0;
      for (int t = 0; t < P.nseg; ++t) total += seg[t];
      sh_thr = (double)P.unif[rt0 + g] * total;
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double thr = sh_thr;
    double acc = 0.0;
    int k = -1, lastpos = -1;
    double lastbase = 0.0;
    for (int t = 0; t < P.nseg; ++t) {
      const double m = seg[t];
      if (m > 0.0 && acc + m > thr) { k = t; break; }
      if (m > 0.0) { lastpos = t; lastbase = acc; }
      acc += m;
    }
    if (k >= 0) { sh_k = k; sh_base = acc; sh_fallback = 0; }
    else { sh_k = lastpos; sh_base = lastbase; sh_fallback = 1; }   // rounding: last positive segment
  }
  __syncthreads();
  const int k = sh_k;
  const long long kb = (long long)k * P.seg_elems;
  const long long ke = kb + P.seg_elems < V ? kb + P.seg_elems : V;

  // ---- pass 2: one contiguous run per lane inside segment k
  long long run = (ke - kb + kBlock - 1) / kBlock;
  if (ALIGNED) run = (run + EPV - 1) / EPV * EPV;
  long long rb = kb + (long long)tid * run;
  if (rb > ke) rb = ke;
  long long re = rb + run < ke ? rb + run : ke;
  double T = 0.0;
  for (long long e = rb; e < re; ++e) {
    const float zt = load_elem<DT>(R.t, e);
    const float zd = R.resid ? load_elem<DT>(R.d, e) : 0.f;
    T += (double)weight<DT>(R, zt, zd, tc);
  }
  // exclusive block scan of the lane sums
  const double incl = wave_incl_scan(T, lane);
  if (lane == kWave - 1) sh_wtot[wid] = incl;
  __syncthreads();
  double wbase = 0.0;
  for (int w = 0; w < wid; ++w) wbase += sh_wtot[w];
  const double excl = sh_base + wbase + (incl - T);
  const bool cross = !sh_fallback && T > 0.0 && excl + T > sh_thr;
  const bool haspos = T > 0.0;
  const unsigned long long mc = __ballot(cross);
  const unsigned long long mp = __ballot(haspos);
  if (lane == 0) sh_first[wid] = mc ? wid * kWave + (int)__ffsll((long long)mc) - 1 : INT_MAX;
  __syncthreads();
  int first = min(min(sh_first[0], sh_first[1]), min(sh_first[2], sh_first[3]));
  __syncthreads();
  // last lane with positive mass (used when rounding leaves no crossing)
  if (lane == 0) sh_first[wid] = mp ? wid * kWave + 63 - (int)__clzll((long long)mp) : -1;
  __syncthreads();
  const int lastpos = max(max(sh_first[0], sh_first[1]), max(sh_first[2], sh_first[3]));
  const int who = first != INT_MAX ? first : lastpos;
  if (tid == who) {
    double acc = excl;
    long long y = -1, ylast = -1;
    for (long long e = rb; e < re; ++e) {
      const float zt = load_elem<DT>(R.t, e);
      const float zd = R.resid ? load_elem<DT>(R.d, e) : 0.f;
      const float w = weight<DT>(R, zt, zd, tc);
      if (w > 0.f) {
        acc += (double)w;
        ylast = e;
        if (first != INT_MAX && acc > sh_thr) { y = e; break; }
      }
    }
    sh_y = y >= 0 ? y : ylast;
  }
  __syncthreads();
  const int yv = (int)sh_y;
  const int* x = P.tokens + rd0;
  for (int i = tid; i <= g; i += kBlock) out[i] = i < j ? x[i] : (i == j ? yv : -1);
  if (tid == 0) {
    P.accept_len[b] = j;
    P.cnt[b] = 0u;
  }
}

}  // namespace

int sample_draw_segments(int V, int* seg_elems) {
  // 256 lanes x 4 vectors x 8 elements per segment (a multiple of every
  // vector width), at least one segment.
  const long long per = (long long)kBlock * kDrawVPT * 8;
  long long n = ((long long)V + per - 1) / per;
  if (n < 1) n = 1;
  *seg_elems = (int)per;
  return (int)n;
}

hipError_t launch_sample(const SampleParams& p, int dt, hipStream_t s) {
  const long long grid = (long long)p.B * p.nseg;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const bool aligned = dt == DT_BF16 ? (p.V % 8 == 0) : (p.V % 4 == 0);
  if (dt == DT_BF16) {
    if (aligned) hipLaunchKernelGGL((k_sample<DT_BF16, true>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
    else hipLaunchKernelGGL((k_sample<DT_BF16, false>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
  } else {
    if (aligned) hipLaunchKernelGGL((k_sample<DT_F32, true>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
    else hipLaunchKernelGGL((k_sample<DT_F32, false>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace sv
