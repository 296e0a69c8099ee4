// Row sweep: max, sum of 2^((z - max) log2(e) / T) and lowest-index argmax of
// every logit row, in one HBM pass per row.
//
// Pages: "EAGLE-3 speculative decoding review", "EAGLE: Predict Features, Not
// Tokens" (logits -> softmax -> next-token distribution) and "Does Using a
// Small Model's Answer Reduce Quality?" (greedy takes the target's argmax).
//
// Work split: a row is cut into `nseg` segments of whole 16-byte vectors and
// one workgroup (four waves) reduces one segment into a partial (m, sum,
// argmax).  Lane t of the workgroup loads vectors t, t+256, ... of its
// segment, all kVPT of them before it computes anything (offsets clamped
// into the segment, the excess masked afterwards), with the non-temporal
// cache policy.  Elements of a row outside whole aligned vectors (row head /
// tail when V is not a multiple of the vector width) are loaded one by one
// by segment 0.  With kVPT = 7 a bf16 row of 128256 logits is nine
// segments, so consumers merge a row's few partials inline.  Argmax-only
// sweeps (greedy verification) may ask for kArgmaxVPT = 6 vectors per lane:
// eleven segments per such row, more and shorter workgroups.
//
// Optionally the sweep also picks out z[r][x_r] for a per-row token x_r (the
// drafted token of that position) while the row is in registers, so the
// accept test needs no dependent gather.
//
// Numerics of the sum: with m the segment max, K = fl(m c_hi) and
// a = fl(z c_lo + fl(z c_hi - K)) the exponent of every element carries both
// halves of c = log2(e)/T, so no temperature bias enters.  The partial keeps
// s = sum 2^a together with K; a consumer rescales it to the row max M with
// one fp64 factor 2^(K - M c).  Four fp32 accumulators per lane, fp64 from
// the lane level up, wave reductions by DPP in a fixed order.  There is no
// handoff between workgroups inside the kernel: an agent-scope
// release/acquire per workgroup costs an L2 write-back and invalidate on
// this part, so partials are merged after the kernel boundary.
#include "sv_kernels.hpp"
#include "sweep_segment.hpp"

#include <limits.h>

namespace sv {

namespace {

constexpr int kVPT = kSweepVPT;   // 16-byte vectors per lane per segment

// STEPNP > 0: one early-exit step (see launch_row_step); STEPNP is the lane
// group the draw kernel merges a row's partials with, so the step's accept
// test reproduces the draw's decision bit for bit.
template <int DT, int WANT, int STEPNP = 0, int VPT = kVPT>
__global__ __launch_bounds__(kBlock) void k_row_sweep(RowStatsParams P) {
  __shared__ float sh_m[kBlock / kWave];
  __shared__ double sh_s[kBlock / kWave];
  __shared__ int sh_a[kBlock / kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const long long unit = blockIdx.x;
  long long r;
  int s;
  if constexpr (STEPNP == 0) {
    r = unit / P.nseg;
    s = (int)(unit - r * P.nseg);
  } else {
    // unit -> (sequence b, row k of the block, segment); row k is position
    // step + k/2, target (k even) or draft (k odd); the bonus position g has
    // a target row only, and it can only be the block's last row
    const int i0 = P.step, i1 = P.step_end, ip = P.step_prev, g = P.gather_g;
    const int per = 2 * (i1 - i0) - (i1 > g ? 1 : 0);
    const long long b = unit / (per * P.nseg);
    const int rem = (int)(unit - b * per * P.nseg);
    const int k = rem / P.nseg;
    s = rem - k * P.nseg;
    const int i = i0 + k / 2, kind = k & 1;
    const long long ab = b * (g + 1);
    r = kind == 0 ? ab + i : P.rows0 + b * g + i;
    // The block is needed only if positions 0 .. i0-1 were all accepted, as
    // k_step_alive recorded before this launch (the first block is always
    // needed; it records that for the next test).
    (void)ip;
    if (ip < 0) {
      if (k == 0 && s == 0 && tid == 0) P.step_alive[ab + i0] = 1;
    } else if (!P.step_alive[ab + i0]) {
      return;                                 // uniform
    }
  }
  const bool second = r >= P.rows0;
  const char* base = static_cast<const char*>(second ? P.src1 : P.src0);
  const long long rr = second ? r - P.rows0 : r;
  // where the drafted token of this row is, if the caller asked for the
  // gather (read by sweep_segment once its loads are in flight)
  const int* xtok = nullptr;
  if (P.gather_tokens != nullptr) {
    const long long g1 = second ? P.gather_g : P.gather_g + 1;
    const long long b = rr / g1, i = rr - b * g1;
    if (i < P.gather_g) xtok = P.gather_tokens + b * P.gather_g + i;
  }
  const Partial pp = sweep_segment<DT, WANT, VPT>(base, rr, P.V, s, P.seg_vecs, P.tc, tid, wid, sh_m, sh_s, sh_a, xtok,
                                             P.gather_out != nullptr ? P.gather_out + r : nullptr);
  if (tid == 0) P.part[r * P.nseg + s] = pp;
}

// One wave per row: merge the row's segment partials.
template <int WANT>
__global__ __launch_bounds__(kBlock) void k_row_merge(RowStatsParams P) {
  const int lane = threadIdx.x & (kWave - 1);
  const long long r =
      (long long)blockIdx.x * (kBlock / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (r >= P.rows0 + P.rows1) return;
  float M;
  double S;
  int a;
  merge_partials<WANT, kWave>(P.part + r * P.nseg, P.nseg, P.tc, lane, &M, &S, &a);
  if (lane == 0) {
    P.out_max[r] = M;
    if constexpr ((WANT & 1) != 0) P.out_sum[r] = S;
    if constexpr ((WANT & 2) != 0) P.out_arg[r] = a;
  }
}

// Early exit: whether each sequence needs the block starting at position
// i0 = step.  alive[b][i0] = alive[b][ip] and every position ip .. i0-1
// (ip = step_prev, the previous block's first position) accepted, tested
// from the rows' partials and gathered logits, one position per group of
// STEPNP lanes, each group merging as the draw kernel does, so the decision
// is the draw's bit for bit.  One wave per sequence.
template <int STEPNP>
__global__ __launch_bounds__(kBlock) void k_step_alive(RowStatsParams P) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const long long b = (long long)blockIdx.x * (kBlock / kWave) + tid / kWave;
  if (b >= P.step_B) return;                  // whole waves; no barriers here
  const int i0 = P.step, ip = P.step_prev, g = P.gather_g;
  const long long ab = b * (g + 1);
  // the previous flag is read beside the positions' inputs, not before
  // them: the tests run either way and the flag gates only the result
  int al = P.step_alive[ab + ip];
  {
    constexpr int G = kWave / STEPNP;
    const int gq = lane / STEPNP, gl = lane & (STEPNP - 1);
    for (int c0 = ip; c0 < i0; c0 += G) {
      const int ii = c0 + gq;
      const bool live = ii < i0;              // uniform per lane group
      bool rej = false;
      if (live) {
        const int x = P.gather_tokens[b * g + ii];
        float Mt, Md;
        double St, Sd;
        int a;
        const Partial* pt = P.part + (ab + ii) * P.nseg;
        const Partial* pd = P.part + (P.rows0 + b * g + ii) * P.nseg;
        if (P.nseg <= STEPNP) {
          // both rows' partials in flight together
          const Partial qt = load_partial(pt, P.nseg, gl), qd = load_partial(pd, P.nseg, gl);
          merge_loaded<1, STEPNP>(qt, gl < P.nseg, P.tc, &Mt, &St, &a);
          merge_loaded<1, STEPNP>(qd, gl < P.nseg, P.tc, &Md, &Sd, &a);
        } else {
          merge_partials<1, STEPNP>(pt, P.nseg, P.tc, gl, &Mt, &St, &a);
          merge_partials<1, STEPNP>(pd, P.nseg, P.tc, gl, &Md, &Sd, &a);
        }
        rej = x < 0 || x >= P.V ||
              sample_rejects(P.gather_out[ab + ii], P.gather_out[P.rows0 + b * g + ii], Mt, St, Md, Sd,
                             P.step_unif[ab + ii], P.tc);
      }
      if (__ballot(rej)) al = 0;
    }
  }
  if (lane == 0) P.step_alive[ab + i0] = al;
}

template <int DT, int WANT>
hipError_t launch_sweep_t(const RowStatsParams& p, hipStream_t s) {
  const long long grid = (p.rows0 + p.rows1) * (long long)p.nseg;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (p.vpt != 0 && p.vpt != kVPT) {
    // the argmax-only segments; no other width is built
    if constexpr (WANT == 2) {
      if (p.vpt != kArgmaxVPT || p.seg_vecs > kArgmaxVPT * kBlock) return hipErrorInvalidValue;
      hipLaunchKernelGGL((k_row_sweep<DT, WANT, 0, kArgmaxVPT>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (p.seg_vecs > kVPT * kBlock) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_row_sweep<DT, WANT>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

template <int DT, int NP>
hipError_t launch_step_np(const RowStatsParams& p, hipStream_t s) {
  if (p.step < 0 || p.step_end <= p.step || p.step_end > p.gather_g + 1 || p.step_prev >= p.step) return hipErrorInvalidValue;
  const int per = 2 * (p.step_end - p.step) - (p.step_end > p.gather_g ? 1 : 0);
  const long long grid = (long long)p.step_B * per * p.nseg;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (p.step_prev >= 0) {
    const long long wpb = kBlock / kWave;
    hipLaunchKernelGGL((k_step_alive<NP>), dim3((unsigned)((p.step_B + wpb - 1) / wpb)), dim3(kBlock), 0, s, p);
  }
  hipLaunchKernelGGL((k_row_sweep<DT, 1, NP>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_step_t(const RowStatsParams& p, hipStream_t s) {
  switch (merge_group(p.nseg)) {
    case 1: return launch_step_np<DT, 1>(p, s);
    case 2: return launch_step_np<DT, 2>(p, s);
    case 4: return launch_step_np<DT, 4>(p, s);
    case 8: return launch_step_np<DT, 8>(p, s);
    case 16: return launch_step_np<DT, 16>(p, s);
    case 32: return launch_step_np<DT, 32>(p, s);
    default: return launch_step_np<DT, 64>(p, s);
  }
}

template <int WANT>
hipError_t launch_merge_t(const RowStatsParams& p, hipStream_t s) {
  const long long wpb = kBlock / kWave;
  const long long grid = (p.rows0 + p.rows1 + wpb - 1) / wpb;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_row_merge<WANT>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace

RowSweepShape row_sweep_shape(int V, int dt, int vpt) {
  const long long epv = dt == DT_BF16 ? 8 : 4;
  const long long whole = (long long)V / epv;           // whole vectors per row, at most
  const long long cap = (long long)(vpt > 0 ? vpt : kVPT) * kBlock;   // vectors one workgroup reduces
  long long nseg = (whole + cap - 1) / cap;
  if (nseg < 1) nseg = 1;
  long long seg = (whole + nseg - 1) / nseg;
  if (seg < 1) seg = 1;
  return RowSweepShape{(int)nseg, (int)seg};
}

hipError_t launch_row_sweep(const RowStatsParams& p, int dt, hipStream_t s) {
  if (dt == DT_BF16) {
    switch (p.want) {
      case 1: return launch_sweep_t<DT_BF16, 1>(p, s);
      case 2: return launch_sweep_t<DT_BF16, 2>(p, s);
      case 3: return launch_sweep_t<DT_BF16, 3>(p, s);
    }
  } else {
    switch (p.want) {
      case 1: return launch_sweep_t<DT_F32, 1>(p, s);
      case 2: return launch_sweep_t<DT_F32, 2>(p, s);
      case 3: return launch_sweep_t<DT_F32, 3>(p, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_row_merge(const RowStatsParams& p, hipStream_t s) {
  switch (p.want) {
    case 1: return launch_merge_t<1>(p, s);
    case 2: return launch_merge_t<2>(p, s);
    case 3: return launch_merge_t<3>(p, s);
  }
  return hipErrorInvalidValue;
}

// One position of the early-exit sweep: target and draft row `step` of every
// sequence still alive, with the partial and gather layout of the full sweep.
hipError_t launch_row_step(const RowStatsParams& p, int dt, hipStream_t s) {
  return dt == DT_BF16 ? launch_step_t<DT_BF16>(p, s) : launch_step_t<DT_F32>(p, s);
}

hipError_t launch_row_stats(const RowStatsParams& p, int dt, hipStream_t s) {
  const hipError_t e = launch_row_sweep(p, dt, s);
  if (e != hipSuccess) return e;
  return launch_row_merge(p, s);
}

}  // namespace sv
