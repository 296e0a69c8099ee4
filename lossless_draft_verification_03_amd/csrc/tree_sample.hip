// Stochastic (sampling) verification of a draft tree, after the row sweep.
//
// Pages: "EAGLE-3 speculative decoding review", "The Complete EAGLE-3
// Inference Process" (4. Strict Acceptance: for sampling, min(1, p/q)
// acceptance with residual correction keeps the target distribution, here on
// a tree); "Does Using a Small Model's Answer Reduce Quality?" (A(x) =
// min(1, p(x)/q(x)); resample from norm(max(0, p - q))); "Speculative
// Decoding", 3. Accept or Reject.
//
// Reading of the sibling rule (the pages name it for trees without spelling
// out siblings): the children of a node are tried in increasing node index;
// child k (token x) is tested against p_k(x) / q_k(x), where p_1 = p, q_k is
// the law child k was drawn from, and after each rejection the law moves on
// to p_{k+1} = norm(max(0, p_k - q_k)).  Two drafting laws: children drawn
// independently from the node's draft row q (q_k = q), or one after another
// without replacement (q_k = q with the earlier siblings' tokens removed,
// renormalised: EAGLE-2's k distinct candidates per node, sampled).  An
// accepted child becomes the current node; when every child is rejected one
// token is drawn from the last residual; at a node without children the
// bonus token is drawn from p.  Uniforms: u[n] (n >= 1) is node n's test,
// u[0] the final draw.
//
// Closed form used for the residual chain.  Let R_k = 1 - sum_{i<k} q(x_i)
// over distinct earlier siblings (R_k = 1 for independent draws), so
// q_k = q / R_k off the removed tokens.  With c_1 = 0, W_1 = 1,
//   p_k = max(0, p - c_k q) / W_k,  c_{k+1} = c_k + W_k / R_k,
//   W_{k+1} = sum_v max(0, p(v) - c_{k+1} q(v)).
// (Induction: where p > c_k q and v is not removed, max(0, p_k - q_k) =
// max(0, p - (c_k + W_k / R_k) q) / W_k; elsewhere both sides are 0.  A
// removed token x_i was rejected, so p_i(x_i) < q_i(x_i), which is
// p(x_i) < c_{i+1} q(x_i): the formula already gives it no mass later.)  So
// child k passes iff
//   u < R_k max(0, p(x)/q(x) - c_k) / W_k,
// the ratio p(x)/q(x) formed in fp64 exactly as in the chain sampler, and a
// residual is a draw row with rho = c S_t / S_d.  A zero W (impossible in
// exact arithmetic after a rejection) leaves (c, W) unchanged.  Without
// replacement, a token repeated among siblings is rejected (q_k(x) = 0 and
// p_k(x) = 0) and R_k = 0 (no proposal mass left) gives the ratio rule's
// q = 0 case and leaves (c, W) unchanged.  R_k is the ratio of two sums that
// the W pass after the previous rejection forms from the same fp64 draft
// weights e: over the tokens not removed, and over the whole row.  Nothing
// cancels, so R_k keeps its relative precision however small it is (a
// peaked draft whose first sibling holds all but 1e-12 of q is the usual
// case for k distinct children), and it is exactly 0 when every token with
// weight has been removed.  (1 - sum q(x_i) would lose R_k to cancellation.)
//
// Schedule.  The walk is serial per sequence, but its heavy work is passes
// over one node's two rows: the row statistics of a node the walk enters, and
// one W pass after each rejected sibling that another sibling follows.  One
// CU takes about 20 us for such a pass over a 128K-logit row pair; the chip
// takes a few.  So the walk runs in rounds, one launch each (k_ts_round,
// B x U workgroups of 256 threads).  Every workgroup of a sequence replays
// the walk's decisions from the state the previous round left (they are
// cheap, deterministic and the same in every workgroup): it takes up the
// previous round's pass, tests children until the walk needs another pass
// or reaches its draw, and then does its own segment of that pass (a
// row-sweep segment of the node's target or draft row, or a kTreeSeg-element
// segment of the W pass).  The state and the pass outputs alternate between
// two buffers, so a round reads only what the previous launch wrote, and no
// workgroup waits for another.  k_ts_finish (one 1024-thread workgroup per
// sequence) then takes up the last round and finishes any walk still under
// way on its own CU, calling the same device functions in the same order
// (row-sweep segments merged with the chain sampler's lane grouping; W
// segments summed per wave, combined (w0 + w1) + (w2 + w3), then totalled in
// segment order), so the outputs depend neither on the number of rounds nor
// on n_pre.  The final draw's sub-segment masses are summed by the round in
// which the walk reaches its draw (one segment per workgroup), or by
// k_ts_finish for walks it finishes; k_ts_finish then draws the token by
// inverse CDF, as the chain sampler does.  k_tree_presweep (optional) sweeps
// the rows of the first n_pre nodes of every sequence up front.
#include "sv_kernels.hpp"
#include "sweep_segment.hpp"

#include <limits.h>

namespace sv {

namespace {

constexpr int kTB = 1024;                    // threads of a finishing workgroup
constexpr int kSubE = kTreeSeg / kDrawSub;   // 2048: one wave's sub-segment of a pass segment
constexpr int kRunE = kSubE / kBlock;        // 8: elements per thread in the pick's rescan
static_assert(kDrawSub * kWave == kBlock, "one sub-segment per wave of a 256-thread group");
static_assert(kSubE / kWave <= 32, "one mask bit per element of a lane's share");

// Pending work recorded in a sequence's state.
enum : int {
  kEnter = 0,   // the walk enters node n: its row statistics are needed
  kTest = 1,    // (within a launch only) testing n's children from child i
  kNeedW = 2,   // the W pass of the residual with c = cn is needed
  kDraw = 3,    // the walk is over: draw from the residual with c = cn (from p if cn = 0)
  kDone = 4     // invalid tree or token: outputs written
};

// Test value of the k-th child before the R_k factor: max(0, p(x)/q(x) - c) / W,
// with p(x)/q(x) = 2^((z_t(x) - M_t) c64 - (z_d(x) - M_d) c64) S_d / S_t in
// fp64; p(x) = 0 gives 0, q(x) = 0 < p(x) gives +inf.  For c = 0, W = 1 this
// is the chain sampler's ratio bit for bit.
__device__ __forceinline__ double child_ratio(float zt, float zd, float Mt, double St, float Md, double Sd,
                                              double c, double W, const TempConst& tc) {
  const double et = ((double)zt - (double)Mt) * tc.c64;
  const double ed = ((double)zd - (double)Md) * tc.c64;
  if (!(et > -__builtin_huge_val())) return 0.0;
  if (!(ed > -__builtin_huge_val())) return __builtin_huge_val();
  const double r = exp2_f64(et - ed) * (Sd / St);
  const double d = r - c;
  return d > 0.0 ? d / W : 0.0;
}

__device__ __forceinline__ void set_rho(DrawRow& R, double c, double St, double Sd) {
  R.resid = c > 0.0;
  const double rho = R.resid ? c * (St / Sd) : 0.0;
  R.rho_hi = (float)rho;
  R.rho_lo = (float)(rho - (double)R.rho_hi);
  R.rho = rho;
}

// The rows of the state's node as a draw row with c (a residual if c > 0).
template <int DT>
__device__ __forceinline__ DrawRow node_row(const TreeSampleParams& P, int b, const TreeWalkState& st, double c) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  const long long row = (long long)b * P.N + st.n;
  DrawRow R;
  R.t = static_cast<const char*>(P.tgt) + row * P.V * ES;
  R.d = static_cast<const char*>(P.drf) + row * P.V * ES;
  R.Mt = st.Mt;
  R.Md = st.Md;
  R.Kt = 0.f;
  R.Kd = 0.f;
  set_rho(R, c, st.St, st.Sd);
  return R;
}

// This lane's fp64 sums over elements [s0, s1) (at most kSubE, one wave's
// share) of a residual row R: acc[0] += the weights max(0, e_t - rho e_d)
// formed in fp64 from double-float exponents (one fp64 rounding each), and
// with SD acc[1] += the draft weights e_d and acc[2] += those of tokens other
// than xt[0 .. nx).  Lane-interleaved 16-byte vectors, four per row in flight.
template <int DT, bool ALIGNED, bool SD>
__device__ void wsub(const DrawRow& R, long long s0, long long s1, const TempConst& tc, int lane, const int* xt,
                     int nx, double* acc) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  // SD: bit j marks the lane's j-th element of [s0, s1) (loop order below)
  // as a removed token
  uint32_t xm = 0;
  if constexpr (SD) {
    for (int j = 0; j < nx; ++j) {
      const long long off = (long long)xt[j] - s0;
      if (off < 0 || off >= s1 - s0) continue;
      const int o = (int)off;
      if constexpr (ALIGNED) {
        if (((o / EPV) & (kWave - 1)) == lane) xm |= 1u << ((o / EPV / kWave) * EPV + o % EPV);
      } else {
        if ((o & (kWave - 1)) == lane) xm |= 1u << (o / kWave);
      }
    }
  }
  if constexpr (ALIGNED) {
    constexpr int KV = kSubE / EPV / kWave;     // vectors per lane and row: 4 (bf16) or 8 (fp32)
    constexpr int KC = 4;                        // loaded per round
    const int nvec = (int)((s1 - s0) / EPV);
    if (nvec <= 0) return;
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(R.t + s0 * ES, (uint32_t)nvec * 16u);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(R.d + s0 * ES, (uint32_t)nvec * 16u);
#pragma unroll
    for (int k0 = 0; k0 < KV; k0 += KC) {
      v4i vt[KC], vd[KC];
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const uint32_t off = (uint32_t)min((k0 + k) * kWave + lane, nvec - 1) * 16u;
        vt[k] = load16(rt, off);
        vd[k] = load16(rd, off);
      }
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        if ((k0 + k) * kWave + lane >= nvec) continue;
        float zt[EPV], zd[EPV];
        unpack<DT>(vt[k], zt);
        unpack<DT>(vd[k], zd);
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
          const double et = exp_rel_f64<DT>(zt[i], R.Mt, tc);
          const double ed = exp_rel_f64<DT>(zd[i], R.Md, tc);
          acc[0] += fmax(fma(-R.rho, ed, et), 0.0);
          if constexpr (SD) {
            acc[1] += ed;
            if (!((xm >> ((k0 + k) * EPV + i)) & 1u)) acc[2] += ed;
          }
        }
      }
    }
  } else {
    int j = 0;
    for (long long e = s0 + lane; e < s1; e += kWave, ++j) {
      const double et = exp_rel_f64<DT>(load_elem<DT>(R.t, e), R.Mt, tc);
      const double ed = exp_rel_f64<DT>(load_elem<DT>(R.d, e), R.Md, tc);
      acc[0] += fmax(fma(-R.rho, ed, et), 0.0);
      if constexpr (SD) {
        acc[1] += ed;
        if (!((xm >> j) & 1u)) acc[2] += ed;
      }
    }
  }
}

// Segment s of the W pass of residual row R by one 256-thread group: wave w
// sums sub-segment w, and thread tq == 0 stores the group's sums, combined
// (w0 + w1) + (w2 + w3), to out[0..2] (W, and with SD the draft sums over the
// row and over the kept tokens).  sh: the group's LDS slots.  Every thread of
// the workgroup calls it (two barriers); inactive groups only join them.
template <int DT, bool ALIGNED, bool SD>
__device__ void wpass_segment(const DrawRow& R, long long V, long long s, const TempConst& tc, int tq, int w,
                              int lane, const int* xt, int nx, double (*sh)[3], double* out, bool active) {
  double acc[3] = {0.0, 0.0, 0.0};
  if (active) {
    const long long s0 = min(s * kTreeSeg + (long long)w * kSubE, V);
    const long long s1 = min(s0 + kSubE, V);
    wsub<DT, ALIGNED, SD>(R, s0, s1, tc, lane, xt, nx, acc);
  }
  const double a0 = wave_sum(acc[0]);
  const double a1 = SD ? wave_sum(acc[1]) : 0.0;
  const double a2 = SD ? wave_sum(acc[2]) : 0.0;
  if (lane == 0) {
    sh[w][0] = a0;
    sh[w][1] = a1;
    sh[w][2] = a2;
  }
  __syncthreads();
  if (active && tq == 0) {
#pragma unroll
    for (int k = 0; k < 3; ++k) out[k] = (sh[0][k] + sh[1][k]) + (sh[2][k] + sh[3][k]);
  }
  __syncthreads();
}

// Totals of the W-pass segment records wp[s][0..2] in segment order (chunks
// of 64 segments, each a wave sum); every lane of the calling wave gets them.
__device__ __forceinline__ void wpass_totals(const double* wp, long long nseg, int lane, double* t) {
  double a0 = 0.0, a1 = 0.0, a2 = 0.0;
  for (long long c0 = 0; c0 < nseg; c0 += kWave) {
    const long long s = c0 + lane;
    const bool in = s < nseg;
    a0 += wave_sum(in ? wp[s * 3 + 0] : 0.0);
    a1 += wave_sum(in ? wp[s * 3 + 1] : 0.0);
    a2 += wave_sum(in ? wp[s * 3 + 2] : 0.0);
  }
  t[0] = a0;
  t[1] = a1;
  t[2] = a2;
}

// The final draw's weight sum over elements [s0, s1) (at most kSubE) of row R
// (fp32 weights of draw_weight, fp64 accumulation), as a wave total.
template <int DT, bool ALIGNED>
__device__ double dsub(const DrawRow& R, long long s0, long long s1, const TempConst& tc, int lane) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  double acc = 0.0;
  if constexpr (ALIGNED) {
    constexpr int KV = kSubE / EPV / kWave;
    constexpr int KC = 4;
    const int nvec = (int)((s1 - s0) / EPV);
    if (nvec > 0) {
      const __amdgpu_buffer_rsrc_t rt = make_rsrc(R.t + s0 * ES, (uint32_t)nvec * 16u);
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(R.d + s0 * ES, (uint32_t)nvec * 16u);
#pragma unroll
      for (int k0 = 0; k0 < KV; k0 += KC) {
        v4i vt[KC], vd[KC];
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          const uint32_t off = (uint32_t)min((k0 + k) * kWave + lane, nvec - 1) * 16u;
          vt[k] = load16(rt, off);
          if (R.resid) vd[k] = load16(rd, off);
        }
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          if ((k0 + k) * kWave + lane >= nvec) continue;
          float zt[EPV], zd[EPV];
          unpack<DT>(vt[k], zt);
          if (R.resid) unpack<DT>(vd[k], zd);
#pragma unroll
          for (int i = 0; i < EPV; ++i) acc += (double)draw_weight<DT>(R, zt[i], R.resid ? zd[i] : 0.f, tc);
        }
      }
    }
  } else {
    for (long long e = s0 + lane; e < s1; e += kWave) {
      const float zt = load_elem<DT>(R.t, e);
      const float zd = R.resid ? load_elem<DT>(R.d, e) : 0.f;
      acc += (double)draw_weight<DT>(R, zt, zd, tc);
    }
  }
  return wave_sum(acc);
}

// Rows of the first n_pre nodes of every sequence, swept up front across the
// whole chip (one segment per workgroup, the row sweep's reduction).
template <int DT>
__global__ __launch_bounds__(kBlock) void k_tree_presweep(TreeSampleParams P) {
  __shared__ float sh_m[kBlock / kWave];
  __shared__ double sh_s[kBlock / kWave];
  __shared__ int sh_a[kBlock / kWave];
  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const long long unit = blockIdx.x;
  const long long row = unit / P.nseg;
  const int s = (int)(unit - row * P.nseg);
  const long long half = (long long)P.B * P.n_pre;
  const bool drow = row >= half;
  const long long rl = drow ? row - half : row;
  const long long b = rl / P.n_pre, n = rl - b * P.n_pre;
  const char* base = static_cast<const char*>(drow ? P.drf : P.tgt);
  const Partial pp = sweep_segment<DT, 1, kTreeSampleVPT>(base, b * P.N + n, P.V, s, P.seg_vecs, P.tc, tid, wid, sh_m, sh_s, sh_a,
                                          nullptr, nullptr);
  if (tid == 0) P.pre_part[row * P.nseg + s] = pp;
}

// Workgroups per sequence of a round: enough for either kind of pass.
__host__ __device__ inline long long pass_units(const TreeSampleParams& P) {
  const long long a = 2LL * P.nseg, w = tree_segments(P.V);
  return a > w ? a : w;
}

// The tree of one sequence in LDS (dynamic, 7 N words), and the small
// per-workgroup slots of the walk; TQ = 256-thread quarters of the workgroup.
template <int TQ>
struct WalkLds {
  int* par;
  int* tok;
  float* u;
  float* gt;    // target logit of node c's token in its parent's row
  float* gd;    // draft logit of the same
  int* kids;    // children of the current node, index order
  int* xt;      // without replacement: tokens of the siblings tried so far
  float* preM;  // row statistics of the swept prefix (target rows, then draft rows),
  double* preS; // when staged (prefix_staged)
  double (*sh)[kDrawSub][3];
  float (*qm)[kBlock / kWave];
  double (*qs)[kBlock / kWave];
  int (*qa)[kBlock / kWave];
  int* wcnt;
  float* M;
  double* S;
  double* tot;
};

// The swept prefix's row statistics are merged into LDS up front when all
// 2 n_pre rows fit one pass of NP-lane groups of a 256-thread workgroup;
// otherwise each is merged when the walk enters its node.  Both use the same
// merge, so the bits are the same.
__host__ __device__ inline bool prefix_staged(int n_pre, int NP) { return n_pre > 0 && 2 * n_pre * NP <= kBlock; }

// Bytes of dynamic LDS for a tree of N nodes: seven words per node, then the
// staged prefix statistics of n_stage nodes (8-byte aligned).
__host__ __device__ inline size_t walk_lds_bytes(int N, int n_stage) {
  return (size_t)((7 * N + 1) / 2 * 2) * 4 + (size_t)2 * n_stage * (4 + 8);
}

template <int TQ>
__device__ __forceinline__ void walk_lds_bind(WalkLds<TQ>& L, int* dyn, int N, int n_pre) {
  L.par = dyn;
  L.tok = dyn + N;
  L.u = reinterpret_cast<float*>(dyn + 2 * N);
  L.gt = reinterpret_cast<float*>(dyn + 3 * N);
  L.gd = reinterpret_cast<float*>(dyn + 4 * N);
  L.kids = dyn + 5 * N;
  L.xt = dyn + 6 * N;
  L.preS = reinterpret_cast<double*>(dyn + (7 * N + 1) / 2 * 2);
  L.preM = reinterpret_cast<float*>(L.preS + 2 * n_pre);
}

// Merge the swept prefix's row statistics of sequence b into L.preM / L.preS
// (row r < n_pre: target row of node r; r >= n_pre: draft row of node
// r - n_pre), one NP-lane group per row.  Call only if prefix_staged.
template <int NP, int TQ>
__device__ void stage_prefix(const TreeSampleParams& P, int b, WalkLds<TQ>& L, int tid) {
  const int r = tid / NP;
  if (r < 2 * P.n_pre) {
    const bool drow = r >= P.n_pre;
    const long long n = drow ? r - P.n_pre : r;
    const Partial* src =
        P.pre_part + ((drow ? (long long)P.B * P.n_pre : 0) + (long long)b * P.n_pre + n) * P.nseg;
    float M;
    double S;
    int a;
    merge_partials<1, NP>(src, P.nseg, P.tc, tid & (NP - 1), &M, &S, &a);
    if ((tid & (NP - 1)) == 0) {
      L.preM[r] = M;
      L.preS[r] = S;
    }
  }
  __syncthreads();
}

// Children of node n in index order into L.kids (block scan over contiguous
// runs of nodes per thread); returns their number.  Every thread calls it.
template <int TB, int TQ>
__device__ int list_children(WalkLds<TQ>& L, int n, int N, int tid, int lane, int wid) {
  constexpr int kW = TB / kWave;
  const int per = (N + TB - 1) / TB;
  int cnt = 0;
  for (int j = 0; j < per; ++j) {
    const int c = tid * per + j;
    cnt += c > n && c < N && L.par[c] == n;
  }
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) L.wcnt[wid] = incl;
  __syncthreads();
  int pos = incl - cnt, nk = 0;
  for (int v = 0; v < kW; ++v) {
    const int t = L.wcnt[v];
    if (v < wid) pos += t;
    nk += t;
  }
  for (int j = 0; j < per; ++j) {
    const int c = tid * per + j;
    if (c > n && c < N && L.par[c] == n) L.kids[pos++] = c;
  }
  __syncthreads();
  return nk;
}

// Stage the tree in LDS.  first: validate it, gather every node's token logit
// from its parent's rows (into glog too if write_out) and return whether it
// is invalid; otherwise the logits come from glog.
template <int DT, int TB, int TQ>
__device__ bool stage_tree(const TreeSampleParams& P, int b, WalkLds<TQ>& L, bool first, bool write_out, int tid) {
  const int N = P.N;
  const long long V = P.V;
  const long long row0 = (long long)b * N;
  const int* par_g = P.parent + (long long)b * P.parent_stride;
  float* glog = P.glog + row0 * 2;
  int bad = 0;
  for (int c = tid; c < N; c += TB) {
    const int p = par_g[c];
    const int x = P.tokens[row0 + c];
    float zt, zd;
    if (first) {
      const bool pok = c == 0 ? p == -1 : (p >= 0 && p < c);
      const bool xok = c == 0 || (x >= 0 && (long long)x < V);
      zt = 0.f;
      zd = 0.f;
      if (c > 0 && pok && xok) {
        zt = load_elem<DT>(P.tgt, (row0 + p) * V + x);
        zd = load_elem<DT>(P.drf, (row0 + p) * V + x);
      }
      bad |= !(pok && xok);
      if (write_out) {
        glog[2 * c] = zt;
        glog[2 * c + 1] = zd;
      }
    } else {
      zt = glog[2 * c];
      zd = glog[2 * c + 1];
    }
    L.par[c] = p;
    L.tok[c] = x;
    L.u[c] = P.unif[row0 + c];
    L.gt[c] = zt;
    L.gd[c] = zd;
  }
  return __syncthreads_or(bad) != 0;
}

__device__ __forceinline__ TreeWalkState walk_start() {
  TreeWalkState st;
  st.n = 0;
  st.d = 0;
  st.i = 0;
  st.phase = kEnter;
  st.nk = 0;
  st.mready = 0;
  st.Mt = 0.f;
  st.Md = 0.f;
  st.St = 0.0;
  st.Sd = 0.0;
  st.cc = 0.0;
  st.W = 1.0;
  st.Rk = 1.0;
  st.cn = 0.0;
  st.cfb = 0.0;
  st.pad2_ = 0.0;
  return st;
}

// The walk of sequence b from state st (TB threads, workgroup-uniform):
// take up the pass the state was recorded with if fresh (its row partials in
// part_in, its W records in wp_in), then test children until the walk needs
// a pass (st.phase kEnter beyond the prefix, or kNeedW; the kids of the node
// are in L.kids and st.nk holds their number) or reaches its draw (kDraw).
// COMPLETE: do every pass here instead, one segment per 256-thread quarter,
// into part_in / wp_in, so the walk ends at its draw.  write_out: store the
// accepted path.  Every thread evaluates the same tests on the same values.
template <int DT, bool ALIGNED, int NP, int TB, bool COMPLETE>
__device__ void walk(const TreeSampleParams& P, int b, TreeWalkState& st, bool fresh, WalkLds<TB / kBlock>& L,
                     Partial* part_in, double* wp_in, bool write_out) {
  constexpr int TQ = TB / kBlock;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int N = P.N;
  const long long V = P.V;
  const long long row0 = (long long)b * N;
  const char* tgt = static_cast<const char*>(P.tgt);
  const char* drf = static_cast<const char*>(P.drf);
  const long long nsw = tree_segments(V);
  const int q = wid / (kBlock / kWave), tq = tid & (kBlock - 1), wq = wid & (kBlock / kWave - 1);
  (void)q;
  (void)tq;
  (void)wq;
  for (;;) {
    const int nk = list_children<TB>(L, st.n, N, tid, lane, wid);
    st.nk = nk;
    if (st.phase == kEnter) {
      const bool pre = st.n < P.n_pre;
      if (!pre && !fresh) {
        if constexpr (!COMPLETE) {
          return;                             // a round sweeps the node's rows
        } else {
          // the node's rows here, TQ row-sweep segments at a time, one per
          // quarter (a quarter past the last unit reduces an empty segment)
          const int units = P.nseg * (nk > 0 ? 2 : 1);
          for (int u0 = 0; u0 < units; u0 += TQ) {
            const int u = u0 + q;
            const bool drow = u >= P.nseg && u < units;
            const int s = u < units ? (drow ? u - P.nseg : u) : P.nseg;
            const Partial pp = sweep_segment<DT, 1, kTreeSampleVPT>(drow ? drf : tgt, row0 + st.n, V, s, P.seg_vecs, P.tc, tq, wq,
                                                    L.qm[q], L.qs[q], L.qa[q], nullptr, nullptr);
            if (tq == 0 && u < units) part_in[u] = pp;
          }
          __syncthreads();
        }
      }
      if (pre && prefix_staged(P.n_pre, NP)) {
        st.Mt = L.preM[st.n];
        st.St = L.preS[st.n];
        st.Md = nk > 0 ? L.preM[P.n_pre + st.n] : 0.f;
        st.Sd = nk > 0 ? L.preS[P.n_pre + st.n] : 0.0;
      } else {
        if (wid < 2 && (wid == 0 || nk > 0)) {
          float M;
          double S;
          int a;
          const Partial* src = part_in + wid * P.nseg;
          if (pre)
            src = P.pre_part +
                  ((wid == 0 ? 0 : (long long)P.B * P.n_pre) + (long long)b * P.n_pre + st.n) * P.nseg;
          merge_partials<1, NP>(src, P.nseg, P.tc, lane & (NP - 1), &M, &S, &a);
          if (lane == 0) {
            L.M[wid] = M;
            L.S[wid] = S;
          }
        }
        __syncthreads();
        st.Mt = L.M[0];
        st.St = L.S[0];
        st.Md = nk > 0 ? L.M[1] : 0.f;
        st.Sd = nk > 0 ? L.S[1] : 0.0;
      }
      st.phase = kTest;
      st.i = 0;
      st.cc = 0.0;
      st.W = 1.0;
      st.Rk = 1.0;
      fresh = false;
      __syncthreads();                        // L.M, L.S are read before they are rewritten
    }
    if (nk == 0) {                            // leaf: bonus token from p
      st.cn = 0.0;
      st.cfb = 0.0;
      st.phase = kDraw;
      return;
    }
    bool moved = false;
    for (;;) {
      if (st.phase == kNeedW) {
        // the W pass of the residual after child i: W_{i+1} = sum / S_t, and
        // R_{i+1} from the draft sums
        if (!fresh) {
          if constexpr (!COMPLETE) {
            return;                           // a round forms W
          } else {
            const DrawRow R = node_row<DT>(P, b, st, st.cn);
            for (long long s0 = 0; s0 < nsw; s0 += TQ) {
              const long long s = s0 + q;
              if (P.distinct)
                wpass_segment<DT, ALIGNED, true>(R, V, s, P.tc, tq, wq, lane, L.xt, st.i + 1, L.sh[q],
                                                 wp_in + s * 3, s < nsw);
              else
                wpass_segment<DT, ALIGNED, false>(R, V, s, P.tc, tq, wq, lane, nullptr, 0, L.sh[q], wp_in + s * 3,
                                                  s < nsw);
            }
          }
        }
        if (wid == 0) {
          double t[3];
          wpass_totals(wp_in, nsw, lane, t);
          if (lane == 0) {
            L.tot[0] = t[0];
            L.tot[1] = t[1];
            L.tot[2] = t[2];
          }
        }
        __syncthreads();
        const double Wn = L.tot[0] / st.St;
        if (P.distinct) st.Rk = L.tot[1] > 0.0 ? L.tot[2] / L.tot[1] : 0.0;
        if (Wn > 0.0) {
          st.cc = st.cn;
          st.W = Wn;
        }
        st.i += 1;
        st.phase = kTest;
        fresh = false;
        __syncthreads();                      // L.tot is read before it is rewritten
      }
      const int ci = L.kids[st.i];
      double r = child_ratio(L.gt[ci], L.gd[ci], st.Mt, st.St, st.Md, st.Sd, st.cc, st.W, P.tc);
      if (P.distinct && st.i > 0) {
        int hit = 0;
        for (int j = tid; j < st.i; j += TB) hit |= L.tok[L.kids[j]] == L.tok[ci];
        const bool dup = __syncthreads_or(hit) != 0;
        r = dup ? 0.0 : (st.Rk > 0.0 ? st.Rk * r : (r > 0.0 ? __builtin_huge_val() : 0.0));
      }
      if ((double)L.u[ci] < r) {
        if (write_out && tid == 0) {
          P.out_path[row0 + st.d] = ci;
          P.out_tokens[row0 + st.d] = L.tok[ci];
        }
        st.d += 1;
        st.n = ci;
        st.phase = kEnter;
        moved = true;
        break;
      }
      const double cn = st.Rk > 0.0 ? st.cc + st.W / st.Rk : st.cc;
      if (st.i + 1 == nk) {                   // every child rejected
        st.cn = cn;
        st.cfb = st.cc;
        st.phase = kDraw;
        return;
      }
      if (!(st.Rk > 0.0)) {                   // no proposal mass left: the law stays
        st.i += 1;
        continue;
      }
      st.cn = cn;
      st.phase = kNeedW;
      if (P.distinct) {
        for (int j = tid; j <= st.i; j += TB) L.xt[j] = L.tok[L.kids[j]];
        __syncthreads();
      }
    }
    (void)moved;
    __syncthreads();                          // L.kids is read before it is rebuilt
  }
}

// Shared slots of the final draw.
struct DrawLds {
  double wtot[kBlock / kWave];
  int first[kBlock / kWave];
  long long y;
  double base, thr;
  int k, zero, locfb;
};

// Sub-segment masses of sequence b's final draw for draw segments
// s0, s0 + step, ... (one per 256-thread group g of the caller, wave w of the
// group over sub-segment w): the same sums whichever kernel forms them.
template <int DT, bool ALIGNED>
__device__ void draw_masses(const TreeSampleParams& P, int b, const DrawRow& R, long long s0, long long step, int w,
                            int lane) {
  const long long nsw = tree_segments(P.V);
  for (long long s = s0; s < nsw; s += step) {
    const long long e0 = min(s * kTreeSeg + (long long)w * kSubE, (long long)P.V);
    const long long e1 = min(e0 + kSubE, (long long)P.V);
    const double m = dsub<DT, ALIGNED>(R, e0, e1, P.tc, lane);
    if (lane == 0) P.ws_sub[((long long)b * nsw + s) * kDrawSub + w] = m;
  }
}

// The final draw of sequence b from its sub-segment masses (TB threads; the
// first 256 rescan, the rest join the barriers): total of the masses
// (fallback: the law before the last residual, then p, if rounding leaves
// none; the fallback's masses are formed here by all TB threads), the
// sub-segment holding u[0] * total, a rescan of its kSubE elements (kRunE
// per thread, weights in registers, fp64 block scan), and the outputs.
template <int DT, bool ALIGNED, int TB>
__device__ void draw_final(const TreeSampleParams& P, int b, const TreeWalkState& st, DrawLds& S) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int TQ = TB / kBlock;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int q = wid / (kBlock / kWave), wq = wid & (kBlock / kWave - 1);
  const bool act = tid < kBlock;
  const long long V = P.V;
  const long long nsw = tree_segments(V);
  const int nsub = (int)(nsw * kDrawSub);
  double* const sub = P.ws_sub + (long long)b * nsub;
  const float u = P.unif[(long long)b * P.N];
  DrawRow R = node_row<DT>(P, b, st, st.cn);
  double f0 = 0.0;                            // wave 0: the first 64 masses, kept for the locate step
  for (int attempt = 0;; ++attempt) {
    if (attempt > 0) {
      draw_masses<DT, ALIGNED>(P, b, R, q, TQ, wq, lane);
      __syncthreads();
    }
    if (wid == 0) {
      f0 = lane < nsub ? sub[lane] : 0.0;
      double total = wave_sum(f0);
      for (int c0 = kWave; c0 < nsub; c0 += kWave) total += wave_sum(c0 + lane < nsub ? sub[c0 + lane] : 0.0);
      if (lane == 0) {
        S.zero = total > 0.0 ? 0 : 1;
        S.thr = (double)u * total;
      }
    }
    __syncthreads();
    if (!S.zero || !R.resid) break;           // uniform
    set_rho(R, attempt == 0 ? st.cfb : 0.0, st.St, st.Sd);
    __syncthreads();                          // S.zero is read before it is rewritten
  }
  if (wid == 0) {
    double base;
    int fb;
    const int k = locate_segment(sub, nsub, S.thr, lane, &base, &fb, f0);
    if (lane == 0) {
      S.k = k;
      S.base = base;
      S.locfb = fb;
      S.y = -1;
    }
  }
  __syncthreads();
  const long long kb = (long long)__builtin_amdgcn_readfirstlane(S.k) * kSubE;   // uniform (LDS)
  const long long ke = kb + kSubE < V ? kb + kSubE : V;
  const long long rb0 = kb + (long long)(act ? tid : 0) * kRunE;
  const long long rb = rb0 < ke ? rb0 : ke;
  const long long re = rb + kRunE < ke ? rb + kRunE : ke;
  float w[kRunE];
#pragma unroll
  for (int e = 0; e < kRunE; ++e) w[e] = 0.f;
  if (act) {
    if constexpr (ALIGNED) {
      constexpr int KV = kRunE / EPV;
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
            w[k * EPV + i] = k < nvec ? draw_weight<DT>(R, zt[i], R.resid ? zd[i] : 0.f, P.tc) : 0.f;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < kRunE; ++e) {
        const long long ee = rb + e;
        if (ee < re) {
          const float zt = load_elem<DT>(R.t, ee);
          const float zd = R.resid ? load_elem<DT>(R.d, ee) : 0.f;
          w[e] = draw_weight<DT>(R, zt, zd, P.tc);
        }
      }
    }
  }
  // lane sum in run order through four interleaved fp64 chains
  double T4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int e = 0; e < kRunE; ++e) T4[e & 3] += (double)w[e];
  const double T = (T4[0] + T4[1]) + (T4[2] + T4[3]);
  const double incl = wave_incl_scan(T, lane);
  if (act && lane == kWave - 1) S.wtot[wid] = incl;
  __syncthreads();
  double wbase = 0.0;
  for (int v = 0; v < (act ? wid : 0); ++v) wbase += S.wtot[v];
  const double excl = S.base + wbase + (incl - T);
  const double thr = S.thr;
  const bool cross = act && !S.locfb && T > 0.0 && excl + T > thr;
  const unsigned long long mc = __ballot(cross);
  const unsigned long long mp = __ballot(act && T > 0.0);
  if (act && lane == 0) S.first[wid] = mc ? wid * kWave + (int)__ffsll((long long)mc) - 1 : INT_MAX;
  __syncthreads();
  const int firstc = min(min(S.first[0], S.first[1]), min(S.first[2], S.first[3]));
  __syncthreads();
  if (act && lane == 0) S.first[wid] = mp ? wid * kWave + 63 - (int)__clzll((long long)mp) : -1;
  __syncthreads();
  const int lastpos = max(max(S.first[0], S.first[1]), max(S.first[2], S.first[3]));
  const int who = firstc != INT_MAX ? firstc : lastpos;
  if (act && tid == who) {
    double acc = excl;
    int y = -1, ylast = -1;
#pragma unroll
    for (int e = 0; e < kRunE; ++e) {
      if (w[e] > 0.f) {
        acc += (double)w[e];
        ylast = e;
        if (y < 0 && firstc != INT_MAX && acc > thr) y = e;
      }
    }
    S.y = rb + (y >= 0 ? y : ylast);
  }
  __syncthreads();
  const long long row0 = (long long)b * P.N;
  for (int c = tid; c < P.N; c += TB) {
    if (c >= st.d) P.out_path[row0 + c] = -1;
    if (c > st.d) P.out_tokens[row0 + c] = -1;
  }
  if (tid == 0) {
    P.out_tokens[row0 + st.d] = (int)S.y;
    P.accept_len[b] = st.d;
  }
}

// One round of every sequence's walk: workgroup (b, u) replays the walk from
// the state of the previous round (state_in; the first round stages and
// validates the tree and starts at the root), then does segment u of the
// pass the walk needs next.  Workgroup u = 0 records the new state and the
// accepted path.  Round r reads the pass outputs of round r - 1 (part_in,
// wp_in) and writes its own to the other buffers (part_out, wp_out).
template <int DT, bool ALIGNED, int NP>
__global__ __launch_bounds__(kBlock) void k_ts_round(TreeSampleParams P, int r) {
  extern __shared__ int dyn[];
  __shared__ double sh[1][kDrawSub][3];
  __shared__ float qm[1][kBlock / kWave];
  __shared__ double qs[1][kBlock / kWave];
  __shared__ int qa[1][kBlock / kWave];
  __shared__ int wcnt[kBlock / kWave];
  __shared__ float Ms[2];
  __shared__ double Ss[2];
  __shared__ double tot[3];
  WalkLds<1> L;
  walk_lds_bind(L, dyn, P.N, P.n_pre);
  L.sh = sh;
  L.qm = qm;
  L.qs = qs;
  L.qa = qa;
  L.wcnt = wcnt;
  L.M = Ms;
  L.S = Ss;
  L.tot = tot;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const long long U = pass_units(P);
  const int b = (int)(blockIdx.x / U);
  const long long u = blockIdx.x - (long long)b * U;
  const bool first = r == 0;
  const bool lead = u == 0;
  const long long nsw = tree_segments(P.V);
  const long long Bl = P.B;
  TreeWalkState* state_out = P.state + (long long)((r + 1) & 1) * Bl + b;
  Partial* part_in = P.ws_part + ((long long)((r + 1) & 1) * Bl + b) * 2 * P.nseg;
  Partial* part_out = P.ws_part + ((long long)(r & 1) * Bl + b) * 2 * P.nseg;
  double* wp_in = P.wpart + ((long long)((r + 1) & 1) * Bl + b) * nsw * 3;
  double* wp_out = P.wpart + ((long long)(r & 1) * Bl + b) * nsw * 3;
  TreeWalkState st = first ? walk_start() : P.state[(long long)(r & 1) * Bl + b];
  if (first || st.phase < kDraw) {
    if (prefix_staged(P.n_pre, NP)) stage_prefix<NP>(P, b, L, tid);
    const bool bad = stage_tree<DT, kBlock>(P, b, L, first, lead, tid);
    if (first && bad) {
      if (lead) {
        for (int c = tid; c < P.N; c += kBlock) {
          P.out_path[(long long)b * P.N + c] = -1;
          P.out_tokens[(long long)b * P.N + c] = -1;
        }
        if (tid == 0) P.accept_len[b] = -1;
      }
      st.phase = kDone;
    } else {
      walk<DT, ALIGNED, NP, kBlock, false>(P, b, st, !first, L, part_in, wp_in, lead);
    }
  }
  if (st.phase == kDraw && !st.mready) {
    // the walk reached its draw in this round: segment u of the draw's masses
    if (u < nsw) draw_masses<DT, ALIGNED>(P, b, node_row<DT>(P, b, st, st.cn), u, nsw, wid, lane);
    st.mready = 1;                              // the masses are in place
  } else if (st.phase == kEnter) {
    const long long units = (long long)P.nseg * (st.nk > 0 ? 2 : 1);
    if (u < units) {
      const bool drow = u >= P.nseg;
      const Partial pp = sweep_segment<DT, 1, kTreeSampleVPT>(static_cast<const char*>(drow ? P.drf : P.tgt),
                                              (long long)b * P.N + st.n, P.V, (int)(drow ? u - P.nseg : u),
                                              P.seg_vecs, P.tc, tid, wid, qm[0], qs[0], qa[0], nullptr, nullptr);
      if (tid == 0) part_out[u] = pp;
    }
  } else if (st.phase == kNeedW) {
    if (u < nsw) {
      const DrawRow R = node_row<DT>(P, b, st, st.cn);
      if (P.distinct)
        wpass_segment<DT, ALIGNED, true>(R, P.V, u, P.tc, tid, wid, lane, L.xt, st.i + 1, sh[0], wp_out + u * 3,
                                         true);
      else
        wpass_segment<DT, ALIGNED, false>(R, P.V, u, P.tc, tid, wid, lane, nullptr, 0, sh[0], wp_out + u * 3, true);
    }
  }
  if (lead && tid == 0) *state_out = st;
}

// After the rounds (rounds = R): take up round R - 1's pass, finish every
// walk on its sequence's own workgroup (with R = 0, stage, validate and walk
// from the root), and make the final draw.
template <int DT, bool ALIGNED, int NP>
__global__ __launch_bounds__(kTB) void k_ts_finish(TreeSampleParams P) {
  extern __shared__ int dyn[];
  constexpr int TQ = kTB / kBlock;
  __shared__ double sh[TQ][kDrawSub][3];
  __shared__ float qm[TQ][kBlock / kWave];
  __shared__ double qs[TQ][kBlock / kWave];
  __shared__ int qa[TQ][kBlock / kWave];
  __shared__ int wcnt[kTB / kWave];
  __shared__ float Ms[2];
  __shared__ double Ss[2];
  __shared__ double tot[3];
  WalkLds<TQ> L;
  walk_lds_bind(L, dyn, P.N, P.n_pre);
  L.sh = sh;
  L.qm = qm;
  L.qs = qs;
  L.qa = qa;
  L.wcnt = wcnt;
  L.M = Ms;
  L.S = Ss;
  L.tot = tot;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int R = P.rounds;
  const bool first = R == 0;
  const long long nsw = tree_segments(P.V);
  const long long Bl = P.B;
  // round R - 1 wrote buffer (R - 1) & 1 = (R + 1) & 1; the passes done here
  // reuse it
  Partial* part_in = P.ws_part + ((long long)((R + 1) & 1) * Bl + b) * 2 * P.nseg;
  double* wp_in = P.wpart + ((long long)((R + 1) & 1) * Bl + b) * nsw * 3;
  TreeWalkState st = first ? walk_start() : P.state[(long long)(R & 1) * Bl + b];
  if (first || st.phase < kDraw) {
    if (prefix_staged(P.n_pre, NP)) stage_prefix<NP>(P, b, L, tid);
    const bool bad = stage_tree<DT, kTB>(P, b, L, first, true, tid);
    if (first && bad) {
      for (int c = tid; c < P.N; c += kTB) {
        P.out_path[(long long)b * P.N + c] = -1;
        P.out_tokens[(long long)b * P.N + c] = -1;
      }
      if (tid == 0) P.accept_len[b] = -1;
      st.phase = kDone;
    } else {
      walk<DT, ALIGNED, NP, kTB, true>(P, b, st, !first, L, part_in, wp_in, true);
    }
  }
  if (st.phase != kDraw) return;              // invalid: the outputs are written
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  if (!st.mready) {
    // the walk reached its draw here: the draw's masses, one segment per quarter
    draw_masses<DT, ALIGNED>(P, b, node_row<DT>(P, b, st, st.cn), wid / (kBlock / kWave), TQ,
                             wid & (kBlock / kWave - 1), tid & (kWave - 1));
    __syncthreads();
  }
  __shared__ DrawLds D;
  draw_final<DT, ALIGNED, kTB>(P, b, st, D);
}

template <int DT, bool ALIGNED, int NP>
hipError_t launch_walk_np(const TreeSampleParams& p, hipStream_t s) {
  const long long round_grid = (long long)p.B * pass_units(p);
  if (round_grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const size_t lds = walk_lds_bytes(p.N, prefix_staged(p.n_pre, NP) ? p.n_pre : 0);
  if (lds > (48u << 10)) {
    // large trees: allow the walk kernels more dynamic LDS than the default
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ts_round<DT, ALIGNED, NP>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ts_finish<DT, ALIGNED, NP>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return hipErrorInvalidValue;
  }
  if (p.n_pre > 0) {
    const long long grid = 2LL * p.B * p.n_pre * p.nseg;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_tree_presweep<DT>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
  }
  for (int r = 0; r < p.rounds; ++r)
    hipLaunchKernelGGL((k_ts_round<DT, ALIGNED, NP>), dim3((unsigned)round_grid), dim3(kBlock), lds, s, p, r);
  hipLaunchKernelGGL((k_ts_finish<DT, ALIGNED, NP>), dim3((unsigned)p.B), dim3(kTB), lds, s, p);
  return hipGetLastError();
}

template <int DT, bool ALIGNED>
hipError_t launch_walk_t(const TreeSampleParams& p, hipStream_t s) {
  switch (merge_group(p.nseg)) {
    case 1: return launch_walk_np<DT, ALIGNED, 1>(p, s);
    case 2: return launch_walk_np<DT, ALIGNED, 2>(p, s);
    case 4: return launch_walk_np<DT, ALIGNED, 4>(p, s);
    case 8: return launch_walk_np<DT, ALIGNED, 8>(p, s);
    case 16: return launch_walk_np<DT, ALIGNED, 16>(p, s);
    case 32: return launch_walk_np<DT, ALIGNED, 32>(p, s);
    default: return launch_walk_np<DT, ALIGNED, 64>(p, s);
  }
}

}  // namespace

hipError_t launch_tree_sample(const TreeSampleParams& p, int dt, hipStream_t s) {
  if (p.B < 1 || p.N < 1 || p.N > kTreeMaxNodes || p.V < 1 || (long long)p.V > kMaxSampleVocab || p.n_pre < 0 ||
      p.n_pre > p.N || p.rounds < 0 || p.rounds > kTreeMaxRounds)
    return hipErrorInvalidValue;
  const bool aligned = dt == DT_BF16 ? (p.V % 8 == 0) : (p.V % 4 == 0);
  if (dt == DT_BF16) return aligned ? launch_walk_t<DT_BF16, true>(p, s) : launch_walk_t<DT_BF16, false>(p, s);
  return aligned ? launch_walk_t<DT_F32, true>(p, s) : launch_walk_t<DT_F32, false>(p, s);
}

}  // namespace sv
