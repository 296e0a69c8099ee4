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
// k_tree_presweep (optional): the rows of the first n_pre nodes of every
// sequence, one row segment per workgroup across the whole chip.
// k_tree_walk: one 1024-thread workgroup per sequence.  Beyond the swept
// prefix only the rows of the nodes the walk visits are read: the
// verification needs p at every visited node and q at every visited node
// with children, nothing else.  One CU reduces such a node's two rows in
// about the time the whole chip sweeps a few dozen rows, so the prefix (the
// shallow nodes, which most walks pass through) is swept up front and deeper
// nodes on demand; both use the row sweep's segment reduction, so the
// statistics, and the outputs, do not depend on n_pre.  The workgroup stages
// the tree in LDS, validates it and gathers every node's token logit from its
// parent's target
// and draft rows (one round trip for the whole tree), then walks from the
// root.  At each node: list its children in index order (block scan);
// compute the max and exponential sum of the node's target row (and of its
// draft row if it has children) with the row sweep's segment reduction, four
// segments at a time (one per 256-thread quarter), merged in fp64 exactly as
// the chain sampler merges them; test the children.  A rejection followed by
// another child costs one pass over the node's two rows for W; the final
// draw is one pass for the segment masses, then the inverse CDF inside the
// segment that holds u[0] * total.
#include "sv_kernels.hpp"
#include "sweep_segment.hpp"

#include <limits.h>

namespace sv {

namespace {

constexpr int kTB = 1024;                  // threads per walk workgroup
constexpr int kTW = kTB / kWave;           // waves per walk workgroup
// Elements per thread in one draw segment: four 16-byte vectors per row, so
// the pick's registers (weights plus loads) fit the 128 VGPRs a 1024-thread
// workgroup leaves each lane.
template <int DT>
constexpr int walk_run() { return DT == DT_BF16 ? 32 : 16; }
template <int DT>
constexpr int walk_seg() { return kTB * walk_run<DT>(); }
constexpr int kTChunk = 16;                // segments per LDS reduction round
constexpr int kTQuarters = kTB / kBlock;   // row sweep segments reduced at once
constexpr int kTLdsPart = 64;              // sweep partials per row kept in LDS
constexpr int kTPer = kTreeMaxNodes / kTB; // nodes per thread in the child scan
constexpr int kTMaxSeg = (int)(((long long)kMaxSampleVocab + kTB * 16 - 1) / (kTB * 16));
static_assert(kTreeMaxNodes % kTB == 0, "child scan covers the node range exactly");
static_assert(kTW == kTreeWalkSub && walk_seg<DT_BF16>() == tree_walk_seg(DT_BF16) &&
                  walk_seg<DT_F32>() == tree_walk_seg(DT_F32),
              "the workspace's sub-segment layout matches the walk");

struct WalkLds {
  int par[kTreeMaxNodes];
  int tok[kTreeMaxNodes];
  float u[kTreeMaxNodes];
  float gt[kTreeMaxNodes];   // target logit of node c's token in its parent's row
  float gd[kTreeMaxNodes];   // draft logit of the same
  int kids[kTreeMaxNodes];   // children of the current node, index order
  int xt[kTreeMaxNodes];     // without replacement: tokens of the siblings tried so far
  double seg[kTMaxSeg];      // segment masses of the last pass
  Partial part[2 * kTLdsPart];
  float qm[kTQuarters][kBlock / kWave];
  double qs[kTQuarters][kBlock / kWave];
  int qa[kTQuarters][kBlock / kWave];
  double red[kTChunk * kTW];
  double wtot[kTW];
  int wcnt[kTW];
  int first[kTW];
  float M[2];
  double S[2];
  double total, base, thr;
  double wrem[kTW];
  double sd_all, sd_rem;     // SD passes: draft weight sums over the row, over the tokens kept
  long long y;
  int nk, k, fallback;
};

// Wave wid's share of one segment's draw weights: the wid-th of kTW
// contiguous sub-segments of [e0, e1), lane-interleaved 16-byte vectors, fp64
// accumulation; returns this lane's partial.  F64W: each weight formed in
// fp64 (draw_weight_f64; the W passes of the residual chain), else the final
// draw's fp32 weight (draw_weight, which the pick rescans).  SD (with F64W on
// a residual row): also add this lane's fp64 draft weights e_d to sd[0], and
// those of tokens other than xt[0 .. nx) to sd[1].
template <int DT, bool ALIGNED, bool F64W, bool SD>
__device__ double walk_sub_partial(const DrawRow& R, long long e0, long long e1, const TempConst& tc, int wid,
                                   int lane, double* sd, const int* xt, int nx) {
  static_assert(!SD || F64W, "draft sums come with the fp64 weights");
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int SUB = walk_seg<DT>() / kTW;
  static_assert(SUB / kWave <= 32, "one bit per element of a lane's share");
  const long long s0 = min(e0 + (long long)wid * SUB, e1);
  const long long s1 = min(s0 + SUB, e1);
  double acc = 0.0;
  // SD: bit j set when the lane's j-th element of this sub-segment is a
  // removed token (element order of the loops below)
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
    constexpr int KV = SUB / EPV / kWave;
    const int nvec = (int)((s1 - s0) / EPV);
    if (nvec <= 0) return 0.0;
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(R.t + s0 * ES, (uint32_t)nvec * 16u);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(R.d + s0 * ES, (uint32_t)nvec * 16u);
    v4i vt[KV], vd[KV];
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      const uint32_t off = (uint32_t)min(k * kWave + lane, nvec - 1) * 16u;
      vt[k] = load16(rt, off);
      if (R.resid) vd[k] = load16(rd, off);
    }
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      if (k * kWave + lane >= nvec) continue;
      float zt[EPV], zd[EPV];
      unpack<DT>(vt[k], zt);
      if (R.resid) unpack<DT>(vd[k], zd);
#pragma unroll
      for (int i = 0; i < EPV; ++i) {
        if constexpr (SD) {
          const double ed = exp_rel_f64<DT>(zd[i], R.Md, tc);
          acc += fmax(fma(-R.rho, ed, exp_rel_f64<DT>(zt[i], R.Mt, tc)), 0.0);
          sd[0] += ed;
          if (!((xm >> (k * EPV + i)) & 1u)) sd[1] += ed;
        } else if constexpr (F64W) {
          acc += draw_weight_f64<DT>(R, zt[i], R.resid ? zd[i] : 0.f, tc);
        } else {
          acc += (double)draw_weight<DT>(R, zt[i], R.resid ? zd[i] : 0.f, tc);
        }
      }
    }
  } else {
    int j = 0;
    for (long long e = s0 + lane; e < s1; e += kWave, ++j) {
      const float zt = load_elem<DT>(R.t, e);
      const float zd = R.resid ? load_elem<DT>(R.d, e) : 0.f;
      if constexpr (SD) {
        const double ed = exp_rel_f64<DT>(zd, R.Md, tc);
        acc += fmax(fma(-R.rho, ed, exp_rel_f64<DT>(zt, R.Mt, tc)), 0.0);
        sd[0] += ed;
        if (!((xm >> j) & 1u)) sd[1] += ed;
      } else if constexpr (F64W) {
        acc += draw_weight_f64<DT>(R, zt, zd, tc);
      } else {
        acc += (double)draw_weight<DT>(R, zt, zd, tc);
      }
    }
  }
  return acc;
}

// Segment masses of the draw row into L.seg and their total (segment order,
// fixed combination order throughout); if sub is not null, also every
// segment's kTW sub-segment masses into sub[segment * kTW + sub-segment]
// (global memory, read back by this workgroup after a barrier).  Every
// thread of the block calls it.  F64W and SD as in walk_sub_partial; SD
// leaves the draft row's fp64 weight sums (lanes, then waves, in a fixed
// order) in L.sd_all (every token) and L.sd_rem (every token but xt[0 .. nx)).
template <int DT, bool ALIGNED, bool F64W, bool SD = false>
__device__ double mass_pass(const DrawRow& R, long long V, const TempConst& tc, WalkLds& L, int tid,
                            double* sub, const int* xt = nullptr, int nx = 0) {
  constexpr int SEG = walk_seg<DT>();
  const int lane = tid & (kWave - 1), wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int nseg = (int)((V + SEG - 1) / SEG);
  double sd[2] = {0.0, 0.0};
  for (int s0 = 0; s0 < nseg; s0 += kTChunk) {
    const int s1 = min(s0 + kTChunk, nseg);
    for (int s = s0; s < s1; ++s) {
      const long long e0 = (long long)s * SEG;
      const long long e1 = e0 + SEG < V ? e0 + SEG : V;
      const double a = wave_sum(walk_sub_partial<DT, ALIGNED, F64W, SD>(R, e0, e1, tc, wid, lane, sd, xt, nx));
      if (lane == 0) {
        L.red[(s - s0) * kTW + wid] = a;
        if (sub != nullptr) sub[s * kTW + wid] = a;
      }
    }
    __syncthreads();
    if (tid < s1 - s0) {
      double t = 0.0;
      for (int w = 0; w < kTW; ++w) t += L.red[tid * kTW + w];
      L.seg[s0 + tid] = t;
    }
    __syncthreads();
  }
  if constexpr (SD) {
    const double all = wave_sum(sd[0]), rem = wave_sum(sd[1]);
    if (lane == 0) {
      L.wtot[wid] = all;
      L.wrem[wid] = rem;
    }
    __syncthreads();
  }
  if (wid == 0) {
    double tot = 0.0;
    for (int c0 = 0; c0 < nseg; c0 += kWave) tot += wave_sum(c0 + lane < nseg ? L.seg[c0 + lane] : 0.0);
    if (lane == 0) L.total = tot;
    if constexpr (SD) {
      if (lane == 0) {
        double ta = 0.0, tr = 0.0;
        for (int w = 0; w < kTW; ++w) {
          ta += L.wtot[w];
          tr += L.wrem[w];
        }
        L.sd_all = ta;
        L.sd_rem = tr;
      }
    }
  }
  __syncthreads();
  return L.total;
}

// Inverse-CDF draw over the masses the last mass_pass left in L.seg and in
// sub: the first element whose cumulative weight exceeds thr, or the last
// element with positive weight if rounding leaves none.  The segment, then
// its sub-segment, are located with wave scans; the block rescans that
// sub-segment, RUN elements per thread.
template <int DT, bool ALIGNED>
__device__ long long walk_pick(const DrawRow& R, long long V, double thr, const TempConst& tc, WalkLds& L,
                               int tid, const double* sub) {
  constexpr int SEG = walk_seg<DT>();
  constexpr int SUB = SEG / kTW;
  constexpr int RUN = SUB / kTB;
  static_assert(RUN >= 1 && RUN * kTB == SUB, "one sub-segment per block rescan");
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  const int nseg = (int)((V + SEG - 1) / SEG);
  if (wid == 0) {
    double base;
    int fb;
    const int k = locate_segment(L.seg, nseg, thr, lane, &base, &fb);
    double base2;
    int fb2;
    const int k2 = locate_segment(sub + (long long)k * kTW, kTW, thr - base, lane, &base2, &fb2);
    if (lane == 0) {
      L.k = k * kTW + k2;
      L.base = base + base2;
      L.fallback = fb | fb2;
      L.y = -1;
    }
  }
  __syncthreads();
  const long long kb = (long long)__builtin_amdgcn_readfirstlane(L.k) * SUB;
  const long long ke = kb + SUB < V ? kb + SUB : V;
  const long long rb0 = kb + (long long)tid * RUN;
  const long long rb = rb0 < ke ? rb0 : ke;
  const long long re = rb + RUN < ke ? rb + RUN : ke;
  float w[RUN];
#pragma unroll
  for (int e = 0; e < RUN; ++e) {
    const long long ee = rb + e;
    float v = 0.f;
    if (ee < re) {
      const float zt = load_elem<DT>(R.t, ee);
      const float zd = R.resid ? load_elem<DT>(R.d, ee) : 0.f;
      v = draw_weight<DT>(R, zt, zd, tc);
    }
    w[e] = v;
  }
  double T4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int e = 0; e < RUN; ++e) T4[e & 3] += (double)w[e];
  const double T = (T4[0] + T4[1]) + (T4[2] + T4[3]);
  const double incl = wave_incl_scan(T, lane);
  if (lane == kWave - 1) L.wtot[wid] = incl;
  __syncthreads();
  double wbase = 0.0;
  for (int v = 0; v < wid; ++v) wbase += L.wtot[v];
  const double excl = L.base + wbase + (incl - T);
  const bool cross = !L.fallback && T > 0.0 && excl + T > thr;
  const unsigned long long mc = __ballot(cross);
  const unsigned long long mp = __ballot(T > 0.0);
  if (lane == 0) L.first[wid] = mc ? wid * kWave + (int)__ffsll((long long)mc) - 1 : INT_MAX;
  __syncthreads();
  int first = INT_MAX;
  for (int v = 0; v < kTW; ++v) first = min(first, L.first[v]);
  __syncthreads();
  if (lane == 0) L.first[wid] = mp ? wid * kWave + 63 - (int)__clzll((long long)mp) : -1;
  __syncthreads();
  int lastpos = -1;
  for (int v = 0; v < kTW; ++v) lastpos = max(lastpos, L.first[v]);
  const int who = first != INT_MAX ? first : lastpos;
  if (tid == who) {
    double acc = excl;
    int y = -1, ylast = -1;
#pragma unroll
    for (int e = 0; e < RUN; ++e) {
      if (w[e] > 0.f) {
        acc += (double)w[e];
        ylast = e;
        if (y < 0 && first != INT_MAX && acc > thr) y = e;
      }
    }
    L.y = rb + (y >= 0 ? y : ylast);
  }
  __syncthreads();
  return L.y;
}

// Test value of the k-th child: max(0, p(x)/q(x) - c) / W, with p(x)/q(x) =
// 2^((z_t(x) - M_t) c64 - (z_d(x) - M_d) c64) S_d / S_t in fp64; p(x) = 0
// gives 0, q(x) = 0 < p(x) gives +inf.  For c = 0, W = 1 this is the chain
// sampler's ratio bit for bit.
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
  const Partial pp = sweep_segment<DT, 1>(base, b * P.N + n, P.V, s, P.seg_vecs, P.tc, tid, wid, sh_m, sh_s, sh_a,
                                          -1, nullptr);
  if (tid == 0) P.pre_part[row * P.nseg + s] = pp;
}

template <int DT, bool ALIGNED, int NP>
__global__ __launch_bounds__(kTB) void k_tree_walk(TreeSampleParams P) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  __shared__ WalkLds L;
  // wid is wave-uniform; readfirstlane keeps what derives from it (the row
  // a quarter sweeps, its buffer descriptors) in scalar registers
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int b = blockIdx.x;
  const int N = P.N;
  const long long V = P.V;
  const long long row0 = (long long)b * N;
  const char* tgt = static_cast<const char*>(P.tgt);
  const char* drf = static_cast<const char*>(P.drf);
  const int* par_g = P.parent + (long long)b * P.parent_stride;
  int* out_path = P.out_path + row0;
  int* out_tok = P.out_tokens + row0;

  // stage and validate the tree; gather each node's token logit from its
  // parent's rows (only for nodes whose parent and token are in range)
  int bad = 0;
  for (int c = tid; c < N; c += kTB) {
    const int p = par_g[c];
    const int x = P.tokens[row0 + c];
    const bool pok = c == 0 ? p == -1 : (p >= 0 && p < c);
    const bool xok = c == 0 || (x >= 0 && (long long)x < V);
    float zt = 0.f, zd = 0.f;
    if (c > 0 && pok && xok) {
      zt = load_elem<DT>(tgt, (row0 + p) * V + x);
      zd = load_elem<DT>(drf, (row0 + p) * V + x);
    }
    bad |= !(pok && xok);
    L.par[c] = p;
    L.tok[c] = x;
    L.u[c] = P.unif[row0 + c];
    L.gt[c] = zt;
    L.gd[c] = zd;
  }
  if (__syncthreads_or(bad)) {
    for (int c = tid; c < N; c += kTB) {
      out_path[c] = -1;
      out_tok[c] = -1;
    }
    if (tid == 0) P.accept_len[b] = -1;
    return;                                   // uniform
  }

  int n = 0, d = 0;
  DrawRow R;
  double c_fb = 0.0;                          // the law to fall back to if the draw row has no mass
  const int nseg = P.nseg;
  Partial* part = nseg <= kTLdsPart ? L.part : P.ws_part + (long long)b * 2 * nseg;
  const int q = wid / (kBlock / kWave), tq = tid & (kBlock - 1), wq = wid & (kBlock / kWave - 1);
  for (;;) {
    // children of n in index order: block scan over kTPer nodes per thread
    int flag[kTPer];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kTPer; ++j) {
      const int c = tid * kTPer + j;
      flag[j] = c > n && c < N && L.par[c] == n;
      cnt += flag[j];
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
    for (int v = 0; v < kTW; ++v) {
      const int t = L.wcnt[v];
      if (v < wid) pos += t;
      nk += t;
    }
#pragma unroll
    for (int j = 0; j < kTPer; ++j)
      if (flag[j]) L.kids[pos++] = tid * kTPer + j;
    // segment partials of node n's target row, and of its draft row if it
    // has children: swept up front for n < n_pre, else here, kTQuarters
    // segments per round, one per quarter (a quarter past the last unit
    // reduces an empty segment, with no loads)
    const bool pre = n < P.n_pre;
    const int units = pre ? 0 : nseg * (nk > 0 ? 2 : 1);
    for (int u0 = 0; u0 < units; u0 += kTQuarters) {
      const int u = u0 + q;
      const bool drow = u >= nseg && u < units;
      const int s = u < units ? (drow ? u - nseg : u) : nseg;
      const Partial pp = sweep_segment<DT, 1>(drow ? drf : tgt, row0 + n, V, s, P.seg_vecs, P.tc, tq, wq, L.qm[q],
                                              L.qs[q], L.qa[q], -1, nullptr);
      if (tq == 0 && u < units) part[u] = pp;
    }
    __syncthreads();
    if (wid < 2 && (wid == 0 || nk > 0)) {
      float M;
      double S;
      int a;
      const Partial* src = part + wid * nseg;
      if (pre) src = P.pre_part + ((wid == 0 ? 0 : (long long)P.B * P.n_pre) + (long long)b * P.n_pre + n) * nseg;
      merge_partials<1, NP>(src, nseg, P.tc, lane & (NP - 1), &M, &S, &a);
      if (lane == 0) {
        L.M[wid] = M;
        L.S[wid] = S;
      }
    }
    __syncthreads();
    const float Mt = L.M[0], Md = L.M[1];
    const double St = L.S[0], Sd = L.S[1];
    R.t = tgt + (row0 + n) * V * ES;
    R.d = drf + (row0 + n) * V * ES;
    R.Mt = Mt;
    R.Md = Md;
    if (nk == 0) {                            // leaf: bonus token from p
      set_rho(R, 0.0, St, Sd);
      c_fb = 0.0;
      break;
    }
    // every thread evaluates the same tests on the same LDS values, so the
    // decisions (and the passes between them) are block-uniform
    double cc = 0.0, W = 1.0;
    double Rk = 1.0;                          // without replacement: R_k of the child being tested
    int chosen = -1;
    for (int i = 0; i < nk; ++i) {
      const int ci = L.kids[i];
      double r = child_ratio(L.gt[ci], L.gd[ci], Mt, St, Md, Sd, cc, W, P.tc);
      if (P.distinct && i > 0) {
        int hit = 0;
        for (int j = tid; j < i; j += kTB) hit |= L.tok[L.kids[j]] == L.tok[ci];
        const bool dup = __syncthreads_or(hit) != 0;
        r = dup ? 0.0 : (Rk > 0.0 ? Rk * r : (r > 0.0 ? __builtin_huge_val() : 0.0));
      }
      if ((double)L.u[ci] < r) {
        chosen = ci;
        break;
      }
      const double cn = Rk > 0.0 ? cc + W / Rk : cc;
      if (i + 1 == nk) {                      // every child rejected
        set_rho(R, cn, St, Sd);
        c_fb = cc;
        break;
      }
      set_rho(R, cn, St, Sd);
      if (!(Rk > 0.0)) continue;              // the residual is the current law: (c, W) stay
      // W of the next residual: fp64 weights, so a test's value
      // max(0, p(x)/q(x) - c)/W carries no fp32 rounding of the residual;
      // without replacement the same pass sums the draft row's weights
      double Wn;
      if (P.distinct) {
        for (int j = tid; j <= i; j += kTB) L.xt[j] = L.tok[L.kids[j]];
        __syncthreads();
        Wn = mass_pass<DT, ALIGNED, true, true>(R, V, P.tc, L, tid, nullptr, L.xt, i + 1) / St;
        Rk = L.sd_all > 0.0 ? L.sd_rem / L.sd_all : 0.0;
      } else {
        Wn = mass_pass<DT, ALIGNED, true>(R, V, P.tc, L, tid, nullptr) / St;
      }
      if (Wn > 0.0) {
        cc = cn;
        W = Wn;
      }
    }
    if (chosen < 0) break;
    if (tid == 0) {
      out_path[d] = chosen;
      out_tok[d] = L.tok[chosen];
    }
    ++d;
    n = chosen;
    __syncthreads();                          // LDS of this node is read before it is reused
  }

  // final draw from R (fallback: the law before the last residual, then p)
  double* const sub = P.ws_sub + (long long)b * tree_walk_subsegments(P.V, DT);
  double total = mass_pass<DT, ALIGNED, false>(R, V, P.tc, L, tid, sub);
  if (!(total > 0.0) && R.resid) {
    set_rho(R, c_fb, L.S[0], L.S[1]);
    total = mass_pass<DT, ALIGNED, false>(R, V, P.tc, L, tid, sub);
  }
  if (!(total > 0.0) && R.resid) {
    set_rho(R, 0.0, L.S[0], L.S[1]);
    total = mass_pass<DT, ALIGNED, false>(R, V, P.tc, L, tid, sub);
  }
  const long long y = walk_pick<DT, ALIGNED>(R, V, (double)L.u[0] * total, P.tc, L, tid, sub);
  for (int c = tid; c < N; c += kTB) {
    if (c >= d) out_path[c] = -1;
    if (c > d) out_tok[c] = -1;
  }
  if (tid == 0) {
    out_tok[d] = (int)y;
    P.accept_len[b] = d;
  }
}

template <int DT, bool ALIGNED, int NP>
hipError_t launch_walk_np(const TreeSampleParams& p, hipStream_t s) {
  if (p.n_pre > 0) {
    const long long grid = 2LL * p.B * p.n_pre * p.nseg;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_tree_presweep<DT>), dim3((unsigned)grid), dim3(kBlock), 0, s, p);
  }
  hipLaunchKernelGGL((k_tree_walk<DT, ALIGNED, NP>), dim3((unsigned)p.B), dim3(kTB), 0, s, p);
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
      p.n_pre > p.N)
    return hipErrorInvalidValue;
  const bool aligned = dt == DT_BF16 ? (p.V % 8 == 0) : (p.V % 4 == 0);
  if (dt == DT_BF16) return aligned ? launch_walk_t<DT_BF16, true>(p, s) : launch_walk_t<DT_BF16, false>(p, s);
  return aligned ? launch_walk_t<DT_F32, true>(p, s) : launch_walk_t<DT_F32, false>(p, s);
}

}  // namespace sv
