// EAGLE-2 dynamic draft tree: one expansion depth (spec_tree_expand) and
// the final re-ranking with the tree-attention mask (spec_tree_build).
//
// Pages: "EAGLE math", "EAGLE-2: dynamic draft trees" (grow the tree
// greedily by expanding the nodes with the highest cumulative draft
// probability, prune, re-rank which candidates to keep; the verified node
// count stays fixed; a tree attention mask scores every candidate in one
// pass); "EAGLE-3 speculative decoding review", "EAGLE-2: Does Every Context
// Need the Same Draft Tree?" (a node sees the shared prefix and its own
// ancestors only) and "The Complete EAGLE-3 Inference Process" (2. Generate
// a Draft Tree).
//
// A node's score is its cumulative draft log-probability (fp64), the root 0.
//
//  k_topk_sweep  one workgroup per (frontier row, 8192-logit segment): the
//                segment max, the sum of 2^((z - max) c) and its k largest
//                logits (equal logits: lower index first).  Each lane keeps
//                its own max, exp-sum and two best logits in one pass over its
//                32 registers; one wave then picks the segment's top k from
//                the 256 lanes' pairs in k rounds of a wave argmax.  A lane's
//                third best matters only once both of its candidates are
//                taken; it is then rescanned from the row.
//  k_expand      one workgroup per sequence, one wave per frontier row:
//                merges each row's segments (max, fp64 sum, the k best of the segment lists),
//                forms log q = ((z - M) c - log2 S) ln 2 for the k tokens,
//                writes the children to the node table (frontier slot f,
//                rank r at table position off + f k + r) and picks the next
//                frontier, the K_out best children by (score desc, position
//                asc), by rank counting.
//  k_tree_build  one workgroup per sequence: ranks the drafted nodes by
//                (score desc, depth asc, index asc) and keeps the best M,
//                orders the kept nodes by (depth, score desc, index), remaps
//                parents and writes the ancestor bitmask rows.  A table that
//                breaks the invariants the expansion keeps (parents before
//                children, depth = parent depth + 1, kept parents) is
//                reported with n = -1.
// The sweep streams every frontier row once: HBM-bound like the verify
// sweep.  The other two kernels touch kilobytes.
#include "sv_kernels.hpp"

#include <limits.h>

namespace sv {

namespace {

constexpr int kTreeRun = 32;  // logits per lane per segment
constexpr int kExpandBlock = 1024;  // one wave per frontier row (up to 16 at a time)
constexpr int kBuildBlock = 1024;

__device__ __forceinline__ bool topk_before(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

// (v, i) < (w, j) in the candidate order: larger value first, then lower index
__device__ __forceinline__ bool ord_lt(float v, int i, float w, int j) { return (v > w) | ((v == w) & (i < j)); }

template <int DT, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void k_topk_sweep(TreeExpandParams P) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int KV = kTreeRun / EPV;
  __shared__ float sh_lm[kBlock], sh_ls[kBlock], sh_c1v[kBlock], sh_c2v[kBlock];
  __shared__ int sh_c1i[kBlock], sh_c2i[kBlock];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const long long row = blockIdx.x / P.nseg;
  const int s = (int)(blockIdx.x - row * P.nseg);
  TopkPart* out = P.part + blockIdx.x;
  const long long V = P.V;
  const float NINF = -__builtin_huge_valf();
  if (P.frontier[row] < 0) {
    if (tid < kTopkMax) {
      out->v[tid] = NINF;
      out->idx[tid] = INT_MAX;
    }
    if (tid == 0) {
      out->m = NINF;
      out->s = 0.f;
    }
    return;
  }
  const long long e0 = (long long)s * P.seg_elems;
  const long long e1 = e0 + P.seg_elems < V ? e0 + P.seg_elems : V;
  const char* rowp = static_cast<const char*>(P.logits) + row * V * ES;
  // This lane's elements: register q holds element e0 + pos(q) with
  // pos(q) = ((q / EPV) * kBlock + tid) * EPV + q % EPV (vector k = q / EPV of
  // the lane; coalesced), so q order is index order.  Elements past the
  // segment read as -inf and are never taken (all comparisons are strict).
  float z[kTreeRun];
  int nin;  // registers 0 .. nin-1 hold this lane's elements of the segment
  if constexpr (ALIGNED) {
    const int nvec = (int)((e1 - e0) / EPV);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(rowp + e0 * ES, (uint32_t)nvec * 16u);
    v4i vv[KV];
#pragma unroll
    for (int k = 0; k < KV; ++k) vv[k] = load16(r, (uint32_t)min(k * kBlock + tid, nvec - 1) * 16u);
    int nv = 0;
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      unpack<DT>(vv[k], z + k * EPV);
      const bool in = k * kBlock + tid < nvec;
      nv += in ? 1 : 0;
      if (!in)
#pragma unroll
        for (int i = 0; i < EPV; ++i) z[k * EPV + i] = NINF;
    }
    nin = nv * EPV;
  } else {
    int n = 0;
#pragma unroll
    for (int k = 0; k < KV; ++k)
#pragma unroll
      for (int i = 0; i < EPV; ++i) {
        const long long e = e0 + (long long)(k * kBlock + tid) * EPV + i;
        z[k * EPV + i] = e < e1 ? load_elem<DT>(rowp, e) : NINF;
        n += e < e1 ? 1 : 0;
      }
    nin = n;
  }
  auto gidx = [&](int q) { return (int)(e0 + ((q / EPV) * kBlock + tid) * EPV + (q % EPV)); };
  // one pass: the lane's two best elements (value desc, then q asc); q = -1
  // marks an empty slot.  The first two elements seed the pair, so strict
  // comparisons settle ties by position from then on; elements past nin are
  // -inf and never displace anything.
  float b1v = NINF, b2v = NINF;
  int b1q = -1, b2q = -1;
  if (nin >= 1) {
    b1v = z[0];
    b1q = 0;
  }
  if (nin >= 2) {
    const bool sw = z[1] > z[0];
    b1v = sw ? z[1] : z[0];
    b1q = sw ? 1 : 0;
    b2v = sw ? z[0] : z[1];
    b2q = sw ? 0 : 1;
  }
#pragma unroll
  for (int q = 2; q < kTreeRun; ++q) {
    const bool c1 = z[q] > b1v;
    const bool c2 = z[q] > b2v;
    b2v = c1 ? b1v : (c2 ? z[q] : b2v);
    b2q = c1 ? b1q : (c2 ? q : b2q);
    b1v = c1 ? z[q] : b1v;
    b1q = c1 ? q : b1q;
  }
  // lane sum of 2^((z - m) c) relative to its own max m = b1v
  const float c = P.tc.c_hi;
  float ls = 0.f;
  if (b1v > NINF) {
#pragma unroll
    for (int q = 0; q < kTreeRun; ++q) ls += __builtin_amdgcn_exp2f((z[q] - b1v) * c);
  }
  // publish the lane's (max, sum) and its two candidates
  sh_lm[tid] = b1v;
  sh_ls[tid] = ls;
  sh_c1v[tid] = b1v;
  sh_c1i[tid] = b1q >= 0 ? gidx(b1q) : INT_MAX;
  sh_c2v[tid] = b2v;
  sh_c2i[tid] = b2q >= 0 ? gidx(b2q) : INT_MAX;
  __syncthreads();
  if (wid != 0) return;
  // wave 0: segment (max, sum) from the 256 lanes
  float m4 = NINF;
#pragma unroll
  for (int j = 0; j < 4; ++j) m4 = fmaxf(m4, sh_lm[lane + j * kWave]);
  const float M = wave_max(m4);
  float s4 = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lm = sh_lm[lane + j * kWave];
    s4 += lm > NINF ? sh_ls[lane + j * kWave] * __builtin_amdgcn_exp2f((lm - M) * c) : 0.f;
  }
  const double S = wave_sum((double)s4);
  // wave 0: the segment's top k.  Lane l owns source lanes l + 64 j (j < 4)
  // and their two candidates; a source lane's third best is only needed when
  // both of its candidates were taken, and is then rescanned from the row.
  float cv[8];
  int ci[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cv[2 * j] = sh_c1v[lane + j * kWave];
    ci[2 * j] = sh_c1i[lane + j * kWave];
    cv[2 * j + 1] = sh_c2v[lane + j * kWave];
    ci[2 * j + 1] = sh_c2i[lane + j * kWave];
  }
  for (int r = 0; r < P.k; ++r) {
    float bv = NINF;
    int bi = INT_MAX, bs = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const bool better = ci[t] != INT_MAX && (bi == INT_MAX || ord_lt(cv[t], ci[t], bv, bi));
      bv = better ? cv[t] : bv;
      bi = better ? ci[t] : bi;
      bs = better ? t : bs;
    }
    const float gv = wave_max(bi == INT_MAX ? NINF : bv);
    const int gi = wave_min(bi != INT_MAX && bv == gv ? bi : INT_MAX);
    if (lane == 0) {
      out->v[r] = gv;
      out->idx[r] = gi;
    }
    if (gi != INT_MAX && bi == gi) {
      // consumed: a first candidate leaves its second in play; a second
      // candidate is replaced by the source lane's next best
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t != bs) continue;
        if ((t & 1) == 0) {
          ci[t] = INT_MAX;
        } else {
          const int src = lane + (t >> 1) * kWave;   // source thread of the segment
          float v = NINF;
          int vi = INT_MAX;
          for (int q = 0; q < kTreeRun; ++q) {
            const long long e = e0 + (long long)((q / EPV) * kBlock + src) * EPV + (q % EPV);
            if (e >= e1) continue;
            const float zq = load_elem<DT>(rowp, e);
            const int ei = (int)e;
            if (ord_lt(gv, gi, zq, ei) && (vi == INT_MAX || ord_lt(zq, ei, v, vi))) {
              v = zq;
              vi = ei;
            }
          }
          cv[t] = v;
          ci[t] = vi;
        }
      }
    }
  }
  if (lane == 0) {
    out->m = M;
    out->s = (float)S;
  }
}

__global__ __launch_bounds__(kExpandBlock) void k_expand(TreeExpandParams P) {
  __shared__ double sc[kCandMax];
  __shared__ int sh_count;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int b = blockIdx.x;
  const int k = P.k;
  const long long tb = (long long)b * P.cap;
  const int ncand = P.K_in * k;
  if (tid == 0) sh_count = 0;
  const int nw = blockDim.x / kWave;
  for (int f = wid; f < P.K_in; f += nw) {
    const long long row = (long long)b * P.K_in + f;
    const int pn = P.frontier[row];
    if (pn < 0 || pn >= P.off) {  // empty slot (entries past the written table count as empty)
      for (int r = lane; r < k; r += kWave) {
        const long long pos = tb + P.off + (long long)f * k + r;
        P.parent[pos] = -1;
        P.token[pos] = -1;
        P.score[pos] = -__builtin_huge_val();
        P.depth[pos] = -1;
        sc[f * k + r] = -__builtin_huge_val();
      }
      continue;
    }
    const TopkPart* pr = P.part + row * P.nseg;
    // row max and fp64 sum over the segments
    float m = -__builtin_huge_valf();
    for (int t = lane; t < P.nseg; t += kWave) m = fmaxf(m, pr[t].m);
    const float M = wave_max(m);
    double S = 0.0;
    for (int t = lane; t < P.nseg; t += kWave)
      if (pr[t].s > 0.f) S += (double)pr[t].s * exp2_f64(((double)pr[t].m - (double)M) * P.tc.c64);
    S = wave_sum(S);
    const double l2S = log2(S);
    const double ps = P.score[tb + pn];
    const int pd = P.depth[tb + pn];
    // the k best of the segments' lists (each sorted, best first), k rounds
    float pv = __builtin_huge_valf();
    int pi = -1;
    const bool onefold = P.nseg <= kWave;
    // one segment per lane: its list in registers, head first
    float hv[kTopkMax];
    int hi[kTopkMax];
    if (onefold) {
#pragma unroll
      for (int j = 0; j < kTopkMax; ++j) {
        const bool in = lane < P.nseg && j < k;
        hv[j] = in ? pr[in ? lane : 0].v[j] : -__builtin_huge_valf();
        hi[j] = in ? pr[in ? lane : 0].idx[j] : INT_MAX;
      }
    }
    for (int r = 0; r < k; ++r) {
      float v = -__builtin_huge_valf();
      int ix = INT_MAX;
      if (onefold) {
        v = hv[0];
        ix = hi[0];
      } else {
        // more segments than lanes: each lane scans its segments' lists for
        // the best candidate ordered after the previous winner
        const int nl = P.nseg * kTopkMax;
        for (int c = lane; c < nl; c += kWave) {
          const int t = c / kTopkMax, j = c % kTopkMax;
          if (j >= k) continue;
          const float cv = pr[t].v[j];
          const int ci = pr[t].idx[j];
          if (ci != INT_MAX && topk_before(pv, pi, cv, ci) && topk_before(cv, ci, v, ix)) {
            v = cv;
            ix = ci;
          }
        }
      }
      const float wv = wave_max(v);
      const int wi = wave_min(v == wv ? ix : INT_MAX);
      pv = wv;
      pi = wi;
      if (onefold && ix == wi && wi != INT_MAX) {
        // this lane's head was taken: shift its list up by one
#pragma unroll
        for (int j = 0; j + 1 < kTopkMax; ++j) {
          hv[j] = hv[j + 1];
          hi[j] = hi[j + 1];
        }
        hv[kTopkMax - 1] = -__builtin_huge_valf();
        hi[kTopkMax - 1] = INT_MAX;
      }
      if (lane == 0) {
        const long long pos = tb + P.off + (long long)f * k + r;
        double lq = -__builtin_huge_val();
        if (wv > -__builtin_huge_valf()) lq = (((double)wv - (double)M) * P.tc.c64 - l2S) * kLn2;
        const double sv = ps + lq;
        P.parent[pos] = wi == INT_MAX ? -1 : pn;
        P.token[pos] = wi == INT_MAX ? -1 : wi;
        P.score[pos] = wi == INT_MAX ? -__builtin_huge_val() : sv;
        P.depth[pos] = wi == INT_MAX ? -1 : pd + 1;
        sc[f * k + r] = wi == INT_MAX ? -__builtin_huge_val() : sv;
      }
    }
  }
  __syncthreads();
  // next frontier: rank among the children with a finite score
  for (int c = tid; c < ncand; c += blockDim.x) {
    const double v = sc[c];
    if (!(v > -__builtin_huge_val())) continue;
    int rank = 0;
    for (int c2 = 0; c2 < ncand; ++c2) {
      const double w = sc[c2];
      rank += (w > v || (w == v && c2 < c)) ? 1 : 0;
    }
    atomicAdd(&sh_count, 1);
    if (rank < P.K_out) P.next_frontier[(long long)b * P.K_out + rank] = P.off + c;
  }
  __syncthreads();
  for (int t = sh_count + tid; t < P.K_out; t += blockDim.x) P.next_frontier[(long long)b * P.K_out + t] = -1;
}

// One node of the table as the build kernel ranks it.
struct NodeRec {
  double s;   // score
  int key;    // depth * kBuildMaxNodes + table index
  int flag;   // counted (drafted, then kept)
};

// For this thread's node (score ms, key mk): how many nodes q < n with
// flag != 0 come before it in the order lt.  Every thread reads the same
// record at a time (an LDS broadcast), eight records per wait.
template <class Lt>
__device__ int count_before(int n, const NodeRec* rec, double ms, int mk, Lt lt) {
  int cnt = 0;
  int q = 0;
  for (; q + 8 <= n; q += 8) {
    NodeRec r[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = rec[q + t];
#pragma unroll
    for (int t = 0; t < 8; ++t) cnt += (r[t].flag && lt(r[t].s, r[t].key, ms, mk)) ? 1 : 0;
  }
  for (; q < n; ++q) {
    const NodeRec r = rec[q];
    cnt += (r.flag && lt(r.s, r.key, ms, mk)) ? 1 : 0;
  }
  return cnt;
}

__global__ __launch_bounds__(kBuildBlock) void k_tree_build(TreeBuildParams P) {
  extern __shared__ double tb_lds[];
  const int n = P.n_nodes, tid = threadIdx.x, b = blockIdx.x;
  NodeRec* rec = reinterpret_cast<NodeRec*>(tb_lds);  // [n]
  int* par = reinterpret_cast<int*>(rec + n);         // [n] table parent
  int* pos = par + n;                                 // [n] output position or -1
  int* opar = pos + n;                                // [M + 1] output parent
  const long long tb = (long long)b * P.cap;
  const int NO = P.M + 1;
  const double NINF = -__builtin_huge_val();
  constexpr int kPer = kBuildMaxNodes / kBuildBlock;
  __shared__ int sh_nk;
  if (tid == 0) sh_nk = 0;
  for (int p = tid; p < n; p += kBuildBlock) {
    rec[p].s = P.score[tb + p];
    par[p] = P.parent[tb + p];
    pos[p] = P.depth[tb + p];  // depth, for now
  }
  __syncthreads();
  // drafted nodes, keys, and the invariants of a table the expansion wrote
  bool bad = false;
  for (int p = tid; p < n; p += kBuildBlock) {
    const int q = par[p];
    const bool drafted = p >= 1 && q >= 0 && rec[p].s > NINF;
    rec[p].flag = drafted ? 1 : 0;
    rec[p].key = pos[p] * kBuildMaxNodes + p;
    if (p == 0) bad |= q != -1 || pos[0] != 0;
    else if (drafted)
      bad |= q >= p || (q != 0 && !(par[q] >= 0 && rec[q].s > NINF)) || pos[p] != pos[q] + 1 || pos[p] < 1 ||
             pos[p] >= (1 << 19);
  }
  bad = __syncthreads_or(bad);
  if (!bad) {
    // keep the M best drafted nodes by (score desc, depth asc, index asc)
    int kept[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int p = tid + u * kBuildBlock;
      kept[u] = 0;
      if (p >= n) continue;
      if (p == 0) {
        kept[u] = 1;
        continue;
      }
      const NodeRec me = rec[p];
      if (!me.flag) continue;
      const int rank = count_before(n, rec, me.s, me.key,
                                    [](double s, int kk, double ms, int mk) { return s > ms || (s == ms && kk < mk); });
      kept[u] = rank < P.M ? 1 : 0;
    }
    __syncthreads();
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int p = tid + u * kBuildBlock;
      if (p < n) {
        rec[p].flag = kept[u];
        cnt += (p != 0 && kept[u]) ? 1 : 0;
      }
    }
    if (cnt) atomicAdd(&sh_nk, cnt);
    __syncthreads();
    // kept nodes' parents must be kept (true for scores the expansion wrote)
    bool open = false;
    for (int p = tid; p < n; p += kBuildBlock)
      if (p != 0 && rec[p].flag && !rec[par[p]].flag) open = true;
    bad = __syncthreads_or(open);
  }
  const int nkept = sh_nk;
  const int nout = bad ? 0 : 1 + nkept;
  if (!bad) {
    // output position: (depth asc, score desc, index asc) among the kept
    int o[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int p = tid + u * kBuildBlock;
      o[u] = -1;
      if (p >= n) continue;
      const NodeRec me = rec[p];
      if (!me.flag) continue;
      o[u] = count_before(n, rec, me.s, me.key, [](double s, int kk, double ms, int mk) {
        const int d = kk / kBuildMaxNodes, md = mk / kBuildMaxNodes;
        return d < md || (d == md && (s > ms || (s == ms && kk < mk)));
      });
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int p = tid + u * kBuildBlock;
      if (p < n) pos[p] = o[u];
    }
    __syncthreads();
    for (int p = tid; p < n; p += kBuildBlock) {
      const int oo = pos[p];
      if (oo < 0) continue;
      const long long ob = (long long)b * NO + oo;
      const int po = p == 0 ? -1 : pos[par[p]];
      opar[oo] = po;
      P.out_parent[ob] = po;
      P.out_index[ob] = p;
      P.out_token[ob] = P.token[tb + p];
      P.out_depth[ob] = rec[p].key / kBuildMaxNodes;
    }
    __syncthreads();
  }
  for (int oo = nout + tid; oo < NO; oo += kBuildBlock) {
    const long long ob = (long long)b * NO + oo;
    P.out_parent[ob] = -1;
    P.out_index[ob] = -1;
    P.out_token[ob] = -1;
    P.out_depth[ob] = -1;
  }
  // ancestor bitmask rows (ancestors have decreasing positions)
  for (int oo = tid; oo < NO; oo += kBuildBlock) {
    uint32_t* row = P.out_mask + ((long long)b * NO + oo) * P.W;
    int j = oo < nout ? oo : -1;
    for (int w = P.W - 1; w >= 0; --w) {
      uint32_t bits = 0;
      while (j >= 0 && (j >> 5) == w) {
        bits |= 1u << (j & 31);
        j = opar[j];
      }
      row[w] = bits;
    }
  }
  if (tid == 0) P.out_n[b] = bad ? -1 : nout;
}

}  // namespace

int tree_expand_segments(int V, int* seg_elems) {
  const long long n = ((long long)V + kBlock * kTreeRun - 1) / (kBlock * kTreeRun);
  *seg_elems = kBlock * kTreeRun;
  return (int)(n < 1 ? 1 : n);
}

hipError_t launch_tree_expand(const TreeExpandParams& p, hipStream_t s) {
  const long long rows = (long long)p.B * p.K_in;
  const long long blocks = rows * p.nseg;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const bool aligned = p.dt == DT_BF16 ? p.V % 8 == 0 : p.V % 4 == 0;
  if (p.dt == DT_BF16) {
    if (aligned) hipLaunchKernelGGL((k_topk_sweep<DT_BF16, true>), dim3((unsigned)blocks), dim3(kBlock), 0, s, p);
    else hipLaunchKernelGGL((k_topk_sweep<DT_BF16, false>), dim3((unsigned)blocks), dim3(kBlock), 0, s, p);
  } else {
    if (aligned) hipLaunchKernelGGL((k_topk_sweep<DT_F32, true>), dim3((unsigned)blocks), dim3(kBlock), 0, s, p);
    else hipLaunchKernelGGL((k_topk_sweep<DT_F32, false>), dim3((unsigned)blocks), dim3(kBlock), 0, s, p);
  }
  const int ew = p.K_in < kExpandBlock / kWave ? p.K_in : kExpandBlock / kWave;
  hipLaunchKernelGGL(k_expand, dim3((unsigned)p.B), dim3((unsigned)(ew * kWave)), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_tree_build(const TreeBuildParams& p, hipStream_t s) {
  const size_t lds = (size_t)p.n_nodes * (16 + 4 + 4) + (size_t)(p.M + 1) * 4;
  if (p.n_nodes > kBuildMaxNodes || p.M + 1 > kBuildMaxNodes || lds > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tree_build, dim3((unsigned)p.B), dim3(kBuildBlock), lds, s, p);
  return hipGetLastError();
}

}  // namespace sv
