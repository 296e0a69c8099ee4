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
//  k_topk_sweep  one workgroup per (frontier row, 32768-logit segment): the
//                segment max, the sum of 2^((z - max) c) and its k largest
//                logits (equal logits: lower index first).  The segment is
//                streamed in four 8192-logit chunks, the next chunk's loads
//                in flight while one is processed; each lane keeps only its
//                max and exp-sum (rescaled when the max grows).  Wave 0 then
//                finds T, the k-th largest lane max: every top-k logit is at
//                or above T and lies in a lane whose max reaches T.  Those
//                lanes (usually k to k + 2) are reread, their logits at or
//                above T collected in LDS and ranked.  When ties or -inf rows
//                make that set large, a second pass keeps each lane's two
//                best logits and one wave picks the top k in k rounds over
//                packed (value, index) keys, rescanning a lane once both of
//                its candidates are taken.
//  k_expand      one workgroup per sequence, one wave per frontier row:
//                merges each row's segments (max, fp64 sum, the k best of
//                the segment lists: by rank counting when the lists hold at
//                most 64 entries, else in k rounds),
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
// The sweep reads every frontier row once; the other two kernels touch
// kilobytes.
#include "sv_kernels.hpp"

#include <limits.h>

namespace sv {

namespace {

constexpr int kTreeRun = 32;     // logits per lane per chunk
constexpr int kTreeChunks = 4;   // chunks per segment, streamed with the next one in flight
constexpr int kTreeChunk = kBlock * kTreeRun;
constexpr int kExpandBlock = 512;   // one wave per frontier row (up to 8 at a time)
constexpr int kBuildBlock = 1024;

// Candidate keys: (value desc, index asc) as one unsigned 64-bit order.
// The high word maps the float's bits to an unsigned order that rises with
// the value (sign flipped for positives, all bits for negatives); the low
// word is ~index, so among equal values the lower index has the larger key.
// Key 0 is below every real candidate and marks an empty slot.  -0 is keyed
// as +0, since the two compare equal (the index decides between them).
__device__ __forceinline__ unsigned long long cand_key(float v, int idx) {
  unsigned u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;
  const unsigned mono = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)mono << 32) | (unsigned)(~(unsigned)idx);
}
__device__ __forceinline__ float key_value(unsigned long long k) {
  const unsigned mono = (unsigned)(k >> 32);
  return __uint_as_float((mono & 0x80000000u) ? (mono & 0x7fffffffu) : ~mono);
}
__device__ __forceinline__ int key_index(unsigned long long k) { return (int)(~(unsigned)k); }

template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long x) {
  const unsigned lo = (unsigned)dpp_i<CTRL>((int)(unsigned)x);
  const unsigned hi = (unsigned)dpp_i<CTRL>((int)(unsigned)(x >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long x, int l) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)x, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(x >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}
// 64-bit unsigned max over a full wave (the wave reductions' DPP pattern).
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) {
  x = umax64(x, dpp_u64<kDppXor1>(x));
  x = umax64(x, dpp_u64<kDppXor2>(x));
  x = umax64(x, dpp_u64<kDppHalfMirror>(x));
  x = umax64(x, dpp_u64<kDppMirror>(x));
  return umax64(umax64(readlane_u64(x, 0), readlane_u64(x, 16)), umax64(readlane_u64(x, 32), readlane_u64(x, 48)));
}

// bf16 candidates of one segment fit one unsigned 32-bit order: the value's
// 16 bits mapped as above in the high half, 0xFFFF - (index within the
// segment) in the low half (a segment holds at most 32768 logits, so a real
// key is never 0).  Same order, half the width of each wave reduction.
__device__ __forceinline__ unsigned cand_key16(float v, int li) {
  unsigned u = __float_as_uint(v) >> 16;
  u = u == 0x8000u ? 0u : u;
  const unsigned mono = (u & 0x8000u) ? (~u & 0xFFFFu) : (u | 0x8000u);
  return (mono << 16) | (0xFFFFu - (unsigned)li);
}
__device__ __forceinline__ unsigned wave_max_u32(unsigned x) {
  x = max(x, (unsigned)dpp_i<kDppXor1>((int)x));
  x = max(x, (unsigned)dpp_i<kDppXor2>((int)x));
  x = max(x, (unsigned)dpp_i<kDppHalfMirror>((int)x));
  x = max(x, (unsigned)dpp_i<kDppMirror>((int)x));
  const unsigned a = (unsigned)__builtin_amdgcn_readlane((int)x, 0), b = (unsigned)__builtin_amdgcn_readlane((int)x, 16);
  const unsigned c = (unsigned)__builtin_amdgcn_readlane((int)x, 32), d = (unsigned)__builtin_amdgcn_readlane((int)x, 48);
  return max(max(a, b), max(c, d));
}

static_assert(kTreeChunk * kTreeChunks <= 0x8000, "segment-local indices fit the low half of a 32-bit key");

// Candidate keys of a segment starting at element e0, by element type.
template <int DT>
struct TopkKey;
template <>
struct TopkKey<DT_BF16> {
  using T = unsigned;
  static __device__ __forceinline__ T make(float v, int e, long long e0) { return cand_key16(v, (int)(e - e0)); }
  static __device__ __forceinline__ float value(T k) {
    const unsigned mono = k >> 16;
    const unsigned u = (mono & 0x8000u) ? (mono & 0x7FFFu) : (~mono & 0xFFFFu);
    return __uint_as_float(u << 16);
  }
  static __device__ __forceinline__ int index(T k, long long e0) { return (int)(e0 + (0xFFFFu - (k & 0xFFFFu))); }
  static __device__ __forceinline__ T wmax(T x) { return wave_max_u32(x); }
  static __device__ __forceinline__ T readlane(T x, int l) { return (T)__builtin_amdgcn_readlane((int)x, l); }
};
template <>
struct TopkKey<DT_F32> {
  using T = unsigned long long;
  static __device__ __forceinline__ T make(float v, int e, long long) { return cand_key(v, e); }
  static __device__ __forceinline__ float value(T k) { return key_value(k); }
  static __device__ __forceinline__ int index(T k, long long) { return key_index(k); }
  static __device__ __forceinline__ T wmax(T x) { return wave_max_u64(x); }
  static __device__ __forceinline__ T readlane(T x, int l) { return readlane_u64(x, l); }
};

// (v, i) comes before (w, j) in the candidate order: larger value first,
// then lower index
__device__ __forceinline__ bool topk_before(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

// Element of register q of lane t in chunk ch of the segment starting at e0:
// chunk ch covers [e0 + ch * kTreeChunk, +kTreeChunk); register q of lane t
// is element ((q / EPV) * kBlock + t) * EPV + q % EPV of it (vector q / EPV of
// the lane; coalesced).
template <int EPV>
__device__ __forceinline__ long long topk_elem(long long e0, int ch, int q, int t) {
  return e0 + (long long)ch * kTreeChunk + (long long)(((q / EPV) * kBlock + t) * EPV + (q % EPV));
}

// Issue this lane's 16-byte loads of chunk ch (whole vectors inside
// [e0, e1), offsets clamped into the chunk); returns how many of the lane's
// registers hold elements of the segment.
template <int DT>
__device__ __forceinline__ int topk_issue(const char* rowp, long long e0, long long e1, int ch, int tid, v4i* vv) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int KV = kTreeRun / EPV;
  const long long cb = e0 + (long long)ch * kTreeChunk;
  const long long ce = cb + kTreeChunk < e1 ? cb + kTreeChunk : e1;
  const int nvec = ce > cb ? (int)((ce - cb) / EPV) : 0;
  if (nvec <= 0) return 0;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(rowp + cb * ES, (uint32_t)nvec * 16u);
#pragma unroll
  for (int k = 0; k < KV; ++k) vv[k] = load16(r, (uint32_t)min(k * kBlock + tid, nvec - 1) * 16u);
  int nv = 0;
#pragma unroll
  for (int k = 0; k < KV; ++k) nv += k * kBlock + tid < nvec ? 1 : 0;
  return nv * EPV;
}

constexpr int kLaneElems = kTreeRun * kTreeChunks;   // one lane's elements of a segment
constexpr int kFastLanes = 16;     // candidate lanes the threshold rescan takes (else the pair pass)
constexpr int kFastList = kWave;   // logits at or above the threshold it ranks (else the pair pass)

// Stream lane tid's elements of the segment [e0, e1), chunk by chunk, the
// next chunk's loads in flight while fn(ch, z) runs on the current one.
// z[q] is element topk_elem(e0, ch, q, tid), -inf past the segment.
template <int DT, bool ALIGNED, class F>
__device__ __forceinline__ void topk_stream(const char* rowp, long long e0, long long e1, int tid, F&& fn) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int KV = kTreeRun / EPV;
  const float NINF = -__builtin_huge_valf();
  v4i cur[KV];
  int ncur = 0;
  if constexpr (ALIGNED) ncur = topk_issue<DT>(rowp, e0, e1, 0, tid, cur);
#pragma unroll 1
  for (int ch = 0; ch < kTreeChunks; ++ch) {
    float z[kTreeRun];
    v4i nxt[KV];
    int nnxt = 0;
    if constexpr (ALIGNED) {
      if (ch + 1 < kTreeChunks) nnxt = topk_issue<DT>(rowp, e0, e1, ch + 1, tid, nxt);
#pragma unroll
      for (int k = 0; k < KV; ++k) unpack<DT>(cur[k], z + k * EPV);
      // a chunk wholly inside the segment (uniform) needs no masking
      if (e0 + (long long)(ch + 1) * kTreeChunk > e1) {
#pragma unroll
        for (int q = 0; q < kTreeRun; ++q) z[q] = q < ncur ? z[q] : NINF;
      }
    } else {
#pragma unroll
      for (int q = 0; q < kTreeRun; ++q) {
        const long long e = topk_elem<EPV>(e0, ch, q, tid);
        z[q] = e < e1 ? load_elem<DT>(rowp, e) : NINF;
      }
    }
    fn(ch, z);
    if constexpr (ALIGNED) {
#pragma unroll
      for (int k = 0; k < KV; ++k) cur[k] = nxt[k];
      ncur = nnxt;
    }
  }
}

// The segment's top k when the threshold rescan cannot take it (more than
// kFastLanes lanes reach the threshold, which takes ties or -inf rows, or
// more than kFastList logits do): a second pass in which each lane keeps its
// two best elements, then k rounds of a wave max over packed keys in wave 0.
// A lane's third best matters only once both of its candidates are taken;
// the wave then rescans that lane's elements together.  Every thread of the
// workgroup calls it; the results go to out->v, out->idx.
template <int DT, bool ALIGNED>
__device__ void topk_pairs(const TreeExpandParams& P, const char* rowp, long long e0, long long e1, int tid,
                           TopkPart* out, float* sh_c1v, float* sh_c2v, int* sh_c1i, int* sh_c2i) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  const float NINF = -__builtin_huge_valf();
  // the lane's two best elements (value desc, then index asc; slots hold
  // chunk * kTreeRun + q, -1 when empty).  The lane's first two elements
  // seed the pair, so strict comparisons settle ties by position from then
  // on; elements past the segment are -inf and never displace anything.
  float b1v = NINF, b2v = NINF;
  int b1q = -1, b2q = -1;
  topk_stream<DT, ALIGNED>(rowp, e0, e1, tid, [&](int ch, float (&z)[kTreeRun]) {
    if (ch == 0) {
      // the lane's first two elements (one 16-byte vector) seed the pair
      const long long f0 = topk_elem<EPV>(e0, 0, 0, tid);
      if (f0 < e1) {
        b1v = z[0];
        b1q = 0;
      }
      if (f0 + 1 < e1) {
        const bool sw = z[1] > z[0];
        b1v = sw ? z[1] : z[0];
        b1q = sw ? 1 : 0;
        b2v = sw ? z[0] : z[1];
        b2q = sw ? 0 : 1;
      }
      z[0] = NINF;                           // consumed by the seeding
      z[1] = NINF;
    }
    const int cbase = ch * kTreeRun;
    // with b1v >= b2v the new second value is the middle of (b1v, b2v, z):
    // one med3 and one max for the values, the strict compares for the slots
#pragma unroll
    for (int q = 0; q < kTreeRun; ++q) {
      const bool c1 = z[q] > b1v;
      const bool c2 = z[q] > b2v;
      b2q = c1 ? b1q : (c2 ? cbase + q : b2q);
      b1q = c1 ? cbase + q : b1q;
      b2v = __builtin_amdgcn_fmed3f(b1v, b2v, z[q]);
      b1v = fmaxf(b1v, z[q]);
    }
  });
  auto code_idx = [&](int code) -> int { return (int)topk_elem<EPV>(e0, code / kTreeRun, code % kTreeRun, tid); };
  sh_c1v[tid] = b1v;
  sh_c1i[tid] = b1q >= 0 ? code_idx(b1q) : INT_MAX;
  sh_c2v[tid] = b2v;
  sh_c2i[tid] = b2q >= 0 ? code_idx(b2q) : INT_MAX;
  __syncthreads();
  if (wid != 0) return;
  // lane l owns source lanes l + 64 j (j < 4) and their two candidates' keys
  using KT = TopkKey<DT>;
  using Key = typename KT::T;
  Key ck[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i1 = sh_c1i[lane + j * kWave], i2 = sh_c2i[lane + j * kWave];
    ck[2 * j] = i1 != INT_MAX ? KT::make(sh_c1v[lane + j * kWave], i1, e0) : (Key)0;
    ck[2 * j + 1] = i2 != INT_MAX ? KT::make(sh_c2v[lane + j * kWave], i2, e0) : (Key)0;
  }
  for (int r = 0; r < P.k; ++r) {
    Key best = ck[0];
#pragma unroll
    for (int t = 1; t < 8; ++t) best = best > ck[t] ? best : ck[t];
    const Key g = KT::wmax(best);
    if (lane == 0) {
      out->v[r] = g ? KT::value(g) : NINF;
      out->idx[r] = g ? KT::index(g, e0) : INT_MAX;
    }
    if (g == 0) continue;                                   // uniform
    // keys are unique: one lane owns the taken key, in slot ts
    const unsigned long long own = __ballot(best == g);
    const int ol = (int)__ffsll((long long)own) - 1;
    int ts = 0;
#pragma unroll
    for (int t = 1; t < 8; ++t) ts = ck[t] == g ? t : ts;
    const int tso = __builtin_amdgcn_readlane(ts, ol);
    Key nb = 0;                                            // a first candidate leaves its slot empty
    if (tso & 1) {                                         // uniform: a second candidate was taken
      const int src = ol + (tso >> 1) * kWave;
#pragma unroll
      for (int j = 0; j < kLaneElems / kWave; ++j) {
        const int qq = lane * (kLaneElems / kWave) + j;
        const long long e = topk_elem<EPV>(e0, qq / kTreeRun, qq % kTreeRun, src);
        if (e < e1) {
          const Key kq = KT::make(load_elem<DT>(rowp, e), (int)e, e0);
          if (kq < g) nb = nb > kq ? nb : kq;
        }
      }
      nb = KT::wmax(nb);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) ck[t] = (lane == ol && t == tso) ? nb : ck[t];
  }
}

template <int DT, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void k_topk_sweep(TreeExpandParams P) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  static_assert(kLaneElems % kWave == 0, "a rescan splits a lane's elements evenly over the wave");
  static_assert(kBlock / kWave * kWave == kBlock && kBlock == 4 * kWave, "wave 0 owns four lanes' records per lane");
  __shared__ float sh_lm[kBlock], sh_ls[kBlock], sh_c1v[kBlock], sh_c2v[kBlock];
  __shared__ int sh_c1i[kBlock], sh_c2i[kBlock];
  __shared__ int sh_cl[kFastLanes];                 // candidate lanes of the threshold rescan
  __shared__ float sh_lv[kFastList];                // logits at or above the threshold
  __shared__ int sh_li[kFastList];
  __shared__ int sh_nc, sh_cnt;
  __shared__ float sh_T;
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
  if (tid == 0) {
    sh_nc = 0;
    sh_cnt = 0;
  }
  const long long e0 = (long long)s * P.seg_elems;
  const long long e1 = e0 + P.seg_elems < V ? e0 + P.seg_elems : V;
  const char* rowp = static_cast<const char*>(P.logits) + row * V * ES;
  // One pass over the lane's chunks: its max and its exponential sum
  // against its running max (rescaled when the max grows).
  float ls = 0.f, lm = NINF;
  const float c = P.tc.c_hi;
  topk_stream<DT, ALIGNED>(rowp, e0, e1, tid, [&](int, float (&z)[kTreeRun]) {
    float cm = z[0];
#pragma unroll
    for (int q = 1; q < kTreeRun; ++q) cm = fmaxf(cm, z[q]);
    if (cm > lm) {
      ls = lm > NINF ? ls * __builtin_amdgcn_exp2f((lm - cm) * c) : 0.f;
      lm = cm;
    }
    if (lm > NINF) {
      float cs = 0.f;
#pragma unroll
      for (int q = 0; q < kTreeRun; ++q) cs += __builtin_amdgcn_exp2f((z[q] - lm) * c);
      ls += cs;
    }
  });
  sh_lm[tid] = lm;
  sh_ls[tid] = ls;
  __syncthreads();
  // wave 0: the segment's (max, sum), and the threshold T, the k-th largest
  // lane max counted with multiplicity.  At least k lanes hold a logit at or
  // above T, so every logit of the segment's top k is at or above T and lies
  // in a lane whose max reaches T: the candidate lanes.
  using KT = TopkKey<DT>;
  using Key = typename KT::T;
  float M = NINF;
  double S = 0.0;
  if (wid == 0) {
    float lmj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) lmj[j] = sh_lm[lane + j * kWave];
    M = wave_max(fmaxf(fmaxf(lmj[0], lmj[1]), fmaxf(lmj[2], lmj[3])));
    float s4 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s4 += lmj[j] > NINF ? sh_ls[lane + j * kWave] * __builtin_amdgcn_exp2f((lmj[j] - M) * c) : 0.f;
    S = wave_sum((double)s4);
    // k rounds over (lane max, lane) keys, one instance taken per round
    Key kk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kk[j] = KT::make(lmj[j], (int)e0 + lane + j * kWave, e0);
    Key g = 0;
    for (int r = 0; r < P.k; ++r) {
      const Key b01 = kk[0] > kk[1] ? kk[0] : kk[1], b23 = kk[2] > kk[3] ? kk[2] : kk[3];
      g = KT::wmax(b01 > b23 ? b01 : b23);
#pragma unroll
      for (int j = 0; j < 4; ++j) kk[j] = kk[j] == g ? (Key)0 : kk[j];
    }
    const float T = KT::value(g);
    int nc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool sel = lmj[j] >= T;
      const unsigned long long m = __ballot(sel);
      const int at = nc + (int)__popcll(m & ((1ull << lane) - 1ull));
      if (sel && at < kFastLanes) sh_cl[at] = lane + j * kWave;
      nc += (int)__popcll(m);
    }
    if (lane == 0) {
      sh_nc = nc;
      sh_T = T;
    }
  }
  __syncthreads();
  const int nc = sh_nc;
  bool fast = nc <= kFastLanes;
  if (fast) {
    // rescan the candidate lanes; collect their logits at or above T
    const float T = sh_T;
    auto keep = [&](float v, long long gi) {
      if (v >= T) {
        const int at = atomicAdd(&sh_cnt, 1);
        if (at < kFastList) {
          sh_lv[at] = v;
          sh_li[at] = (int)gi;
        }
      }
    };
    if constexpr (ALIGNED) {
      // one 16-byte vector per item: vector (ch, k) of candidate lane src
      constexpr int KV = kTreeRun / EPV, kLaneVecs = kTreeChunks * KV;
      for (int it = tid; it < nc * kLaneVecs; it += kBlock) {
        const int src = sh_cl[it / kLaneVecs], vj = it % kLaneVecs;
        const long long gb = topk_elem<EPV>(e0, vj / KV, (vj % KV) * EPV, src);
        if (gb < e1) {                                     // whole vectors: in or out of the segment
          float z[EPV];
          unpack<DT>(*reinterpret_cast<const v4i*>(rowp + gb * ES), z);
#pragma unroll
          for (int i = 0; i < EPV; ++i) keep(z[i], gb + i);
        }
      }
    } else {
      for (int e = tid; e < nc * kLaneElems; e += kBlock) {
        const int src = sh_cl[e / kLaneElems], qq = e % kLaneElems;
        const long long gi = topk_elem<EPV>(e0, qq / kTreeRun, qq % kTreeRun, src);
        if (gi < e1) keep(load_elem<DT>(rowp, gi), gi);
      }
    }
    __syncthreads();
    fast = sh_cnt <= kFastList;
  }
  if (fast) {
    if (wid != 0) return;
    // rank the collected logits (lane c holds entry c) by (value desc, index asc)
    using KT = TopkKey<DT>;
    using Key = typename KT::T;
    const int cnt = sh_cnt;
    const Key key = lane < cnt ? KT::make(sh_lv[lane], sh_li[lane], e0) : (Key)0;
    int rank = 0;
    for (int c2 = 0; c2 < cnt; ++c2) rank += (int)(KT::readlane(key, c2) > key);
    if (lane < cnt && rank < P.k) {
      out->v[rank] = KT::value(key);
      out->idx[rank] = KT::index(key, e0);
    }
    for (int r = cnt + lane; r < P.k; r += kWave) {       // fewer logits than k in the segment
      out->v[r] = NINF;
      out->idx[r] = INT_MAX;
    }
  } else {
    topk_pairs<DT, ALIGNED>(P, rowp, e0, e1, tid, out, sh_c1v, sh_c2v, sh_c1i, sh_c2i);
    if (wid != 0) return;
  }
  if (lane == 0) {
    out->m = M;
    out->s = (float)S;
  }
}

__global__ __launch_bounds__(kExpandBlock) void k_expand(TreeExpandParams P) {
  __shared__ double sc[kCandMax];
  __shared__ int sh_rank[kCandMax];
  __shared__ int sh_count;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int b = blockIdx.x;
  const int k = P.k;
  const long long tb = (long long)b * P.cap;
  const int ncand = P.K_in * k;
  const float NINF = -__builtin_huge_valf();
  if (tid == 0) sh_count = 0;
  for (int c = tid; c < ncand; c += blockDim.x) sh_rank[c] = 0;
  const int nw = blockDim.x / kWave;
  // With at most 64 list entries per row, lane c holds entry c % k of segment
  // c / k and its rank among them gives its output slot directly; otherwise
  // the lists merge in k rounds.
  const int nent = P.nseg * k;
  const bool by_rank = nent <= kWave;
  for (int f = wid; f < P.K_in; f += nw) {
    const long long row = (long long)b * P.K_in + f;
    const TopkPart* pr = P.part + row * P.nseg;
    // Everything below reads the row's partials whether or not the slot is
    // live (the sweep writes an empty record for a dead slot), so these loads
    // do not wait for the frontier entry; a dead slot's outputs are empty.
    const int pn = P.frontier[row];
    float cv = NINF;
    int ci = INT_MAX;
    int cj = -1;                                  // the entry's place in its list
    if (by_rank && lane < nent) {
      const int s = lane / k;
      cj = lane - s * k;
      cv = pr[s].v[cj];
      ci = pr[s].idx[cj];
    }
    // the segments' (max, sum) records: one per lane when they fit a wave
    float sm = NINF, ss = 0.f;
    if (P.nseg <= kWave && lane < P.nseg) {
      sm = pr[lane].m;
      ss = pr[lane].s;
    }
    // the parent's score and depth (the only loads that wait for the frontier)
    const bool live = pn >= 0 && pn < P.off;  // entries past the written table count as empty
    const double ps = P.score[tb + (live ? pn : 0)];
    const int pd = P.depth[tb + (live ? pn : 0)];
    // row max and fp64 sum over the segments
    float m = sm;
    for (int t = lane + kWave; t < P.nseg; t += kWave) m = fmaxf(m, pr[t].m);
    if (P.nseg > kWave) m = fmaxf(m, pr[lane].m);
    const float M = wave_max(m);
    double S = ss > 0.f ? (double)ss * exp2_f64(((double)sm - (double)M) * P.tc.c64) : 0.0;
    if (P.nseg > kWave) {
      S = 0.0;
      for (int t = lane; t < P.nseg; t += kWave) {
        const float tm = pr[t].m, ts = pr[t].s;
        if (ts > 0.f) S += (double)ts * exp2_f64(((double)tm - (double)M) * P.tc.c64);
      }
    }
    S = wave_sum(S);
    const double l2S = log2(S);
    // child r of the row: token i with logit v (i == INT_MAX: none)
    auto put = [&](int r, float v, int i) {
      const long long pos = tb + P.off + (long long)f * k + r;
      const bool real = live && i != INT_MAX;
      double sv = -__builtin_huge_val();
      if (real && v > NINF) sv = ps + (((double)v - (double)M) * P.tc.c64 - l2S) * kLn2;
      P.parent[pos] = real ? pn : -1;
      P.token[pos] = real ? i : -1;
      P.score[pos] = sv;
      P.depth[pos] = real ? pd + 1 : -1;
      sc[f * k + r] = sv;
    };
    if (by_rank) {
      // rank = entries before this one in (value desc, index asc), as 64-bit
      // keys (0: empty entry); equal keys (only empty entries) go by lane, so
      // the ranks are a permutation and ranks 0..k-1 fill every slot once.
      // The k-th best entry is no worse than the best of the segments' k-th
      // entries (each segment has k entries at least that good), so only
      // entries at or above that bound can rank below k, and every entry
      // before one of them is one of them: the counts run over those alone.
      const unsigned long long key = (ci != INT_MAX) ? cand_key(cv != cv ? NINF : cv, ci) : 0ull;
      const unsigned long long bound = wave_max_u64(cj == k - 1 ? key : 0ull);
      const bool cand = lane < nent && key >= bound;
      int rank = 0;
      for (unsigned long long mm = __ballot(cand); mm; mm &= mm - 1) {
        const int c2 = __builtin_ctzll(mm);
        const unsigned long long w = readlane_u64(key, c2);
        rank += (int)((w > key) | ((w == key) & (c2 < lane)));
      }
      if (cand && rank < k) put(rank, cv, ci);
      continue;
    }
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
        hv[j] = in ? pr[in ? lane : 0].v[j] : NINF;
        hi[j] = in ? pr[in ? lane : 0].idx[j] : INT_MAX;
      }
    }
    for (int r = 0; r < k; ++r) {
      float v = NINF;
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
          const float cv2 = pr[t].v[j];
          const int ci2 = pr[t].idx[j];
          if (ci2 != INT_MAX && topk_before(pv, pi, cv2, ci2) && topk_before(cv2, ci2, v, ix)) {
            v = cv2;
            ix = ci2;
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
        hv[kTopkMax - 1] = NINF;
        hi[kTopkMax - 1] = INT_MAX;
      }
      if (lane == 0) put(r, wv, wi);
    }
  }
  __syncthreads();
  // next frontier: rank among the children with a finite score, the
  // comparisons of one child split over a power-of-two group of threads
  const int nt = blockDim.x;
  const int lp = ncand >= nt ? 0 : 31 - __builtin_clz((unsigned)(nt / ncand));
  const int parts = 1 << lp;
  for (int it = tid; it < (ncand << lp); it += nt) {
    const int c = it >> lp;
    const double v = sc[c];
    if (!(v > -__builtin_huge_val())) continue;
    int cnt = 0;
    for (int c2 = it & (parts - 1); c2 < ncand; c2 += parts) {
      const double w = sc[c2];
      cnt += (int)((w > v) | ((w == v) & (c2 < c)));
    }
    if (cnt) atomicAdd(&sh_rank[c], cnt);
  }
  __syncthreads();
  for (int c = tid; c < ncand; c += nt) {
    const bool fin = sc[c] > -__builtin_huge_val();
    const unsigned long long fm = __ballot(fin);
    if (fin && lane == __builtin_ctzll(fm)) atomicAdd(&sh_count, __popcll(fm));
    if (fin && sh_rank[c] < P.K_out) P.next_frontier[(long long)b * P.K_out + sh_rank[c]] = P.off + c;
  }
  __syncthreads();
  for (int t = sh_count + tid; t < P.K_out; t += blockDim.x) P.next_frontier[(long long)b * P.K_out + t] = -1;
}

// For one node (score ms, key mk): how many nodes q0 <= q < q1 come before
// it by (score desc, key asc); a node not counted has a NaN score, which no
// comparison passes.  The threads of a wave read the same scores (LDS
// broadcasts), eight per wait; the keys are read only for a batch in which
// some lane meets an equal score (its own, at least once).
__device__ int count_before(const double* rs, const int* rkey, int q0, int q1, double ms, int mk) {
  int cnt = 0;
  int q = q0;
  for (; q + 8 <= q1; q += 8) {
    double r[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = rs[q + t];
    bool eq = false;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      cnt += (int)(r[t] > ms);
      eq |= r[t] == ms;
    }
    if (__ballot(eq)) {
#pragma unroll
      for (int t = 0; t < 8; ++t) cnt += (int)((r[t] == ms) & (rkey[q + t] < mk));
    }
  }
  for (; q < q1; ++q) {
    const double r = rs[q];
    cnt += (int)((r > ms) | ((r == ms) & (rkey[q] < mk)));
  }
  return cnt;
}

__global__ __launch_bounds__(kBuildBlock) void k_tree_build(TreeBuildParams P) {
  extern __shared__ double tb_lds[];
  const int n = P.n_nodes, tid = threadIdx.x, b = blockIdx.x;
  double* rs = tb_lds;                                // [n] score (NaN once a node is not ranked)
  int* rkey = reinterpret_cast<int*>(rs + n);         // [n] depth * kBuildMaxNodes + table index
  int* flag = rkey + n;                               // [n] drafted, then kept
  int* par = flag + n;                                // [n] table parent
  int* pos = par + n;                                 // [n] depth, then rank, then output position
  int* opar = pos + n;                                // [M + 1] kept nodes by rank, then output parents
  const long long tb = (long long)b * P.cap;
  const int NO = P.M + 1;
  const double NINF = -__builtin_huge_val();
  __shared__ int sh_nk;
  if (tid == 0) sh_nk = 0;
  for (int p = tid; p < n; p += kBuildBlock) {
    rs[p] = P.score[tb + p];
    par[p] = P.parent[tb + p];
    pos[p] = P.depth[tb + p];
  }
  __syncthreads();
  // drafted nodes, keys, and the invariants of a table the expansion wrote
  bool bad = false;
  for (int p = tid; p < n; p += kBuildBlock) {
    const int q = par[p];
    const bool drafted = p >= 1 && q >= 0 && rs[p] > NINF;
    flag[p] = drafted ? 1 : 0;
    rkey[p] = pos[p] * kBuildMaxNodes + p;
    if (p == 0) bad |= q != -1 || pos[0] != 0;
    else if (drafted)
      bad |= q >= p || (q != 0 && !(par[q] >= 0 && rs[q] > NINF)) || pos[p] != pos[q] + 1 || pos[p] < 1 ||
             pos[p] >= (1 << 19);
  }
  bad = __syncthreads_or(bad);
  if (!bad) {
    // keep the M best drafted nodes by (score desc, depth asc, index asc):
    // a drafted node's rank counts the drafted nodes before it, T threads
    // per node each over a range of the table, summed in pos[] (the depths
    // there are no longer needed: the keys carry them)
    for (int p = tid; p < n; p += kBuildBlock) {
      pos[p] = 0;
      if (!flag[p]) rs[p] = __builtin_nan("");
    }
    __syncthreads();
    const int T = n < kBuildBlock ? kBuildBlock / n : 1;
    const int L = (n + T - 1) / T;
    for (int w = tid; w < n * T; w += kBuildBlock) {
      const int p = w / T, c = w - p * T;
      if (!flag[p]) continue;
      const int q0 = c * L, q1 = q0 + L < n ? q0 + L : n;
      const int cnt = count_before(rs, rkey, q0, q1, rs[p], rkey[p]);
      if (cnt) atomicAdd(&pos[p], cnt);
    }
    __syncthreads();
    // kept: the root and ranks below M; a kept drafted node's rank is its
    // slot in the list of kept nodes (opar[], until the parents go there)
    int cnt = 0;
    for (int p = tid; p < n; p += kBuildBlock) {
      int k = p == 0 ? 1 : 0;
      if (p != 0 && flag[p]) {
        const int r = pos[p];
        k = r < P.M ? 1 : 0;
        if (k) opar[r] = p;
      }
      flag[p] = k;
      cnt += (p != 0 && k) ? 1 : 0;
    }
    if (cnt) atomicAdd(&sh_nk, cnt);
    __syncthreads();
    // kept nodes' parents must be kept (true for scores the expansion wrote)
    bool open = false;
    for (int p = tid; p < n; p += kBuildBlock)
      if (p != 0 && flag[p] && !flag[par[p]]) open = true;
    bad = __syncthreads_or(open);
  }
  const int nkept = sh_nk;
  const int nout = bad ? 0 : 1 + nkept;
  if (!bad) {
    // output position: the root first, then (depth asc, score desc, index
    // asc) counted over the kept drafted nodes only, each node's comparisons
    // split over a power-of-two group of threads
    for (int p = tid; p < n; p += kBuildBlock) pos[p] = p == 0 ? 0 : -1;
    __syncthreads();
    for (int i = tid; i < nkept; i += kBuildBlock) pos[opar[i]] = 1;
    __syncthreads();
    const int lp = (nkept == 0 || nkept >= kBuildBlock) ? 0 : 31 - __builtin_clz((unsigned)(kBuildBlock / nkept));
    for (int w = tid; w < (nkept << lp); w += kBuildBlock) {
      const int p = opar[w >> lp];
      const double ms = rs[p];
      const int mk = rkey[p];
      const unsigned md = (unsigned)mk / kBuildMaxNodes;
      int o = 0;
      for (int j = w & ((1 << lp) - 1); j < nkept; j += 1 << lp) {
        const int q = opar[j];
        const double s = rs[q];
        const int kq = rkey[q];
        const unsigned d = (unsigned)kq / kBuildMaxNodes;
        o += (int)((d < md) | ((d == md) & ((s > ms) | ((s == ms) & (kq < mk)))));
      }
      if (o) atomicAdd(&pos[p], o);
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
      P.out_depth[ob] = rkey[p] / kBuildMaxNodes;
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
  constexpr long long seg = (long long)kTreeChunk * kTreeChunks;
  const long long n = ((long long)V + seg - 1) / seg;
  *seg_elems = (int)seg;
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
  const size_t lds = (size_t)p.n_nodes * (8 + 4 * 4) + (size_t)(p.M + 1) * 4;
  if (p.n_nodes > kBuildMaxNodes || p.M + 1 > kBuildMaxNodes || lds > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tree_build, dim3((unsigned)p.B), dim3(kBuildBlock), lds, s, p);
  return hipGetLastError();
}

}  // namespace sv
