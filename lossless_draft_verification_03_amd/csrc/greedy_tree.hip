// Greedy and greedy-tree verification, after the row sweep has produced the
// lowest-index argmax of every target row.
//
// Pages: "EAGLE-3 speculative decoding review", "Does Using a Small Model's
// Answer Reduce Quality?" (accept iff the draft equals the target's argmax;
// otherwise emit the target token and stop), "EAGLE-2: Does Every Context Need
// the Same Draft Tree?" (a node sees only the shared prefix and its own
// ancestors) and "The Complete EAGLE-3 Inference Process" (4. Strict
// Acceptance: the longest prefix matching the target's choices); "EAGLE
// math", "EAGLE-2: dynamic draft trees".
#include "sv_kernels.hpp"

#include <limits.h>

namespace sv {

namespace {

constexpr int SPEC_TREE_LDS_NODES = 4096;   // = SPEC_MAX_TREE_NODES

// One workgroup per sequence: lane groups of NP lanes merge the argmax
// partials of the g + 1 target rows, then lane i of wave 0 compares draft i
// with the argmax of row i and a ballot gives the first mismatch.
template <int NP>
__global__ __launch_bounds__(kBlock) void k_greedy_finish(GreedyParams P) {
  __shared__ int sh_arg[64];
  const int tid = threadIdx.x;
  const long long b = blockIdx.x;
  const int g = P.g;
  const int* x = P.tokens + b * g;
  const int xi = tid < g ? x[tid] : 0;
  for (int row = tid / NP; row <= g; row += kBlock / NP) {
    float M;
    double S;
    int a;
    merge_partials<2, NP>(P.part + (b * (g + 1) + row) * P.nseg, P.nseg, TempConst{}, tid & (NP - 1), &M, &S, &a);
    if ((tid & (NP - 1)) == 0) sh_arg[row] = a;
  }
  __syncthreads();
  if (tid >= kWave) return;
  const int ai = tid <= g ? sh_arg[tid] : 0;
  const unsigned long long mm = __ballot(tid < g && xi != ai);
  const int j = mm ? (int)__ffsll((long long)mm) - 1 : g;
  const int aj = sh_arg[j];
  int* out = P.out_tokens + b * (g + 1);
  if (tid <= g) out[tid] = tid < j ? xi : (tid == j ? aj : -1);
  if (tid == 0) P.accept_len[b] = j;
}

// One workgroup per sequence.  Lane groups first merge the argmax partials
// of the N node rows.  ok(n) = ok(parent(n)) and tok(n) == argmax(parent(n)),
// depth(n) = depth(parent(n)) + 1, both resolved by pointer jumping over the
// ancestor links in LDS (log2 N rounds).  The accepted node maximises
// (depth, -index) over ok nodes.
template <int NP>
__global__ __launch_bounds__(kBlock) void k_tree_finish(TreeParams P) {
  __shared__ short s_anc[2][SPEC_TREE_LDS_NODES];
  __shared__ unsigned char s_ok[2][SPEC_TREE_LDS_NODES];
  __shared__ short s_dep[2][SPEC_TREE_LDS_NODES];
  __shared__ short s_par[SPEC_TREE_LDS_NODES];
  __shared__ int s_arg[SPEC_TREE_LDS_NODES];
  __shared__ int s_bad;
  __shared__ int s_key[kBlock / kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const long long b = blockIdx.x;
  const int N = P.N;
  const int* par = P.parent + b * P.parent_stride;
  const int* tok = P.node_tokens + b * N;
  if (tid == 0) s_bad = 0;
  for (int row = tid / NP; row < N; row += kBlock / NP) {
    float M;
    double S;
    int a;
    merge_partials<2, NP>(P.part + (b * N + row) * P.nseg, P.nseg, TempConst{}, tid & (NP - 1), &M, &S, &a);
    if ((tid & (NP - 1)) == 0) s_arg[row] = a;
  }
  __syncthreads();
  for (int n = tid; n < N; n += kBlock) {
    const int p = par[n];
    const bool valid = n == 0 ? p == -1 : (p >= 0 && p < n);
    if (!valid) s_bad = 1;
    s_par[n] = (short)(n == 0 ? 0 : (valid ? p : 0));
  }
  __syncthreads();
  int* out_path = P.out_path + b * N;
  int* out_tok = P.out_tokens + b * N;
  if (s_bad) {
    for (int n = tid; n < N; n += kBlock) {
      out_path[n] = -1;
      out_tok[n] = -1;
    }
    if (tid == 0) P.accept_len[b] = -1;
    return;
  }
  for (int n = tid; n < N; n += kBlock) {
    const int p = s_par[n];
    s_anc[0][n] = (short)p;
    s_ok[0][n] = n == 0 ? 1 : (unsigned char)(tok[n] == s_arg[p]);
    s_dep[0][n] = (short)(n == 0 ? 0 : 1);
  }
  __syncthreads();
  int cur = 0;
  for (int span = 1; span < N; span <<= 1) {
    for (int n = tid; n < N; n += kBlock) {
      const int a = s_anc[cur][n];
      s_anc[cur ^ 1][n] = s_anc[cur][a];
      s_ok[cur ^ 1][n] = s_ok[cur][n] & s_ok[cur][a];
      s_dep[cur ^ 1][n] = (short)(s_dep[cur][n] + s_dep[cur][a]);
    }
    __syncthreads();
    cur ^= 1;
  }
  // key = depth * 4096 + (4095 - n): the maximum is the deepest ok node with
  // the lowest index.
  int key = -1;
  for (int n = tid; n < N; n += kBlock)
    if (s_ok[cur][n]) key = max(key, (int)s_dep[cur][n] * 4096 + (4095 - n));
  key = wave_max_i(key);
  if (lane == 0) s_key[wid] = key;
  __syncthreads();
  key = max(max(s_key[0], s_key[1]), max(s_key[2], s_key[3]));
  const int nstar = 4095 - (key & 4095);
  const int depth = key >> 12;
  for (int n = tid; n < N; n += kBlock) {
    out_path[n] = -1;
    out_tok[n] = -1;
  }
  __syncthreads();
  if (tid == 0) {
    int m = nstar;
    for (int d = depth - 1; d >= 0; --d) {
      out_path[d] = m;
      out_tok[d] = tok[m];
      m = s_par[m];
    }
    out_tok[depth] = s_arg[nstar];
    P.accept_len[b] = depth;
  }
}

// p, q and the normalised residual of row pairs, through the same element
// function as the linear sampling draw (exp_koff).  Test probe; one workgroup
// per row.
template <int DT>
__global__ __launch_bounds__(kBlock) void k_probe(ProbeParams P) {
  __shared__ double sh4[4];
  const int tid = threadIdx.x;
  const long long r = blockIdx.x;
  const long long V = P.V;
  constexpr int ES = DT == DT_BF16 ? 2 : 4;
  const char* t = static_cast<const char*>(P.tgt) + r * V * ES;
  const char* d = P.drf ? static_cast<const char*>(P.drf) + r * V * ES : nullptr;
  // the linear draw's weights: 2^(z c - K) with K = fl(M c_hi), and the
  // fp64 factors 2^(K - M c) back to 2^((z - M) c)
  const float Mt = P.row_max[r];
  const double St = P.row_sum[r];
  const float Kt = koff_of(Mt, P.tc);
  const double ft = exp2_f64((double)Kt - (double)Mt * P.tc.c64);
  float Md = 0.f, Kd = 0.f;
  double Sd = 1.0, fd = 1.0, rho = 0.0;
  if (d) {
    Md = P.row_max[P.rows + r];
    Sd = P.row_sum[P.rows + r];
    Kd = koff_of(Md, P.tc);
    fd = exp2_f64((double)Kd - (double)Md * P.tc.c64);
    rho = St / Sd * (fd / ft);
  }
  const float rho_hi = (float)rho, rho_lo = (float)(rho - (double)rho_hi);
  double part = 0.0;
  for (long long e = tid; e < V; e += kBlock) {
    const float et = exp_koff(load_elem<DT>(t, e), Kt, P.tc);
    P.out_p[r * V + e] = (double)et * ft / St;
    if (d) {
      const float ed = exp_koff(load_elem<DT>(d, e), Kd, P.tc);
      if (P.out_q) P.out_q[r * V + e] = (double)ed * fd / Sd;
      float w = fmaf(-ed, rho_hi, et);
      w = fmaxf(fmaf(-ed, rho_lo, w), 0.f);
      part += (double)w;
      if (P.out_resid) P.out_resid[r * V + e] = (double)w;
    }
  }
  if (!d || !P.out_resid) return;
  part = wave_sum(part);
  if ((tid & (kWave - 1)) == 0) sh4[tid / kWave] = part;
  __syncthreads();
  const double tot = (sh4[0] + sh4[1]) + (sh4[2] + sh4[3]);
  const double inv = tot > 0.0 ? 1.0 / tot : 0.0;
  for (long long e = tid; e < V; e += kBlock) P.out_resid[r * V + e] *= inv;
}

__global__ void k_fill_zero(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t k = i; k < n16; k += stride) p[k] = make_uint4(0, 0, 0, 0);
  if (i < ntail) tail[i] = 0;
}

// Stream read: workgroup c reads 16-byte vectors [c V, (c + 1) V) of the
// buffer, V = kBlock * kStreamVPT, each lane issuing its kStreamVPT
// non-temporal loads before it uses any (the row sweep's access pattern
// without its arithmetic), and XORs them into one word per workgroup so the
// loads stay live.  A bandwidth probe, not part of any verification call.
constexpr int kStreamVPT = 8;

__global__ __launch_bounds__(kBlock) void k_stream_read(const char* src, long long nvec, uint32_t* sink) {
  __shared__ uint32_t sh[kBlock / kWave];
  const int tid = threadIdx.x;
  const long long v0 = (long long)blockIdx.x * kBlock * kStreamVPT;
  const long long nv = nvec - v0 < (long long)kBlock * kStreamVPT ? nvec - v0 : (long long)kBlock * kStreamVPT;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src + v0 * 16, (uint32_t)nv * 16u);
  v4i x[kStreamVPT];
#pragma unroll
  for (int k = 0; k < kStreamVPT; ++k) x[k] = load16(r, (uint32_t)(k * kBlock + tid) * 16u);   // past nv: 0
  uint32_t acc = 0;
#pragma unroll
  for (int k = 0; k < kStreamVPT; ++k) acc ^= (uint32_t)(x[k][0] ^ x[k][1] ^ x[k][2] ^ x[k][3]);
  acc ^= (uint32_t)dpp_i<kDppXor1>((int)acc);
  acc ^= (uint32_t)dpp_i<kDppXor2>((int)acc);
  acc ^= (uint32_t)dpp_i<kDppHalfMirror>((int)acc);
  acc ^= (uint32_t)dpp_i<kDppMirror>((int)acc);
  acc = (uint32_t)__builtin_amdgcn_readlane((int)acc, 0) ^ (uint32_t)__builtin_amdgcn_readlane((int)acc, 16) ^
        (uint32_t)__builtin_amdgcn_readlane((int)acc, 32) ^ (uint32_t)__builtin_amdgcn_readlane((int)acc, 48);
  if ((tid & (kWave - 1)) == 0) sh[tid / kWave] = acc;
  __syncthreads();
  if (tid == 0) sink[blockIdx.x] = sh[0] ^ sh[1] ^ sh[2] ^ sh[3];
}

}  // namespace

long long stream_read_workgroups(long long bytes) {
  const long long per = (long long)kBlock * kStreamVPT * 16;
  return (bytes + per - 1) / per;
}

hipError_t launch_stream_read(const void* src, long long bytes, uint32_t* sink, hipStream_t s) {
  const long long grid = stream_read_workgroups(bytes);
  if (grid < 1) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(kBlock), 0, s, static_cast<const char*>(src),
                     bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_greedy_finish(const GreedyParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.B), block(kBlock);
  switch (merge_group(p.nseg)) {
    case 1: hipLaunchKernelGGL(k_greedy_finish<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(k_greedy_finish<2>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(k_greedy_finish<4>, grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL(k_greedy_finish<8>, grid, block, 0, s, p); break;
    case 16: hipLaunchKernelGGL(k_greedy_finish<16>, grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL(k_greedy_finish<32>, grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL(k_greedy_finish<64>, grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_tree_finish(const TreeParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.B), block(kBlock);
  switch (merge_group(p.nseg)) {
    case 1: hipLaunchKernelGGL(k_tree_finish<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(k_tree_finish<2>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(k_tree_finish<4>, grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL(k_tree_finish<8>, grid, block, 0, s, p); break;
    case 16: hipLaunchKernelGGL(k_tree_finish<16>, grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL(k_tree_finish<32>, grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL(k_tree_finish<64>, grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_probe(const ProbeParams& p, int dt, hipStream_t s) {
  if (dt == DT_BF16) hipLaunchKernelGGL(k_probe<DT_BF16>, dim3((unsigned)p.rows), dim3(kBlock), 0, s, p);
  else hipLaunchKernelGGL(k_probe<DT_F32>, dim3((unsigned)p.rows), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint4*>(ptr), n16,
                     static_cast<unsigned char*>(ptr) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace sv
