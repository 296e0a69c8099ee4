// LM-head projection z = h W on the MFMA units (bf16 x bf16 -> fp32).
//
// Pages: "EAGLE-3 speculative decoding review", "EAGLE: Predict Features, Not
// Tokens" (the LM head maps the top-layer feature to vocabulary logits, and
// the EAGLE draft reuses the target's LM head); "EAGLE math", "EAGLE's move"
// and "Why feature drafting lands a higher acceptance rate" (drafted features
// are decoded through the target's own, unchanged head).
//
// C[M, N] = A[M, K] W[K, N]; A = feature rows (K contiguous), W = the head
// with the vocabulary innermost, C fp32.  Rows of A come from two tensors
// (target features, then draft features) so the head is streamed once for
// both.  Workgroup tile 128 x 128, K step 32, four waves in a 2 x 2 grid of
// 64 x 64 wave tiles, each a 2 x 2 grid of v_mfma_f32_32x32x16_bf16.  W tiles
// are transposed into LDS (k contiguous per column) so both MFMA operands are
// 16-byte LDS reads.
#include "sv_kernels.hpp"

namespace sv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDK = BK + 8;   // padded k pitch (elements) of both LDS tiles

template <bool NVEC>
__global__ __launch_bounds__(256) void k_lmhead(LmHeadParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM][LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN][LDK];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const long long n0 = (long long)blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int M = P.M0 + P.M1;
  const int K = P.K;
  const long long N = P.N;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int k0 = 0; k0 < K; k0 += BK) {
    // A tile: 128 rows x 32 k = 512 vectors of 8 bf16.
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int q = tid + t * 256;
      const int m = q >> 2, kv = (q & 3) * 8;
      const int gm = m0 + m;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (gm < M) {
        const uint16_t* src = gm < P.M0 ? P.A0 + (long long)gm * K : P.A1 + (long long)(gm - P.M0) * K;
        v = *reinterpret_cast<const uint4*>(src + k0 + kv);
      }
      *reinterpret_cast<uint4*>(&As[m][kv]) = v;
    }
    // W tile: 32 k x 128 n, written transposed (n-major, k contiguous).
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int q = tid + t * 256;
      const int k = q >> 4, nv = (q & 15) * 8;
      const long long gn = n0 + nv;
      const uint16_t* src = P.W + (long long)(k0 + k) * N + gn;
      uint16_t vals[8];
      if (NVEC && gn + 8 <= N) {
        const uint4 v = *reinterpret_cast<const uint4*>(src);
        vals[0] = v.x & 0xffff; vals[1] = v.x >> 16; vals[2] = v.y & 0xffff; vals[3] = v.y >> 16;
        vals[4] = v.z & 0xffff; vals[5] = v.z >> 16; vals[6] = v.w & 0xffff; vals[7] = v.w >> 16;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) vals[i] = gn + i < N ? src[i] : (uint16_t)0;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) Bs[nv + i][k] = vals[i];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&As[wm * 64 + i * 32 + (lane & 31)][kk + (lane >> 5) * 8]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Bs[wn * 64 + j * 32 + (lane & 31)][kk + (lane >> 5) * 8]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // Output layout of the 32 x 32 MFMA: lane l holds column l % 32 and rows
  // 8 (r / 4) + 4 (l / 32) + r % 4 for r = 0..15.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const long long col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) P.C[(long long)row * N + col] = acc[i][j][r];
      }
    }
}

}  // namespace

hipError_t launch_lmhead(const LmHeadParams& p, hipStream_t s) {
  const int M = p.M0 + p.M1;
  const long long gx = ((long long)p.N + BN - 1) / BN;
  const long long gy = ((long long)M + BM - 1) / BM;
  if (gx > 0x7fffffffLL || gy > 65535) return hipErrorInvalidValue;
  if (p.N % 8 == 0) hipLaunchKernelGGL(k_lmhead<true>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(k_lmhead<false>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace sv
