// LM-head projection z = h W on the MFMA units (bf16 x bf16 -> fp32).
//
// Pages: "EAGLE-3 speculative decoding review", "EAGLE: Predict Features, Not
// Tokens" (the LM head maps the top-layer feature to vocabulary logits, and
// the EAGLE draft reuses the target's LM head); "EAGLE math", "EAGLE's move"
// and "Why feature drafting lands a higher acceptance rate" (drafted features
// are decoded through the target's own, unchanged head).
//
// C[M, N] = A[M, K] W; A = feature rows (K contiguous, one tensor:
// lmhead_verify first gathers target and draft features into one block so
// the head is streamed once for both), C fp32.  W comes in either layout:
// [N, K] with the feature dimension innermost (a linear layer's weight as
// checkpoints store it), or [K, N] with the vocabulary
// innermost.
//
// Workgroup tile 256 x 256, K step 32, four waves in a 2 x 2 grid of
// 128 x 128 wave tiles, each a 4 x 4 grid of v_mfma_f32_32x32x16_bf16 with
// 256 fp32 accumulators per lane.  When at most 192 rows remain for the last
// M tile it is 192 x 256 instead (96 x 128 wave tiles, 3 x 4 MFMA blocks),
// so M = 704 does not issue the MFMAs of 768 rows.
//
// Operand staging: the global loads write straight into LDS (buffer loads
// with the LDS destination; lane i of one such load fills bytes 16 i .. 16 i
// + 15 after the wave-uniform base), so no registers hold tiles in flight.
// Four LDS stages form a ring and the loads of step k + 3 are issued during
// step k, between its MFMAs, about three steps of MFMA work ahead of their
// use, spread one per two MFMAs.  The one barrier per step sits in the middle
// of the step's MFMA stream and is preceded by an explicit wait for this
// wave's oldest load group only.
//
// LDS layouts (16-byte chunks, XOR-swizzled so the operand reads below hit
// distinct banks; the swizzle only renames which global chunk a lane fetches):
//   A stage: 256 rows x 64 bytes; chunk c of row r sits at 4 r + (c ^ sa(r)).
//     The MFMA A operand (lane l: row l % 32, 8 consecutive k) is one
//     ds_read_b128.
//   W[N][K] stage: 256 rows (n) x 64 bytes, exactly like A; the MFMA B
//     operand (lane l: column l % 32, 8 consecutive k) is one ds_read_b128.
//   W[K][N] stage: 32 rows (k) x 512 bytes, as stored (n innermost); the
//     32-byte unit u of row r sits at unit u ^ sb(r).  The B operand needs
//     8 consecutive k of one column per lane; gfx950's transposing read
//     ds_read_b64_tr_b16 delivers four at a time: within each 16-lane group,
//     output lane i, element t comes from source lane i/4 + 4t, element i%4,
//     so a source lane j that reads row k0 + j/4, columns n0 + 4 (j%4) .. +3
//     hands lane i the values W[k0 .. k0+3][n0 + i].  A transposing read
//     moves half the bytes of a ds_read_b128 in more LDS cycles, which makes
//     this layout LDS-bound.  Vocabulary sizes that are not a multiple of 8
//     (rows not 16-byte aligned) stage this layout through registers with
//     element loads instead.
//
// Tiles are ordered so that the M tiles of an N tile land on the same XCD
// (workgroups are dealt round-robin over the 8 XCDs), letting them share the
// W tile through that XCD's L2.
#include "sv_kernels.hpp"

#include <limits.h>

namespace sv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 32, NS = 4;
constexpr int kChunksPerStage = BM * BK / 8;      // 1024 16-byte chunks (A and W alike)
constexpr int kLoadsPerWave = kChunksPerStage / 256;  // 4 wave loads of 64 chunks
constexpr int kXcd = 8;
static_assert(BM * BK == BK * BN, "A and W stages have the same size");

// A row r: chunk swizzle (2 bits).  Rows 0..7 of any aligned 8-row group
// (and 0..15 of a 16-row group) land on distinct (row pair, chunk) bank slots.
__device__ __forceinline__ int swz_a(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1); }
// W row r: 32-byte-unit swizzle (3 bits), by r % 4 from {0, 2, 5, 7}.
__device__ __forceinline__ int swz_b(int r) { return (0x7520 >> (4 * (r & 3))) & 0xF; }

// s_waitcnt with only vmcnt = n (gfx9 encoding: expcnt and lgkmcnt at max)
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

// 16-byte buffer load of lane i into LDS bytes lds_base + 16 i ..  Issued
// through asm so that the compiler's wait analysis does not track it: its
// completion is waited for explicitly (wait_vm) before the barrier of the step
// that reads it.  rsrc: wave-uniform buffer descriptor words.
__device__ __forceinline__ void dma16(const v4i& rsrc, uint32_t lds_base, uint32_t voff, uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}

// raw descriptor words: base, stride 0, num_records = bytes, the same
// format word make_rsrc uses
__device__ __forceinline__ v4i rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)p;
}

__device__ __forceinline__ s16x4 lds_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) uint16_t*)p));
}

// W layouts and staging paths of the kernel
constexpr int kWDvElem = 0;  // W[K][N], N % 8 != 0: element loads through registers
constexpr int kWDvDma = 1;   // W[K][N]: LDS-DMA, transposing LDS reads
constexpr int kWVd = 2;      // W[N][K]: LDS-DMA, plain LDS reads (like A)

// Row statistics of one wave tile's 128 columns, in the row sweep's partial
// form: m = the max, K = fl(m c_hi), s = sum 2^(fl(z c_lo + fl(z c_hi - K)))
// with four fp32 accumulators per lane (sixteen terms each) and fp64 from the
// lane up.  A row's 128 columns sit in lanes l and l + 32 (the output layout
// below).  FULL: all 128 columns lie inside V; else the first nv do.
template <int MI, bool FULL>
__device__ __forceinline__ void lmhead_row_stats(const LmHeadParams& P, const f32x16 (&acc)[MI][4], int m0,
                                                 long long n0, long long c0, int wm, int wn, int lane, int nv) {
  const float NEG_INF = -__builtin_huge_valf();
  const float c_hi = P.tc.c_hi, c_lo = P.tc.c_lo;
  const int h = 4 * (lane >> 5);
  const int pidx = (int)(n0 / BN) * 2 + wn;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    float m = NEG_INF;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (FULL || 32 * j + 8 * (r >> 2) + (r & 3) + h < nv) m = fmaxf(m, acc[i][j][r]);
    m = fmaxf(m, __shfl_xor(m, 32));
    float K = 0.f;
    double S = 0.0;
    if (m != NEG_INF) {   // the same in both lanes of a row
      K = m * c_hi;
      float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (FULL || 32 * j + 8 * (r >> 2) + (r & 3) + h < nv) {
            const float z = acc[i][j][r];
            a[r & 3] += __builtin_amdgcn_exp2f(fmaf(z, c_lo, fmaf(z, c_hi, -K)));
          }
      const double sl = ((double)a[0] + (double)a[1]) + ((double)a[2] + (double)a[3]);
      S = sl + __shfl_xor(sl, 32);   // the same sum in both lanes of the row
    }
    const int row = m0 + wm * 32 * MI + i * 32 + (lane & 31);
    if (lane < 32 && row < P.M) {
      LmPartial pp;
      pp.m = m;
      pp.K = K;
      pp.s = S;
      P.part[(long long)row * P.pstride + pidx] = pp;
    }
  }
}

// One workgroup tile: rows m0 .. m0 + 64 MI - 1 of C (MI = 4: 256 rows; MI =
// 3: 192 rows, the last M tile when at most 192 rows remain, so that M = 704
// issues the MFMAs of 704 rows rather than 768), columns n0 .. n0 + 255.
// The four waves form a 2 x 2 grid of (32 MI) x 128 wave tiles.
template <int WL, int MI, bool STATS>
__device__ __forceinline__ void lmhead_tile(const LmHeadParams& P, int m0, long long n0, uint16_t* const* SA,
                                            uint16_t* const* SB, int lane, int wid) {
  constexpr int TM = 64 * MI;                  // rows of the tile
  constexpr int LA = TM * BK / 8 / 256;        // A loads per wave and K step (= MI)
  static_assert(MI == 3 || MI == 4, "tile heights 192 and 256");
  const int wm = wid >> 1, wn = wid & 1;
  const int M = P.M, K = P.K;
  const long long N = P.N;

  // A rows past M read as zero through the descriptor bound (row-major A),
  // or as the zeros the staging wrote (staged A: the tile's blocks of 256
  // rows x 64 bytes, one per K step)
  const bool staged = P.a_staged != 0;
  const int arows = min(TM, M - m0);
  const v4i ra = staged ? rsrc_words(P.A + (long long)(m0 / BM) * (K / BK) * (BM * BK), (uint32_t)((K / BK) * BM * BK * 2))
                        : rsrc_words(P.A + (long long)m0 * K, (uint32_t)((long long)arows * K * 2));
  const uint32_t arow_bytes = staged ? (uint32_t)(BK * 2) : (uint32_t)K * 2u;   // A row stride
  const uint32_t astep_bytes = staged ? (uint32_t)(BM * BK * 2) : (uint32_t)(BK * 2);   // per K step
  const uint16_t* const wtile = P.W + n0;
  const long long wtotal = (long long)K * N - n0;  // elements of W from wtile on

  // Chunk p of a stage (p = 64 (L wid + t) + lane, L loads per wave) is what
  // this lane fetches in its t-th load of the step: aoff for the A stage (LA
  // loads), voff for a W[N][K] stage and boff for a W[K][N] stage (four
  // loads each).
  uint32_t aoff[LA], voff[kLoadsPerWave], boff[kLoadsPerWave];
#pragma unroll
  for (int t = 0; t < LA; ++t) {
    const int p = (wid * LA + t) * 64 + lane;
    const int ra_ = p >> 2, pca = p & 3;
    aoff[t] = (uint32_t)ra_ * arow_bytes + (uint32_t)(16 * (pca ^ swz_a(ra_)));
  }
#pragma unroll
  for (int t = 0; t < kLoadsPerWave; ++t) {
    const int p = (wid * kLoadsPerWave + t) * 64 + lane;
    const int ra_ = p >> 2, pca = p & 3;
    voff[t] = (uint32_t)(ra_ * K * 2 + 16 * (pca ^ swz_a(ra_)));
    const int rb = p >> 5, pcb = p & 31;
    const int cb = 2 * ((pcb >> 1) ^ swz_b(rb)) + (pcb & 1);  // logical chunk of that slot
    boff[t] = (uint32_t)((long long)rb * N * 2 + 16 * cb);
  }

  // load q (0..LA-1: A chunks, LA..LA+3: W chunks) of K step ks into ring
  // slot S; rb = the W descriptor of that step
  auto issue_one = [&](auto Sc, int ks, int q, const v4i& rb) {
    constexpr int S = decltype(Sc)::value;
    const int k0 = ks * BK;
    if (q < LA) {
      dma16(ra, lds_addr(SA[S] + (wid * LA + q) * 512), aoff[q], (uint32_t)ks * astep_bytes);
    } else if (WL == kWDvDma) {
      const int t = q - LA;
      dma16(rb, lds_addr(SB[S] + (wid * kLoadsPerWave + t) * 512), boff[t], 0u);
    } else if (WL == kWVd) {
      // rows n0 .. n0 + 255 of W[N][K]: the same row layout and swizzle as A
      const int t = q - LA;
      dma16(rb, lds_addr(SB[S] + (wid * kLoadsPerWave + t) * 512), voff[t], (uint32_t)k0 * 2u);
    } else if (q == LA) {
      // element loads of the whole W stage; columns past N read as zero
      const long long kbase = (long long)k0 * N;
#pragma unroll
      for (int t = 0; t < kLoadsPerWave; ++t) {
        const int p = (wid * kLoadsPerWave + t) * 64 + lane;
        const int rb_ = p >> 5, pcb = p & 31;
        const int cb = 2 * ((pcb >> 1) ^ swz_b(rb_)) + (pcb & 1);
        const long long gn = n0 + 8 * cb;
        const uint16_t* src = wtile + kbase + (long long)rb_ * N + 8 * cb;
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = gn + i < N ? src[i] : (uint16_t)0;
        v4i v;
        v[0] = (int)(e[0] | ((uint32_t)e[1] << 16));
        v[1] = (int)(e[2] | ((uint32_t)e[3] << 16));
        v[2] = (int)(e[4] | ((uint32_t)e[5] << 16));
        v[3] = (int)(e[6] | ((uint32_t)e[7] << 16));
        *reinterpret_cast<v4i*>(SB[S] + p * 8) = v;
      }
    }
  };
  auto w_rsrc = [&](int ks) {
    // W[N][K]: one descriptor for the tile's rows (rows past N read as zero)
    if (WL == kWVd) return rsrc_words(P.W + n0 * K, (uint32_t)(min((long long)BN, N - n0) * K * 2));
    // W[K][N]: K step ks of this tile's columns
    const long long kbase = (long long)ks * BK * N;
    return rsrc_words(wtile + kbase, (uint32_t)min((wtotal - kbase) * 2, (long long)BK * N * 2));
  };

  f32x16 acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // A operand: row wm*32*MI + 32 i + (lane % 32), chunk kk/8 + lane/32; the
  // row's swizzle only depends on lane % 16
  const int arow = lane & 31, achk = lane >> 5, asw = swz_a(arow);
  // B operand (16-lane group g, lane jl in it): rows kk + 8 (g/2) + jl/4
  // (+4 for the second read), unit wn*8 + 2 j + (g % 2), bytes 8 (jl % 4)
  const int g = lane >> 4, jl = lane & 15;
  const int brow = 8 * (g >> 1) + (jl >> 2);
  const int bsw = swz_b(brow);
  int bofs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bofs[j] = brow * BN + 16 * (wn * 8 + ((2 * j + (g & 1)) ^ bsw)) + 4 * (jl & 3);

  // operand fragments: set 0 holds the k sub-step kk = 0 of a K step, set 1
  // the sub-step kk = 16
  bf16x8 fa[2][MI], fb[2][4];
  // fragment pair idx of sub-step H: A rows wm*32*MI + 32 idx.. (idx < MI),
  // W columns wn*128 + 32 idx..
  auto read_pair = [&](auto Sc, auto Hc, int idx) {
    constexpr int S = decltype(Sc)::value, H = decltype(Hc)::value, kk = 16 * H;
    const uint16_t* As = SA[S];
    const uint16_t* Bs = SB[S];
    const int ac = ((kk >> 3) + achk) ^ asw;
    if (idx < MI) fa[H][idx] = *reinterpret_cast<const bf16x8*>(As + (wm * 32 * MI + idx * 32 + arow) * BK + ac * 8);
    if (WL == kWVd) {
      fb[H][idx] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 128 + idx * 32 + arow) * BK + ac * 8);
    } else {
      const uint16_t* p = Bs + kk * BN + bofs[idx];
      const s16x4 lo = lds_tr16(p);
      const s16x4 hi = lds_tr16(p + 4 * BN);
      s16x4 both[2] = {lo, hi};
      fb[H][idx] = *reinterpret_cast<const bf16x8*>(both);
    }
  };
  auto read_frags = [&](auto Sc, auto Hc) {
#pragma unroll
    for (int idx = 0; idx < 4; ++idx) read_pair(Sc, Hc, idx);
  };
  auto mfma = [&](auto Hc, int q) {
    constexpr int H = decltype(Hc)::value;
    const int i = q >> 2, j = q & 3;
    // W fragment as the MFMA's first operand: acc[i][j] holds the 32 x 32
    // block transposed, vocabulary along the registers (see the epilogue)
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[H][j], fa[H][i], acc[i][j], 0, 0, 0);
  };
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;

  // loads in flight per K step and wave (the element path waits for its own
  // W loads, leaving only the A loads)
  constexpr int kGroup = WL == kWDvElem ? LA : LA + kLoadsPerWave;
  constexpr int kMf = 4 * MI;                  // MFMAs per wave and K sub-step
  constexpr int kPairs = MI == 4 ? 12 : 9;     // MFMA / LDS-read pairs of the first half
  const int nk = K / BK;

  // One K step in two halves.  First half: the kk = 0 MFMAs, while the
  // kk = 16 fragments of this step are read.  Then the barrier that releases
  // K step ks + 1 (every wave is past step ks - 1 there, so ring slot
  // (ks + 3) % 4 is free too).  Second half: the kk = 16 MFMAs, with the
  // loads of step ks + 3 and the kk = 0 fragments of step ks + 1 issued
  // between them, so the MFMA pipe does not wait on a barrier or an LDS read.
  // Past the last K step the loads re-fetch that step into the free slot
  // (never read) and the fragment reads fetch unused data: the wait counts
  // stay the same on every step and the stream has no branches.
  auto step = [&](auto Sc, int ks) {
    constexpr int S = decltype(Sc)::value;
    read_frags(Sc, H1{});
#pragma unroll
    for (int q = 0; q < kMf; ++q) mfma(H0{}, q);
    // interleave: one MFMA, one LDS read, kPairs times; then the other MFMAs
#pragma unroll
    for (int r = 0; r < kPairs; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMf - kPairs, 0);
    __builtin_amdgcn_sched_barrier(0);
    // this wave's loads of step ks + 1 are done once at most the group of
    // step ks + 2 remains outstanding
    wait_vm<kGroup>();
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const int kl = min(ks + 3, nk - 1);
    const v4i rb = w_rsrc(kl);
    // the loads go out one per two MFMAs so the texture address unit sees a
    // steady stream (a load that finds its queue full stalls this wave's
    // MFMA issue behind it); the fragment reads fill the odd slots
#pragma unroll
    for (int q = 0; q < kMf; ++q) {
      mfma(H1{}, q);
      if ((q & 1) == 0) {
        __builtin_amdgcn_sched_barrier(0);
        issue_one(std::integral_constant<int, (S + 3) % NS>{}, kl, q >> 1, rb);
        __builtin_amdgcn_sched_barrier(0);
      } else if (q < 8) {
        read_pair(std::integral_constant<int, (S + 1) % NS>{}, H0{}, q >> 1);
      }
    }
    // loads left over when the step has fewer MFMA slots than loads (MI = 3)
#pragma unroll
    for (int e = kMf / 2; e < LA + kLoadsPerWave; ++e)
      issue_one(std::integral_constant<int, (S + 3) % NS>{}, kl, e, rb);
    __builtin_amdgcn_sched_barrier(0);
  };

  {
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    const int k1 = min(1, nk - 1), k2 = min(2, nk - 1);
    const v4i r0 = w_rsrc(0);
#pragma unroll
    for (int q = 0; q < LA + kLoadsPerWave; ++q) issue_one(S0{}, 0, q, r0);
    const v4i r1 = w_rsrc(k1);
#pragma unroll
    for (int q = 0; q < LA + kLoadsPerWave; ++q) issue_one(S1{}, k1, q, r1);
    const v4i r2 = w_rsrc(k2);
#pragma unroll
    for (int q = 0; q < LA + kLoadsPerWave; ++q) issue_one(S2{}, k2, q, r2);
    wait_vm<2 * kGroup>();
    asm volatile("s_barrier" ::: "memory");
    read_frags(S0{}, H0{});
  }
  for (int ks = 0; ks < nk; ks += NS) {
    step(std::integral_constant<int, 0>{}, ks);
    if (ks + 1 < nk) step(std::integral_constant<int, 1>{}, ks + 1);
    if (ks + 2 < nk) step(std::integral_constant<int, 2>{}, ks + 2);
    if (ks + 3 < nk) step(std::integral_constant<int, 3>{}, ks + 3);
  }
  // no load may still be writing LDS when the workgroup ends
  wait_vm<0>();

  // Output layout (W fragment first): lane l holds feature row l % 32 of
  // block i and the vocabulary columns 8 q + 4 (l / 32) + t of block j in
  // registers 4 q + t (q, t = 0..3), so each group of four registers is four
  // consecutive logits of one row.  When the wave's 128 columns lie inside V
  // and rows keep 16-byte alignment (V % 4 == 0; C is 16-byte aligned), each
  // group is one 16-byte store; otherwise (a ragged last tile) element stores.
  const long long c0 = n0 + wn * 128;
  const bool vec = (N & 3) == 0 && c0 + 128 <= N;   // uniform per wave
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int row = m0 + wm * 32 * MI + i * 32 + (lane & 31);
    if (row >= M) continue;
    float* const crow = P.C + (long long)row * N + c0 + 4 * (lane >> 5);
    if (vec) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = acc[i][j][4 * q + t];
          *reinterpret_cast<f32x4*>(crow + j * 32 + 8 * q) = v;
        }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const long long col = c0 + j * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (col < N) crow[j * 32 + 8 * (r >> 2) + (r & 3)] = acc[i][j][r];
        }
    }
  }

  // Row statistics of the wave's 128 columns, in the row sweep's partial
  // form: m = the max, K = fl(m c_hi), s = sum 2^(fl(z c_lo + fl(z c_hi - K)))
  // with four fp32 accumulators per lane (sixteen terms each) and fp64 from
  // the lane up.  A row's 128 columns sit in lanes l and l + 32.
  if constexpr (STATS) {
    // lane l's column offsets inside the wave tile are 32 j + 8 q + t + h,
    // h = 4 (l / 32); nv of the 128 columns lie inside V (wave-uniform)
    const long long rem = N - c0;
    const int nv = rem >= 128 ? 128 : (rem > 0 ? (int)rem : 0);
    if (nv == 128) lmhead_row_stats<MI, true>(P, acc, m0, n0, c0, wm, wn, lane, nv);
    else lmhead_row_stats<MI, false>(P, acc, m0, n0, c0, wm, wn, lane, nv);
  }
}

template <int WL, bool STATS>
__global__ __launch_bounds__(256) void k_lmhead(LmHeadParams P, int mtiles, int ntiles) {
  // one LDS object per ring slot: the A stage, then the W stage
  __shared__ __attribute__((aligned(1024))) uint16_t s0[2 * BM * BK], s1[2 * BM * BK], s2[2 * BM * BK],
      s3[2 * BM * BK];
  uint16_t* const SA[NS] = {s0, s1, s2, s3};
  uint16_t* const SB[NS] = {s0 + BM * BK, s1 + BM * BK, s2 + BM * BK, s3 + BM * BK};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware tile order: slot s on XCD x takes N tile (s / mtiles) * 8 + x
  const int w = blockIdx.x;
  const int xcd = w % kXcd, slot = w / kXcd;
  const int mt = slot % mtiles;
  const int nt = (slot / mtiles) * kXcd + xcd;
  if (nt >= ntiles) return;
  const int m0 = mt * BM;
  const long long n0 = (long long)nt * BN;
  if (P.M - m0 <= 192) lmhead_tile<WL, 3, STATS>(P, m0, n0, SA, SB, lane, wid);   // uniform
  else lmhead_tile<WL, 4, STATS>(P, m0, n0, SA, SB, lane, wid);
}

// One workgroup per row: the row's GEMM partials merged in fp64, as the
// sampling kernels merge row-sweep partials (M = the max of the partial
// maxima, S = sum s 2^(K - M c)), stored as one partial with K = fl(M c_hi)
// and s = S 2^(M c - K).  Each thread holds up to kMergeRun partials per
// pass, all loaded before use; a second pass reads them again (cache-hot) for
// the sum.  Thread 0 first gathers the drafted token's logit of the row.
constexpr int kMergeRun = 4;

__global__ __launch_bounds__(256) void k_lmhead_merge(LmHeadMergeParams P) {
  __shared__ float sh_m[4];
  __shared__ double sh_s[4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const long long r = blockIdx.x;
  const float NEG_INF = -__builtin_huge_valf();
  if (tid == 0 && P.tokens != nullptr) {
    const long long rows_t = (long long)P.B * (P.g + 1);
    int x = -1;
    if (r < rows_t) {
      const int b = (int)(r / (P.g + 1)), i = (int)(r % (P.g + 1));
      if (i < P.g) x = P.tokens[(long long)b * P.g + i];
    } else {
      x = P.tokens[r - rows_t];               // draft rows follow the tokens' [B, g] order
    }
    if (x >= 0 && (long long)x < P.N) P.gathered[r] = P.C[r * P.N + x];
  }
  const LmPartial* pr = P.part + r * P.nparts;
  const int n = P.nparts;
  float m = NEG_INF;
  for (int base = 0; base < n; base += kMergeRun * 256) {
    float pm[kMergeRun];
#pragma unroll
    for (int k = 0; k < kMergeRun; ++k) {
      const int t = base + k * 256 + tid;
      pm[k] = t < n ? pr[t].m : NEG_INF;
    }
#pragma unroll
    for (int k = 0; k < kMergeRun; ++k) m = fmaxf(m, pm[k]);
  }
  m = wave_max(m);
  if (lane == 0) sh_m[wid] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(sh_m[0], sh_m[1]), fmaxf(sh_m[2], sh_m[3]));
  double sv = 0.0;
  if (M != NEG_INF) {
    const double Mc = (double)M * P.tc.c64;
    for (int base = 0; base < n; base += kMergeRun * 256) {
      LmPartial pp[kMergeRun];
#pragma unroll
      for (int k = 0; k < kMergeRun; ++k) {
        const int t = base + k * 256 + tid;
        if (t < n) {
          pp[k] = pr[t];
        } else {
          pp[k].m = NEG_INF;
          pp[k].K = 0.f;
          pp[k].s = 0.0;
        }
      }
#pragma unroll
      for (int k = 0; k < kMergeRun; ++k)
        if (pp[k].m != NEG_INF) sv += pp[k].s * exp2_f64((double)pp[k].K - Mc);
    }
  }
  sv = wave_sum(sv);
  if (lane == 0) sh_s[wid] = sv;
  __syncthreads();
  if (tid == 0) {
    const double S = (sh_s[0] + sh_s[1]) + (sh_s[2] + sh_s[3]);
    Partial o;
    o.m = M;
    o.arg = INT_MAX;
    o.pad_ = 0.f;
    o.K = 0.f;
    o.s = 0.0;
    if (M != NEG_INF) {
      o.K = M * P.tc.c_hi;
      o.s = S * exp2_f64((double)M * P.tc.c64 - (double)o.K);
    }
    P.out[r] = o;
  }
}

// One 16-byte chunk per thread: chunk q of the staged buffer is chunk q % 4
// of row (q / 4) % 256 of block q / 1024 (block = M tile * K/32 + K step).
// The writes are contiguous; each row's four chunks are one 64-byte read.
__global__ __launch_bounds__(256) void k_lmhead_stage(LmHeadStageParams P) {
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
  const int nk = P.K / BK;
  const long long blk = q >> 10;
  if (blk >= (long long)((P.M + BM - 1) / BM) * nk) return;
  const int c = (int)(q & 3), r = (int)((q >> 2) & (BM - 1));
  const long long mt = blk / nk;
  const int ks = (int)(blk - mt * nk);
  const long long m = mt * BM + r;
  v4i v = {0, 0, 0, 0};
  if (m < P.M) {
    const uint16_t* src = m < P.rows0 ? P.src0 + m * P.K : P.src1 + (m - P.rows0) * P.K;
    v = *reinterpret_cast<const v4i*>(src + ks * BK + c * 8);
  }
  *reinterpret_cast<v4i*>(P.dst + q * 8) = v;
}

}  // namespace

size_t lmhead_staged_bytes(long long M, long long K) {
  return (size_t)((M + BM - 1) / BM) * (size_t)(K / BK) * BM * BK * 2;
}

hipError_t launch_lmhead_stage(const LmHeadStageParams& p, hipStream_t s) {
  if (p.K % BK != 0 || p.K < BK || p.M < 1 || p.rows0 < 0 || p.rows0 > p.M) return hipErrorInvalidValue;
  const long long chunks = (long long)lmhead_staged_bytes(p.M, p.K) / 16;
  const long long blocks = (chunks + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_lmhead_stage, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_lmhead(const LmHeadParams& p, hipStream_t s) {
  if (p.K % BK != 0 || p.K < BK || p.M < 1 || p.N < 1) return hipErrorInvalidValue;
  const long long nt = ((long long)p.N + BN - 1) / BN;
  const long long mt = ((long long)p.M + BM - 1) / BM;
  const long long per_xcd = (nt + kXcd - 1) / kXcd;
  const long long grid = per_xcd * mt * kXcd;
  // 32-bit buffer offsets: one A tile, one W tile, one K step of W[K][N]
  if (grid > 0x7fffffffLL || (long long)BM * p.K * 2 >= (1LL << 32)) return hipErrorInvalidValue;
  if (!p.w_vd && (long long)BK * p.N * 2 >= (1LL << 32)) return hipErrorInvalidValue;
  if (p.part != nullptr && p.pstride < lmhead_stat_parts(p.N)) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), b(256);
  if (p.part != nullptr) {
    if (p.w_vd)
      hipLaunchKernelGGL((k_lmhead<kWVd, true>), g, b, 0, s, p, (int)mt, (int)nt);
    else if (p.N % 8 == 0)
      hipLaunchKernelGGL((k_lmhead<kWDvDma, true>), g, b, 0, s, p, (int)mt, (int)nt);
    else
      hipLaunchKernelGGL((k_lmhead<kWDvElem, true>), g, b, 0, s, p, (int)mt, (int)nt);
  } else if (p.w_vd) {
    hipLaunchKernelGGL((k_lmhead<kWVd, false>), g, b, 0, s, p, (int)mt, (int)nt);
  } else if (p.N % 8 == 0) {  // rows of W[K][N] start 16-byte aligned
    hipLaunchKernelGGL((k_lmhead<kWDvDma, false>), g, b, 0, s, p, (int)mt, (int)nt);
  } else {
    hipLaunchKernelGGL((k_lmhead<kWDvElem, false>), g, b, 0, s, p, (int)mt, (int)nt);
  }
  return hipGetLastError();
}

hipError_t launch_lmhead_merge(const LmHeadMergeParams& p, hipStream_t s) {
  if (p.M < 1 || p.nparts < 1 || p.part == nullptr || p.out == nullptr) return hipErrorInvalidValue;
  if (p.tokens != nullptr && (p.C == nullptr || p.gathered == nullptr || p.g < 1)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_lmhead_merge, dim3((unsigned)p.M), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace sv
