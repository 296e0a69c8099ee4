// KV-cache compaction to the accepted path.
//
// Pages: "EAGLE-3 speculative decoding review", "The Complete EAGLE-3
// Inference Process" (5. Update the KV Cache: keep the accepted path's
// cache, drop rejected branches, resume from the committed prefix) and
// "Implementation Is More Complex Than a Simple Two-Model Setup" (the
// serving side prunes the KV cache to the accepted branch).
//
// The verification forward left node n's entry at slot L_b + n (node 0 is
// the root, the last committed token).  The accepted path n_1 < ... < n_d
// moves to slots L_b + 1 .. L_b + d; the new length is L_b + 1 + d.
//
// One kernel, one thread per (sequence, plane, 16-byte column of an entry).
// Every thread checks its sequence's path (it must rise strictly from 1 and
// stay inside the cache; a short, cached read, eight entries per round
// trip) and thread (plane 0, column 0) writes new_len (or -1).  Then the
// thread walks the path in depth order and moves its column of node n_t's
// entry to slot L_b + t.  A thread owns
// the same column of every entry of its (sequence, plane), so the one
// overlap -- a slot read at depth t and written at a later depth t' (when
// n_t = t') -- is ordered by the thread's own program order; a slot written
// at depth t is never read afterwards, because n_t' > n_t >= t for t' > t.
// Up to 8 depths are loaded before they are stored; columns whose node
// already sits in place (n_t = t) are skipped.
// Purely a gather-copy: HBM-bound, 32 bytes of traffic per moved 16-byte
// column.
#include "sv_kernels.hpp"

namespace sv {

namespace {

constexpr int kKvBlock = 256;
constexpr int kKvBatch = 8;

__global__ __launch_bounds__(kKvBlock) void k_kv_compact(KvParams P) {
  const long long cpe = P.entry_bytes / 16;
  const long long i = (long long)blockIdx.x * kKvBlock + threadIdx.x;
  const long long c = i % cpe;
  const long long bp = i / cpe;
  const int p = (int)(bp % P.planes);
  const long long b = bp / P.planes;
  if (b >= P.B) return;
  const int L = P.prefix_len[b], d = P.accept_len[b];
  const int32_t* pp = P.path ? P.path + b * P.path_stride : nullptr;
  bool ok = d >= 0 && L >= 0 && (long long)L + 1 + d <= P.S;
  if (ok && pp) {
    // batches of independent loads, then the comparisons (no early exit
    // between the loads of a batch)
    ok = d <= P.path_stride;
    int prev = 0;
    for (int t0 = 0; ok && t0 < d; t0 += kKvBatch) {
      int n[kKvBatch];
#pragma unroll
      for (int k = 0; k < kKvBatch; ++k) n[k] = t0 + k < d ? pp[t0 + k] : 0;
#pragma unroll
      for (int k = 0; k < kKvBatch; ++k) {
        if (t0 + k < d) {
          ok = ok && n[k] > prev;
          prev = n[k];
        }
      }
    }
    ok = ok && (long long)L + prev < P.S;
  }
  if (p == 0 && c == 0) P.new_len[b] = ok ? L + 1 + d : -1;
  if (!ok || !pp) return;
  char* const col = P.kv + b * P.seq_stride + (long long)p * P.plane_stride + c * 16;
  for (int t0 = 0; t0 < d; t0 += kKvBatch) {
    v4i v[kKvBatch];
    int n[kKvBatch];
#pragma unroll
    for (int k = 0; k < kKvBatch; ++k) {
      n[k] = t0 + k < d ? pp[t0 + k] : 0;
      if (t0 + k < d && n[k] != t0 + k + 1)
        v[k] = *reinterpret_cast<const v4i*>(col + (long long)(L + n[k]) * P.entry_bytes);
    }
#pragma unroll
    for (int k = 0; k < kKvBatch; ++k)
      if (t0 + k < d && n[k] != t0 + k + 1)
        *reinterpret_cast<v4i*>(col + (long long)(L + t0 + k + 1) * P.entry_bytes) = v[k];
  }
}

}  // namespace

hipError_t launch_kv_compact(const KvParams& p, hipStream_t s) {
  // without a path nothing moves: one thread per sequence writes new_len
  const long long per_seq = p.path ? (long long)p.planes * (p.entry_bytes / 16) : 1;
  const long long blocks = ((long long)p.B * per_seq + kKvBlock - 1) / kKvBlock;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  KvParams q = p;
  if (!p.path) {
    q.planes = 1;
    q.entry_bytes = 16;
  }
  hipLaunchKernelGGL(k_kv_compact, dim3((unsigned)blocks), dim3(kKvBlock), 0, s, q);
  return hipGetLastError();
}

}  // namespace sv
