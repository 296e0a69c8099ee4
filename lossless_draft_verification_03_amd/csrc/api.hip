// C ABI of libspecverify: argument checks, workspace layout, launches.
// Every entry point validates its arguments before it launches anything and
// never throws; see include/specverify.h for the contract of each call.
#include "specverify.h"

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "sv_kernels.hpp"

using namespace sv;

static_assert(SPEC_MAX_TREE_NODES == kTreeMaxNodes, "tree size limit of the walk kernel");
static_assert((long long)SPEC_MAX_SAMPLE_VOCAB == kMaxSampleVocab, "vocabulary limit of the draw kernels");
static_assert(SPEC_MAX_TREE_ROUNDS == kTreeMaxRounds, "round limit of the tree sampler");

namespace {

constexpr size_t kAlign = 256;

size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Workspace regions; all offsets are from the workspace base.  Every region
// is fully written before it is read within one call, so a workspace needs
// no initialisation and can be shared by calls of any layout (one at a time).
struct Layout {
  size_t info, part, rmax, rsum, rarg, gath, segsum, gpart, hcat, logits, total;
  size_t tstate, tglog, twpart;        // tree sampler: walk states, token logits, W sums
  long long rows;
  int nseg, nseg2;
};

// Nodes whose rows the tree sampler sweeps before its walk.  n_sweep >= 0
// is the caller's choice (at most N); -1 picks as many leading nodes as fit
// about kTreePresweepBytes of target and draft rows.  A walk reaches a node
// beyond the prefix one round later, and a round costs about what sweeping
// this many bytes does (measured on 32 trees of 63 nodes at V = 128256, bf16:
// 4 nodes, against 0 to 10).
constexpr long long kTreePresweepBytes = 64LL << 20;

// Chip-wide rounds of a tree-sampling call when the caller leaves it open:
// a round costs about 2.5 us when no walk needs it, while a pass left to the
// finishing kernel costs one CU about 20 us, so enough rounds for the walks
// of the usual tree shapes (a visit beyond the prefix and a W pass per
// level), at most one per node beyond the root.
int tree_auto_rounds(int N) {
  const int r = 8;
  return N - 1 < r ? (N - 1 > 0 ? N - 1 : 0) : r;
}

long long tree_presweep_nodes(long long B, long long N, long long V, int dt, long long n_sweep) {
  if (n_sweep >= 0) return n_sweep < N ? n_sweep : N;
  const long long pair = 2 * V * (dt == DT_BF16 ? 2 : 4);
  const long long n = kTreePresweepBytes / (B * pair);
  return n < N ? n : N;
}

// dt = element type of the rows the sweep reads (the sweep's segment count
// depends on it); the public size query takes the larger (fp32) layout.
bool make_layout(int mode, long long B, long long gN, long long V, long long d, int dt, Layout* L) {
  memset(L, 0, sizeof(*L));
  if (B < 1 || B > SPEC_MAX_BATCH || V < 1 || V > 0x7fffffffLL) return false;
  long long rows = 0, seqs = 0;
  switch (mode) {
    case SPEC_MODE_SAMPLE:
    case SPEC_MODE_LMHEAD:
      if (gN < 1 || gN > SPEC_MAX_GAMMA) return false;
      rows = B * (2 * gN + 1);
      seqs = B;
      break;
    case SPEC_MODE_GREEDY:
      if (gN < 1 || gN > SPEC_MAX_GAMMA) return false;
      rows = B * (gN + 1);
      break;
    case SPEC_MODE_TREE:
      if (gN < 1 || gN > SPEC_MAX_TREE_NODES) return false;
      rows = B * gN;
      break;
    case SPEC_MODE_TREE_SAMPLE: {
      // the walk's per-sequence partials of one target and one draft row
      // (two buffers, alternating between rounds), then those of the swept
      // prefix (d carries the call's n_sweep); sized for whichever element
      // type needs more
      if (gN < 1 || gN > SPEC_MAX_TREE_NODES || d < -1 || d > gN) return false;
      long long pre = 0;
      for (int t = 0; t < 2; ++t) {
        const long long need =
            2 * B * tree_presweep_nodes(B, gN, V, t, d) * row_sweep_shape((int)V, t, kTreeSampleVPT).nseg;
        if (need > pre) pre = need;
      }
      rows = 4 * B + (pre + row_sweep_shape((int)V, DT_F32, kTreeSampleVPT).nseg - 1) /
                         row_sweep_shape((int)V, DT_F32, kTreeSampleVPT).nseg;
      break;
    }
    case SPEC_MODE_ROWSTATS:
      rows = B;
      break;
    default:
      return false;
  }
  if (mode == SPEC_MODE_LMHEAD) {
    if (d < 64 || d % 64 != 0 || d > (1 << 20)) return false;
    dt = DT_F32;
  }
  if (mode == SPEC_MODE_TREE_SAMPLE) dt = DT_F32;
  // greedy and greedy-tree verification sweep with the argmax-only segments,
  // the tree sampler with its own
  const int vpt = (mode == SPEC_MODE_GREEDY || mode == SPEC_MODE_TREE) ? kArgmaxVPT
                  : mode == SPEC_MODE_TREE_SAMPLE                        ? kTreeSampleVPT
                                                                         : 0;
  const RowSweepShape sh = row_sweep_shape((int)V, dt, vpt);
  int seg_elems = 0;
  // fp32 rows take the most draw segments
  const int nseg2 = seqs ? sample_draw_segments((int)V, DT_F32, &seg_elems) : 0;
  size_t o = 0;
  L->info = o;   o = up(o + (size_t)seqs * sizeof(DrawInfo));
  L->part = o;   o = up(o + (size_t)rows * sh.nseg * sizeof(Partial));
  L->rmax = o;   o = up(o + (size_t)rows * 4);
  L->rsum = o;   o = up(o + (size_t)rows * 8);
  L->rarg = o;   o = up(o + (size_t)rows * 4);
  L->gath = o;   o = up(o + (size_t)rows * 4);
  // the linear draw's sub-segment masses; the tree walk's in the tree sampler
  const size_t segsum_bytes = mode == SPEC_MODE_TREE_SAMPLE ? (size_t)B * tree_segments(V) * kDrawSub * 8
                                                            : (size_t)seqs * nseg2 * kDrawSub * 8;
  L->segsum = o; o = up(o + segsum_bytes);
  if (mode == SPEC_MODE_TREE_SAMPLE) {
    L->tstate = o; o = up(o + (size_t)2 * B * sizeof(TreeWalkState));
    L->tglog = o;  o = up(o + (size_t)B * gN * 2 * 4);
    L->twpart = o; o = up(o + (size_t)2 * B * tree_segments(V) * 3 * 8);
  }
  // the LM head's per-row partials (its GEMM epilogue's row statistics)
  L->gpart = o;
  if (mode == SPEC_MODE_LMHEAD) o = up(o + (size_t)rows * lmhead_stat_parts(V) * sizeof(LmPartial));
  L->hcat = o;
  if (mode == SPEC_MODE_LMHEAD) o = up(o + lmhead_staged_bytes(rows, d));
  L->logits = o;
  if (mode == SPEC_MODE_LMHEAD) o = up(o + (size_t)rows * (size_t)V * 4);
  L->total = o;
  L->rows = rows;
  L->nseg = sh.nseg;
  L->nseg2 = nseg2;
  return true;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool temp_const(float T, TempConst* tc) {
  if (!(T > 0.0f) || !isfinite(T)) return false;
  const double c = 1.4426950408889634074 / (double)T;   // log2(e) / T
  if (!(c < 1e30)) return false;
  float hi = (float)c;
  if ((double)hi >= c) hi = nextafterf(hi, 0.0f);
  tc->c_hi = hi;
  tc->c_lo = (float)(c - (double)hi);
  if (!(tc->c_lo > 0.0f)) tc->c_lo = 1e-30f;
  tc->d_min = (float)(-200.0 / (double)hi);
  tc->pad_ = 0.f;
  tc->c64 = c;
  return true;
}

spec_status hip_status(hipError_t e) { return e == hipSuccess ? SPEC_OK : SPEC_EHIP; }

bool dtype_ok(spec_dtype dt) { return dt == SPEC_F32 || dt == SPEC_BF16; }

int elem_size(spec_dtype dt) { return dt == SPEC_BF16 ? 2 : 4; }

bool row_bytes_ok(long long V, spec_dtype dt) { return V * elem_size(dt) < (1LL << 31); }

spec_status check_ws(void* ws, size_t ws_bytes, const Layout& L) {
  if (!ws || !aligned(ws, kAlign)) return SPEC_EWORKSPACE;
  if (ws_bytes < L.total) return SPEC_EWORKSPACE;
  return SPEC_OK;
}

// Sweep only (partials in the workspace), or sweep + merge into L's
// per-row arrays when `merge` is set.
hipError_t row_sweep(const void* src0, long long rows0, const void* src1, long long rows1, int V,
                     int dt, int want, const TempConst& tc, void* ws, const Layout& L, hipStream_t s,
                     bool merge = false, int vpt = 0) {
  RowStatsParams p;
  memset(&p, 0, sizeof(p));
  const RowSweepShape sh = row_sweep_shape(V, dt, vpt);
  p.src0 = src0;
  p.src1 = src1;
  p.rows0 = rows0;
  p.rows1 = rows1;
  p.V = V;
  p.nseg = sh.nseg;
  p.seg_vecs = sh.seg_vecs;
  p.want = want;
  p.vpt = vpt;
  p.tc = tc;
  p.part = at<Partial>(ws, L.part);
  p.out_max = at<float>(ws, L.rmax);
  p.out_sum = at<double>(ws, L.rsum);
  p.out_arg = at<int>(ws, L.rarg);
  return merge ? launch_row_stats(p, dt, s) : launch_row_sweep(p, dt, s);
}

// Sweep parameters of the sampling path (target rows, then draft rows; the
// drafted tokens' logits gathered on the way).
RowStatsParams sample_sweep_params(const void* tgt, const void* drf, const int32_t* tokens, int B, int g, int V,
                                   int dt, const TempConst& tc, void* ws, const Layout& L) {
  RowStatsParams r;
  memset(&r, 0, sizeof(r));
  const RowSweepShape sh = row_sweep_shape(V, dt);
  r.src0 = tgt;
  r.src1 = drf;
  r.rows0 = (long long)B * (g + 1);
  r.rows1 = (long long)B * g;
  r.V = V;
  r.nseg = sh.nseg;
  r.seg_vecs = sh.seg_vecs;
  r.want = 1;
  r.tc = tc;
  r.part = at<Partial>(ws, L.part);
  r.gather_tokens = tokens;
  r.gather_g = g;
  r.gather_out = at<float>(ws, L.gath);
  return r;
}

// Accept scan and final draw on the partials the sweep left in the workspace.
// nseg_rows: partials per row (-1: the row sweep's segments).
spec_status draw_on(const void* tgt, const void* drf, int dt, const int32_t* tokens, const float* unif, int B,
                    int g, int V, const TempConst& tc, int32_t* accept_len, int32_t* out_tokens, void* ws,
                    const Layout& L, hipStream_t s, int nseg_rows = -1) {
  SampleParams p;
  memset(&p, 0, sizeof(p));
  p.tgt = tgt;
  p.drf = drf;
  p.tokens = tokens;
  p.unif = unif;
  p.part = at<Partial>(ws, L.part);
  p.nseg_rows = nseg_rows > 0 ? nseg_rows : row_sweep_shape(V, dt).nseg;
  p.gathered = at<float>(ws, L.gath);
  p.B = B;
  p.g = g;
  p.V = V;
  p.nseg = sample_draw_segments(V, dt, &p.seg_elems);
  p.tc = tc;
  p.info = at<DrawInfo>(ws, L.info);
  p.segsum = at<double>(ws, L.segsum);
  p.accept_len = accept_len;
  p.out_tokens = out_tokens;
  return hip_status(launch_sample(p, dt, s));
}

spec_status sample_on(const void* tgt, const void* drf, int dt, const int32_t* tokens,
                      const float* unif, int B, int g, int V, const TempConst& tc,
                      int32_t* accept_len, int32_t* out_tokens, void* ws, const Layout& L,
                      hipStream_t s) {
  const RowStatsParams r = sample_sweep_params(tgt, drf, tokens, B, g, V, dt, tc, ws, L);
  if (launch_row_sweep(r, dt, s) != hipSuccess) return SPEC_EHIP;
  return draw_on(tgt, drf, dt, tokens, unif, B, g, V, tc, accept_len, out_tokens, ws, L, s);
}

// Common argument checks of the two sampling entry points.
spec_status check_sample_args(const void* target_logits, const void* draft_logits, spec_dtype dt,
                              const int32_t* draft_tokens, const float* uniforms, int B, int gamma, int V,
                              float temperature, int32_t* accept_len, int32_t* out_tokens, void* ws,
                              size_t ws_bytes, TempConst* tc, Layout* L) {
  if (!dtype_ok(dt)) return SPEC_EDTYPE;
  if (B < 1 || B > SPEC_MAX_BATCH || gamma < 1 || gamma > SPEC_MAX_GAMMA || V < 1 || V > SPEC_MAX_SAMPLE_VOCAB ||
      !row_bytes_ok(V, dt))
    return SPEC_EINVAL;
  if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !accept_len || !out_tokens)
    return SPEC_EINVAL;
  if (!aligned(target_logits, 16) || !aligned(draft_logits, 16) || !aligned(draft_tokens, 4) ||
      !aligned(uniforms, 4) || !aligned(accept_len, 4) || !aligned(out_tokens, 4))
    return SPEC_EALIGN;
  if (!temp_const(temperature, tc)) return SPEC_EINVAL;
  if (!make_layout(SPEC_MODE_SAMPLE, B, gamma, V, 0, DT_F32, L)) return SPEC_EINVAL;
  return check_ws(ws, ws_bytes, *L);
}

// ------------------------------------------------- allocation-free calls
// The workspace of spec_verify_sample_noalloc: one static device array per
// GPU, held until the process ends.  In host code `scratch` names a host-side
// stand-in, so kernels get the device address that hipGetSymbolAddress
// returns for the current device, looked up once per device.
constexpr size_t kScratchBytes = (size_t)SPEC_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array, or null on a HIP
// error (no device, symbol not found).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t spec_workspace_bytes(int mode, int B, int gamma_or_N, int V, int d) {
  if (mode == SPEC_MODE_TREE_EXPAND) {
    if (B < 1 || B > SPEC_MAX_BATCH || gamma_or_N < 1 || gamma_or_N > kFrontierMax || V < 1) return 0;
    int seg;
    const long long n = (long long)B * gamma_or_N * tree_expand_segments(V, &seg) * (long long)sizeof(TopkPart);
    return (size_t)((n + kAlign - 1) / kAlign * kAlign);
  }
  Layout L;
  if (!make_layout(mode, B, gamma_or_N, V, d, DT_F32, &L)) return 0;
  return L.total;
}

spec_status spec_workspace_init(void* ws, size_t ws_bytes, hipStream_t s) {
  if (!ws || !aligned(ws, kAlign)) return SPEC_EWORKSPACE;
  return hip_status(launch_fill_zero(ws, ws_bytes, s));
}

long long spec_stream_read_sink_words(long long bytes) {
  if (bytes < 16 || bytes % 16 != 0) return 0;
  return stream_read_workgroups(bytes);
}

spec_status spec_stream_read(const void* src, long long bytes, uint32_t* sink, long long sink_words,
                             hipStream_t s) {
  if (!src || !sink || bytes < 16 || bytes % 16 != 0 || bytes > (1LL << 40)) return SPEC_EINVAL;
  if (sink_words < stream_read_workgroups(bytes)) return SPEC_EINVAL;
  if (!aligned(src, 16) || !aligned(sink, 4)) return SPEC_EALIGN;
  return hip_status(launch_stream_read(src, bytes, sink, s));
}

const char* spec_status_str(spec_status st) {
  switch (st) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_EINVAL: return "SPEC_EINVAL: invalid size, count, pointer or scalar argument";
    case SPEC_EDTYPE: return "SPEC_EDTYPE: unknown dtype";
    case SPEC_EALIGN: return "SPEC_EALIGN: misaligned pointer";
    case SPEC_EWORKSPACE: return "SPEC_EWORKSPACE: workspace missing, misaligned or too small";
    case SPEC_EHIP: return "SPEC_EHIP: HIP runtime error";
  }
  return "unknown spec_status";
}

spec_status spec_row_stats(const void* logits, spec_dtype dt, int rows, int V, float temperature,
                           int want, float* out_max, double* out_sum, int32_t* out_argmax,
                           void* ws, size_t ws_bytes, hipStream_t s) {
  if (!dtype_ok(dt)) return SPEC_EDTYPE;
  if (rows < 1 || V < 1 || want < 1 || want > 3 || !row_bytes_ok(V, dt)) return SPEC_EINVAL;
  if (!logits || !out_max || ((want & 1) && !out_sum) || ((want & 2) && !out_argmax)) return SPEC_EINVAL;
  if (!aligned(logits, 16) || !aligned(out_max, 4) || (out_sum && !aligned(out_sum, 8)) ||
      (out_argmax && !aligned(out_argmax, 4)))
    return SPEC_EALIGN;
  TempConst tc;
  memset(&tc, 0, sizeof(tc));
  if ((want & 1) && !temp_const(temperature, &tc)) return SPEC_EINVAL;
  Layout L;
  if (!make_layout(SPEC_MODE_ROWSTATS, rows, 0, V, 0, DT_F32, &L)) return SPEC_EINVAL;
  const spec_status w = check_ws(ws, ws_bytes, L);
  if (w != SPEC_OK) return w;
  RowStatsParams p;
  memset(&p, 0, sizeof(p));
  const RowSweepShape sh = row_sweep_shape(V, (int)dt);
  p.src0 = logits;
  p.rows0 = rows;
  p.V = V;
  p.nseg = sh.nseg;
  p.seg_vecs = sh.seg_vecs;
  p.want = want;
  p.tc = tc;
  p.part = at<Partial>(ws, L.part);
  p.out_max = out_max;
  p.out_sum = out_sum;
  p.out_arg = out_argmax;
  return hip_status(launch_row_stats(p, (int)dt, s));
}

int spec_row_segments(int V, spec_dtype dt) {
  if (!dtype_ok(dt) || V < 1) return 0;
  return row_sweep_shape(V, (int)dt).nseg;
}

spec_status spec_row_partials(const void* logits, spec_dtype dt, int rows, int V, float temperature, int want,
                              void* partials, size_t partials_bytes, hipStream_t s) {
  static_assert(sizeof(Partial) == 24, "partial record layout");
  if (!dtype_ok(dt)) return SPEC_EDTYPE;
  if (rows < 1 || V < 1 || want < 1 || want > 3 || !row_bytes_ok(V, dt)) return SPEC_EINVAL;
  if (!logits || !partials) return SPEC_EINVAL;
  if (!aligned(logits, 16) || !aligned(partials, 8)) return SPEC_EALIGN;
  TempConst tc;
  memset(&tc, 0, sizeof(tc));
  if ((want & 1) && !temp_const(temperature, &tc)) return SPEC_EINVAL;
  const RowSweepShape sh = row_sweep_shape(V, (int)dt);
  if ((unsigned long long)partials_bytes / sizeof(Partial) / (unsigned long long)sh.nseg < (unsigned long long)rows)
    return SPEC_EINVAL;
  RowStatsParams p;
  memset(&p, 0, sizeof(p));
  p.src0 = logits;
  p.rows0 = rows;
  p.V = V;
  p.nseg = sh.nseg;
  p.seg_vecs = sh.seg_vecs;
  p.want = want;
  p.tc = tc;
  p.part = static_cast<Partial*>(partials);
  return hip_status(launch_row_sweep(p, (int)dt, s));
}

spec_status spec_verify_sample(const void* target_logits, const void* draft_logits, spec_dtype dt,
                               const int32_t* draft_tokens, const float* uniforms, int B, int gamma,
                               int V, float temperature, int32_t* accept_len, int32_t* out_tokens,
                               void* ws, size_t ws_bytes, hipStream_t s) {
  TempConst tc;
  Layout L;
  const spec_status st = check_sample_args(target_logits, draft_logits, dt, draft_tokens, uniforms, B, gamma, V,
                                           temperature, accept_len, out_tokens, ws, ws_bytes, &tc, &L);
  if (st != SPEC_OK) return st;
  return sample_on(target_logits, draft_logits, (int)dt, draft_tokens, uniforms, B, gamma, V, tc,
                   accept_len, out_tokens, ws, L, s);
}

spec_status spec_verify_sample_noalloc(const void* target_logits, const void* draft_logits, spec_dtype dt,
                                       const int32_t* draft_tokens, const float* uniforms, int B, int gamma, int V,
                                       float temperature, int32_t* accept_len, int32_t* out_tokens,
                                       hipStream_t s) {
  // the same checks as spec_verify_sample, with the layout checked against
  // the scratch array's size instead of a caller's workspace
  TempConst tc;
  Layout L;
  const spec_status st = check_sample_args(target_logits, draft_logits, dt, draft_tokens, uniforms, B, gamma, V,
                                           temperature, accept_len, out_tokens, reinterpret_cast<void*>(kAlign),
                                           kScratchBytes, &tc, &L);
  if (st != SPEC_OK) return st;
  void* ws = scratch_ptr();
  if (ws == nullptr) return SPEC_EHIP;
  return sample_on(target_logits, draft_logits, (int)dt, draft_tokens, uniforms, B, gamma, V, tc, accept_len,
                   out_tokens, ws, L, s);
}

spec_status spec_verify_sample_early_exit(const void* target_logits, const void* draft_logits, spec_dtype dt,
                                          const int32_t* draft_tokens, const float* uniforms, int B, int gamma,
                                          int V, float temperature, int positions_per_launch, int32_t* accept_len,
                                          int32_t* out_tokens, void* ws, size_t ws_bytes, hipStream_t s) {
  TempConst tc;
  Layout L;
  const spec_status st = check_sample_args(target_logits, draft_logits, dt, draft_tokens, uniforms, B, gamma, V,
                                           temperature, accept_len, out_tokens, ws, ws_bytes, &tc, &L);
  if (st != SPEC_OK) return st;
  if (positions_per_launch < -1 || positions_per_launch > gamma + 1) return SPEC_EINVAL;
  const int K = positions_per_launch;
  RowStatsParams r = sample_sweep_params(target_logits, draft_logits, draft_tokens, B, gamma, V, (int)dt, tc, ws, L);
  r.step_B = B;
  r.step_unif = uniforms;
  r.step_alive = at<int>(ws, L.rarg);  // [B, gamma+1]; the sampler leaves this region unused
  // blocks of K positions; for K = 0 position 0, then the rest; for K = -1
  // blocks of 1, 2, 4, ... positions
  for (int i0 = 0, prev = -1, len = K > 0 ? K : 1; i0 <= gamma; len = K > 0 ? K : (K == 0 ? gamma : 2 * len)) {
    r.step = i0;
    r.step_end = i0 + len < gamma + 1 ? i0 + len : gamma + 1;
    r.step_prev = prev;
    if (launch_row_step(r, (int)dt, s) != hipSuccess) return SPEC_EHIP;
    prev = i0;
    i0 = r.step_end;
  }
  return draw_on(target_logits, draft_logits, (int)dt, draft_tokens, uniforms, B, gamma, V, tc, accept_len,
                 out_tokens, ws, L, s);
}

spec_status spec_verify_greedy(const void* target_logits, spec_dtype dt, const int32_t* draft_tokens,
                               int B, int gamma, int V, int32_t* accept_len, int32_t* out_tokens,
                               void* ws, size_t ws_bytes, hipStream_t s) {
  if (!dtype_ok(dt)) return SPEC_EDTYPE;
  if (B < 1 || B > SPEC_MAX_BATCH || gamma < 1 || gamma > SPEC_MAX_GAMMA || V < 1 || !row_bytes_ok(V, dt))
    return SPEC_EINVAL;
  if (!target_logits || !draft_tokens || !accept_len || !out_tokens) return SPEC_EINVAL;
  if (!aligned(target_logits, 16) || !aligned(draft_tokens, 4) || !aligned(accept_len, 4) ||
      !aligned(out_tokens, 4))
    return SPEC_EALIGN;
  Layout L;
  if (!make_layout(SPEC_MODE_GREEDY, B, gamma, V, 0, DT_F32, &L)) return SPEC_EINVAL;
  const spec_status w = check_ws(ws, ws_bytes, L);
  if (w != SPEC_OK) return w;
  TempConst tc;
  memset(&tc, 0, sizeof(tc));
  hipError_t e = row_sweep(target_logits, (long long)B * (gamma + 1), nullptr, 0, V, (int)dt, 2, tc, ws, L, s,
                           false, kArgmaxVPT);
  if (e != hipSuccess) return SPEC_EHIP;
  GreedyParams p;
  p.part = at<Partial>(ws, L.part);
  p.nseg = row_sweep_shape(V, (int)dt, kArgmaxVPT).nseg;
  p.tokens = draft_tokens;
  p.B = B;
  p.g = gamma;
  p.accept_len = accept_len;
  p.out_tokens = out_tokens;
  return hip_status(launch_greedy_finish(p, s));
}

spec_status spec_verify_tree(const void* target_logits, spec_dtype dt, const int32_t* node_tokens,
                             const int32_t* parent, int parent_batch_stride, int B, int N, int V,
                             int32_t* accept_len, int32_t* out_path, int32_t* out_tokens, void* ws,
                             size_t ws_bytes, hipStream_t s) {
  if (!dtype_ok(dt)) return SPEC_EDTYPE;
  if (B < 1 || B > SPEC_MAX_BATCH || N < 1 || N > SPEC_MAX_TREE_NODES || V < 1 || !row_bytes_ok(V, dt))
    return SPEC_EINVAL;
  if (parent_batch_stride != 0 && parent_batch_stride != N) return SPEC_EINVAL;
  if (!target_logits || !node_tokens || !parent || !accept_len || !out_path || !out_tokens)
    return SPEC_EINVAL;
  if (!aligned(target_logits, 16) || !aligned(node_tokens, 4) || !aligned(parent, 4) ||
      !aligned(accept_len, 4) || !aligned(out_path, 4) || !aligned(out_tokens, 4))
    return SPEC_EALIGN;
  Layout L;
  if (!make_layout(SPEC_MODE_TREE, B, N, V, 0, DT_F32, &L)) return SPEC_EINVAL;
  const spec_status w = check_ws(ws, ws_bytes, L);
  if (w != SPEC_OK) return w;
  TempConst tc;
  memset(&tc, 0, sizeof(tc));
  hipError_t e = row_sweep(target_logits, (long long)B * N, nullptr, 0, V, (int)dt, 2, tc, ws, L, s, false,
                           kArgmaxVPT);
  if (e != hipSuccess) return SPEC_EHIP;
  TreeParams p;
  p.part = at<Partial>(ws, L.part);
  p.nseg = row_sweep_shape(V, (int)dt, kArgmaxVPT).nseg;
  p.node_tokens = node_tokens;
  p.parent = parent;
  p.parent_stride = parent_batch_stride;
  p.B = B;
  p.N = N;
  p.accept_len = accept_len;
  p.out_path = out_path;
  p.out_tokens = out_tokens;
  return hip_status(launch_tree_finish(p, s));
}

spec_status spec_verify_tree_sample(const void* target_logits, const void* draft_logits, spec_dtype dt,
                                    const int32_t* node_tokens, const int32_t* parent, int parent_batch_stride,
                                    const float* uniforms, int B, int N, int V, float temperature,
                                    spec_siblings siblings, int n_sweep, int n_rounds, int32_t* accept_len,
                                    int32_t* out_path, int32_t* out_tokens, void* ws, size_t ws_bytes,
                                    hipStream_t s) {
  if (!dtype_ok(dt)) return SPEC_EDTYPE;
  if (siblings != SPEC_SIBLINGS_IID && siblings != SPEC_SIBLINGS_DISTINCT) return SPEC_EINVAL;
  if (n_rounds < -1 || n_rounds > SPEC_MAX_TREE_ROUNDS) return SPEC_EINVAL;
  if (B < 1 || B > SPEC_MAX_BATCH || N < 1 || N > SPEC_MAX_TREE_NODES || V < 1 || V > SPEC_MAX_SAMPLE_VOCAB ||
      !row_bytes_ok(V, dt))
    return SPEC_EINVAL;
  if (parent_batch_stride != 0 && parent_batch_stride != N) return SPEC_EINVAL;
  if (n_sweep < -1 || n_sweep > N) return SPEC_EINVAL;
  if (!target_logits || !draft_logits || !node_tokens || !parent || !uniforms || !accept_len || !out_path ||
      !out_tokens)
    return SPEC_EINVAL;
  if (!aligned(target_logits, 16) || !aligned(draft_logits, 16) || !aligned(node_tokens, 4) ||
      !aligned(parent, 4) || !aligned(uniforms, 4) || !aligned(accept_len, 4) || !aligned(out_path, 4) ||
      !aligned(out_tokens, 4))
    return SPEC_EALIGN;
  TempConst tc;
  if (!temp_const(temperature, &tc)) return SPEC_EINVAL;
  Layout L;
  if (!make_layout(SPEC_MODE_TREE_SAMPLE, B, N, V, n_sweep, DT_F32, &L)) return SPEC_EINVAL;
  const spec_status w = check_ws(ws, ws_bytes, L);
  if (w != SPEC_OK) return w;
  const RowSweepShape sh = row_sweep_shape(V, (int)dt, kTreeSampleVPT);
  TreeSampleParams p;
  p.tgt = target_logits;
  p.drf = draft_logits;
  p.tokens = node_tokens;
  p.parent = parent;
  p.parent_stride = parent_batch_stride;
  p.unif = uniforms;
  p.B = B;
  p.N = N;
  p.V = V;
  p.tc = tc;
  p.distinct = siblings == SPEC_SIBLINGS_DISTINCT;
  p.nseg = sh.nseg;
  p.seg_vecs = sh.seg_vecs;
  p.n_pre = (int)tree_presweep_nodes(B, N, V, (int)dt, n_sweep);
  p.rounds = n_rounds >= 0 ? n_rounds : tree_auto_rounds(N);
  p.ws_part = at<Partial>(ws, L.part);
  p.pre_part = p.ws_part + 4LL * B * sh.nseg;
  p.ws_sub = at<double>(ws, L.segsum);
  p.state = at<TreeWalkState>(ws, L.tstate);
  p.glog = at<float>(ws, L.tglog);
  p.wpart = at<double>(ws, L.twpart);
  p.accept_len = accept_len;
  p.out_path = out_path;
  p.out_tokens = out_tokens;
  return hip_status(launch_tree_sample(p, (int)dt, s));
}

spec_status lmhead_project(const uint16_t* feat, int M, int d, const uint16_t* W, spec_wlayout wl,
                           int V, float* out_logits, hipStream_t s) {
  if (M < 1 || M > (1 << 22) || d < 64 || d % 64 != 0 || d > (1 << 20) || V < 1) return SPEC_EINVAL;
  if (V >= (1 << 25) || (wl != SPEC_W_DV && wl != SPEC_W_VD)) return SPEC_EINVAL;
  if (!feat || !W || !out_logits) return SPEC_EINVAL;
  if (!aligned(feat, 16) || !aligned(W, 16) || !aligned(out_logits, 16)) return SPEC_EALIGN;
  LmHeadParams p;
  p.A = feat;
  p.M = M;
  p.W = W;
  p.w_vd = wl == SPEC_W_VD;
  p.K = d;
  p.N = V;
  p.C = out_logits;
  p.a_staged = 0;
  p.part = nullptr;
  p.pstride = 0;
  memset(&p.tc, 0, sizeof(p.tc));
  return hip_status(launch_lmhead(p, s));
}

size_t lmhead_project_workspace_bytes(int M, int d) {
  if (M < 1 || M > (1 << 22) || d < 64 || d % 64 != 0 || d > (1 << 20)) return 0;
  return lmhead_staged_bytes(M, d);
}

spec_status lmhead_project_staged(const uint16_t* feat, int M, int d, const uint16_t* W, spec_wlayout wl, int V,
                                  float* out_logits, void* ws, size_t ws_bytes, hipStream_t s) {
  if (M < 1 || M > (1 << 22) || d < 64 || d % 64 != 0 || d > (1 << 20) || V < 1) return SPEC_EINVAL;
  if (V >= (1 << 25) || (wl != SPEC_W_DV && wl != SPEC_W_VD)) return SPEC_EINVAL;
  if (!feat || !W || !out_logits) return SPEC_EINVAL;
  if (!aligned(feat, 16) || !aligned(W, 16) || !aligned(out_logits, 16)) return SPEC_EALIGN;
  if (!ws || !aligned(ws, kAlign) || ws_bytes < lmhead_staged_bytes(M, d)) return SPEC_EWORKSPACE;
  LmHeadStageParams sp;
  sp.src0 = feat;
  sp.rows0 = M;
  sp.src1 = feat;
  sp.M = M;
  sp.K = d;
  sp.dst = static_cast<uint16_t*>(ws);
  if (launch_lmhead_stage(sp, s) != hipSuccess) return SPEC_EHIP;
  LmHeadParams p;
  p.A = sp.dst;
  p.M = M;
  p.W = W;
  p.w_vd = wl == SPEC_W_VD;
  p.K = d;
  p.N = V;
  p.C = out_logits;
  p.a_staged = 1;
  p.part = nullptr;
  p.pstride = 0;
  memset(&p.tc, 0, sizeof(p.tc));
  return hip_status(launch_lmhead(p, s));
}

}  // extern "C"

namespace {

// lmhead_verify for either weight layout: stage the feature rows, one GEMM
// into the workspace's float32 logits whose epilogue also leaves per-row
// partials of the row statistics, a merge of those partials (with the gather
// of the drafted tokens' logits), then the accept scan and the draw on them:
// the logits are read again only for the rows the draw needs.
spec_status lmhead_verify_layout(const uint16_t* target_feat, const uint16_t* draft_feat, const uint16_t* W,
                                 int w_vd, const int32_t* draft_tokens, const float* uniforms, int B, int gamma,
                                 int d, int V, float temperature, int32_t* accept_len, int32_t* out_tokens,
                                 void* ws, size_t ws_bytes, hipStream_t s) {
  if (B < 1 || B > SPEC_MAX_BATCH || gamma < 1 || gamma > SPEC_MAX_GAMMA || V < 1 || V > SPEC_MAX_SAMPLE_VOCAB)
    return SPEC_EINVAL;
  if (d < 64 || d % 64 != 0 || d > (1 << 20)) return SPEC_EINVAL;
  if (V >= (1 << 25)) return SPEC_EINVAL;
  if (!target_feat || !draft_feat || !W || !draft_tokens || !uniforms || !accept_len || !out_tokens)
    return SPEC_EINVAL;
  if (!aligned(target_feat, 16) || !aligned(draft_feat, 16) || !aligned(W, 16) ||
      !aligned(draft_tokens, 4) || !aligned(uniforms, 4) || !aligned(accept_len, 4) ||
      !aligned(out_tokens, 4))
    return SPEC_EALIGN;
  TempConst tc;
  if (!temp_const(temperature, &tc)) return SPEC_EINVAL;
  Layout L;
  if (!make_layout(SPEC_MODE_LMHEAD, B, gamma, V, d, DT_F32, &L)) return SPEC_EINVAL;
  const spec_status w = check_ws(ws, ws_bytes, L);
  if (w != SPEC_OK) return w;
  float* Z = at<float>(ws, L.logits);
  // the GEMM reads all B(2 gamma + 1) feature rows, target rows first, from
  // one staged block (so W streams once for both)
  LmHeadStageParams sp;
  sp.src0 = target_feat;
  sp.rows0 = B * (gamma + 1);
  sp.src1 = draft_feat;
  sp.M = B * (2 * gamma + 1);
  sp.K = d;
  sp.dst = at<uint16_t>(ws, L.hcat);
  if (launch_lmhead_stage(sp, s) != hipSuccess) return SPEC_EHIP;
  LmHeadParams p;
  p.A = sp.dst;
  p.a_staged = 1;
  p.M = B * (2 * gamma + 1);
  p.W = W;
  p.w_vd = w_vd;
  p.K = d;
  p.N = V;
  p.C = Z;
  p.part = at<LmPartial>(ws, L.gpart);
  p.pstride = lmhead_stat_parts(V);
  p.tc = tc;
  if (launch_lmhead(p, s) != hipSuccess) return SPEC_EHIP;
  LmHeadMergeParams mp;
  mp.part = p.part;
  mp.nparts = p.pstride;
  mp.C = Z;
  mp.M = p.M;
  mp.N = V;
  mp.tokens = draft_tokens;
  mp.B = B;
  mp.g = gamma;
  mp.tc = tc;
  mp.out = at<Partial>(ws, L.part);
  mp.gathered = at<float>(ws, L.gath);
  if (launch_lmhead_merge(mp, s) != hipSuccess) return SPEC_EHIP;
  const float* Zd = Z + (size_t)B * (gamma + 1) * (size_t)V;
  return draw_on(Z, Zd, DT_F32, draft_tokens, uniforms, B, gamma, V, tc, accept_len, out_tokens, ws, L, s,
                 1);
}

}  // namespace

extern "C" {

spec_status lmhead_verify(const uint16_t* target_feat, const uint16_t* draft_feat, const uint16_t* W,
                          const int32_t* draft_tokens, const float* uniforms, int B, int gamma, int d, int V,
                          float temperature, int32_t* accept_len, int32_t* out_tokens, void* ws,
                          size_t ws_bytes, hipStream_t s) {
  return lmhead_verify_layout(target_feat, draft_feat, W, 0, draft_tokens, uniforms, B, gamma, d, V,
                              temperature, accept_len, out_tokens, ws, ws_bytes, s);
}

spec_status lmhead_verify_wvd(const uint16_t* target_feat, const uint16_t* draft_feat, const uint16_t* W_vd,
                              const int32_t* draft_tokens, const float* uniforms, int B, int gamma, int d, int V,
                              float temperature, int32_t* accept_len, int32_t* out_tokens, void* ws,
                              size_t ws_bytes, hipStream_t s) {
  return lmhead_verify_layout(target_feat, draft_feat, W_vd, 1, draft_tokens, uniforms, B, gamma, d, V,
                              temperature, accept_len, out_tokens, ws, ws_bytes, s);
}

spec_status spec_probe_probs(const void* target_logits, const void* draft_logits, spec_dtype dt, int rows,
                             int V, float temperature, double* out_p, double* out_q, double* out_resid,
                             void* ws, size_t ws_bytes, hipStream_t s) {
  if (!dtype_ok(dt)) return SPEC_EDTYPE;
  if (rows < 1 || rows > SPEC_MAX_BATCH / 2 || V < 1 || !row_bytes_ok(V, dt)) return SPEC_EINVAL;
  if (!target_logits || !out_p || (!draft_logits && (out_q || out_resid))) return SPEC_EINVAL;
  if (!aligned(target_logits, 16) || (draft_logits && !aligned(draft_logits, 16)) || !aligned(out_p, 8) ||
      (out_q && !aligned(out_q, 8)) || (out_resid && !aligned(out_resid, 8)))
    return SPEC_EALIGN;
  TempConst tc;
  if (!temp_const(temperature, &tc)) return SPEC_EINVAL;
  Layout L;
  if (!make_layout(SPEC_MODE_ROWSTATS, 2LL * rows, 0, V, 0, DT_F32, &L)) return SPEC_EINVAL;
  const spec_status w = check_ws(ws, ws_bytes, L);
  if (w != SPEC_OK) return w;
  hipError_t e = row_sweep(target_logits, rows, draft_logits, draft_logits ? rows : 0, V, (int)dt, 1, tc, ws,
                           L, s, true);
  if (e != hipSuccess) return SPEC_EHIP;
  ProbeParams p;
  p.tgt = target_logits;
  p.drf = draft_logits;
  p.row_max = at<float>(ws, L.rmax);
  p.row_sum = at<double>(ws, L.rsum);
  p.rows = rows;
  p.V = V;
  p.tc = tc;
  p.out_p = out_p;
  p.out_q = out_q;
  p.out_resid = out_resid;
  return hip_status(launch_probe(p, (int)dt, s));
}

spec_status spec_kv_compact(void* kv, int B, int planes, int S, long long entry_bytes, long long seq_stride,
                            long long plane_stride, const int32_t* prefix_len, const int32_t* path,
                            int path_stride, const int32_t* accept_len, int32_t* new_len, hipStream_t s) {
  if (B < 1 || B > SPEC_MAX_BATCH || planes < 1 || S < 1 || entry_bytes < 16 || entry_bytes > (1LL << 30))
    return SPEC_EINVAL;
  if (seq_stride < 0 || plane_stride < 0 || (path && path_stride < 1)) return SPEC_EINVAL;
  if (!kv || !prefix_len || !accept_len || !new_len) return SPEC_EINVAL;
  // distinct (sequence, plane) blocks of S entries must not overlap: either
  // planes nest inside sequences or sequences inside planes
  const long long blk = (long long)S * entry_bytes;
  if (blk > (1LL << 46)) return SPEC_EINVAL;
  const bool seq_outer = (planes == 1 || plane_stride >= blk) &&
                         (B == 1 || seq_stride >= (long long)(planes - 1) * plane_stride + blk);
  const bool plane_outer = (B == 1 || seq_stride >= blk) &&
                           (planes == 1 || plane_stride >= (long long)(B - 1) * seq_stride + blk);
  if (!seq_outer && !plane_outer) return SPEC_EINVAL;
  if (entry_bytes % 16 || seq_stride % 16 || plane_stride % 16 || !aligned(kv, 16) || !aligned(prefix_len, 4) ||
      (path && !aligned(path, 4)) || !aligned(accept_len, 4) || !aligned(new_len, 4))
    return SPEC_EALIGN;
  KvParams p;
  p.kv = static_cast<char*>(kv);
  p.B = B;
  p.planes = planes;
  p.S = S;
  p.entry_bytes = entry_bytes;
  p.seq_stride = seq_stride;
  p.plane_stride = plane_stride;
  p.prefix_len = prefix_len;
  p.path = path;
  p.path_stride = path ? path_stride : 0;
  p.accept_len = accept_len;
  p.new_len = new_len;
  return hip_status(launch_kv_compact(p, s));
}

spec_status spec_tree_expand(const void* draft_logits, spec_dtype dt, const int32_t* frontier, int B, int K_in,
                             int V, float temperature, int k, int K_out, int32_t* node_parent,
                             int32_t* node_token, double* node_score, int32_t* node_depth, int cap, int off,
                             int32_t* next_frontier, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!dtype_ok(dt)) return SPEC_EDTYPE;
  if (B < 1 || B > SPEC_MAX_BATCH || K_in < 1 || K_in > kFrontierMax || K_out < 1 || K_out > kFrontierMax ||
      k < 1 || k > kTopkMax || K_in * k > kCandMax || V < k || !row_bytes_ok(V, dt))
    return SPEC_EINVAL;
  if (off < 1 || cap < 1 || (long long)off + (long long)K_in * k > cap) return SPEC_EINVAL;
  if (!draft_logits || !frontier || !node_parent || !node_token || !node_score || !node_depth || !next_frontier)
    return SPEC_EINVAL;
  TempConst tc;
  if (!temp_const(temperature, &tc)) return SPEC_EINVAL;
  if (!aligned(draft_logits, 16) || !aligned(frontier, 4) || !aligned(node_parent, 4) || !aligned(node_token, 4) ||
      !aligned(node_score, 8) || !aligned(node_depth, 4) || !aligned(next_frontier, 4))
    return SPEC_EALIGN;
  const size_t need = spec_workspace_bytes(SPEC_MODE_TREE_EXPAND, B, K_in, V, 0);
  if (!ws || !aligned(ws, kAlign) || ws_bytes < need) return SPEC_EWORKSPACE;
  TreeExpandParams p;
  p.logits = draft_logits;
  p.dt = dt == SPEC_BF16 ? DT_BF16 : DT_F32;
  p.frontier = frontier;
  p.B = B;
  p.K_in = K_in;
  p.V = V;
  p.tc = tc;
  p.k = k;
  p.K_out = K_out;
  p.parent = node_parent;
  p.token = node_token;
  p.score = node_score;
  p.depth = node_depth;
  p.cap = cap;
  p.off = off;
  p.next_frontier = next_frontier;
  p.part = static_cast<TopkPart*>(ws);
  p.nseg = tree_expand_segments(V, &p.seg_elems);
  return hip_status(launch_tree_expand(p, s));
}

spec_status spec_tree_build(const int32_t* node_parent, const int32_t* node_token, const double* node_score,
                            const int32_t* node_depth, int B, int cap, int n_nodes, int M, int32_t* out_n,
                            int32_t* out_parent, int32_t* out_token, int32_t* out_depth, int32_t* out_index,
                            uint32_t* out_mask, hipStream_t s) {
  if (B < 1 || B > SPEC_MAX_BATCH || n_nodes < 1 || n_nodes > cap || n_nodes > kBuildMaxNodes || M < 0 ||
      M + 1 > kBuildMaxNodes)
    return SPEC_EINVAL;
  if (!node_parent || !node_token || !node_score || !node_depth || !out_n || !out_parent || !out_token ||
      !out_depth || !out_index || !out_mask)
    return SPEC_EINVAL;
  if (!aligned(node_parent, 4) || !aligned(node_token, 4) || !aligned(node_score, 8) || !aligned(node_depth, 4) ||
      !aligned(out_n, 4) || !aligned(out_parent, 4) || !aligned(out_token, 4) || !aligned(out_depth, 4) ||
      !aligned(out_index, 4) || !aligned(out_mask, 4))
    return SPEC_EALIGN;
  TreeBuildParams p;
  p.parent = node_parent;
  p.token = node_token;
  p.score = node_score;
  p.depth = node_depth;
  p.B = B;
  p.cap = cap;
  p.n_nodes = n_nodes;
  p.M = M;
  p.out_n = out_n;
  p.out_parent = out_parent;
  p.out_token = out_token;
  p.out_depth = out_depth;
  p.out_index = out_index;
  p.out_mask = out_mask;
  p.W = (M + 1 + 31) / 32;
  return hip_status(launch_tree_build(p, s));
}

}  // extern "C"
