// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_common.hpp"

namespace sv {

// ------------------------------------------------------------ row sweep
// One pass over every row of up to two logit tensors (rows0 rows of the
// first, rows1 of the second, both [*, V]).  Each wave reduces one segment of
// one row into a partial; a second kernel merges each row's partials.
struct RowStatsParams {
  const void* src0;
  const void* src1;
  long long rows0;
  long long rows1;
  int V;
  int nseg;       // workgroup segments per row
  int seg_vecs;   // full 16-byte vectors per segment
  int want;       // bit 0: max/sum, bit 1: argmax
  int vpt;        // vectors per lane of the segments (0: the default; kArgmaxVPT for want == 2)
  TempConst tc;
  Partial* part;  // [rows][nseg]
  // optional gather: for target row (b, i) with i < gather_g and draft row
  // (b, i), store z[row][tokens[b][i]] into gather_out[row] (rows of the
  // second tensor continue after rows0)
  const int* gather_tokens;
  int gather_g;
  float* gather_out;
  float* out_max; // [rows]
  double* out_sum;// [rows] (want & 1)
  int* out_arg;   // [rows] (want & 2)
  // early-exit block (launch_row_step): positions step .. step_end-1 of B
  // sequences, their target and draft rows, swept only while every earlier
  // position was accepted; alive[b][step] records that.  step_prev is the
  // previous block's first position (-1 for the first block): the block's
  // workgroups test positions step_prev .. step-1 from the previous block's
  // partials
  int step;
  int step_end;
  int step_prev;
  int step_B;
  const float* step_unif;  // [B, gamma+1]
  int* step_alive;         // [B, gamma+1]
};

struct RowSweepShape {
  int nseg;
  int seg_vecs;
};
// Segments of vpt * kBlock vectors (vpt = 0: the default of every path that
// sums; the argmax-only sweeps of greedy verification use kArgmaxVPT: more,
// smaller segments, which fill the chip better for those shorter passes).
constexpr int kArgmaxVPT = 6;
// The tree sampler's row statistics (presweep and the walk's entry passes)
// keep 8-vector segments: then a node's two rows take at most as many
// workgroups (2 nseg) as a W pass (V / 8192), so the rounds' grids stay at
// one W pass's width.
constexpr int kTreeSampleVPT = 8;
RowSweepShape row_sweep_shape(int V, int dt, int vpt = 0);
// Sweep then merge (final per-row statistics in out_*).
hipError_t launch_row_stats(const RowStatsParams& p, int dt, hipStream_t s);
// The sweep alone (partials only); its consumers merge partials inline.
hipError_t launch_row_sweep(const RowStatsParams& p, int dt, hipStream_t s);
hipError_t launch_row_step(const RowStatsParams& p, int dt, hipStream_t s);
hipError_t launch_row_merge(const RowStatsParams& p, hipStream_t s);

// ---------------------------------------------------------- sampling
// Two kernels after the row sweep: the accept scan plus the residual / bonus
// segment masses (B x nseg workgroups; each merges its sequence's row
// partials) and the inverse-CDF draw (one workgroup per sequence).
struct SampleParams {
  const void* tgt;        // [B, g+1, V]
  const void* drf;        // [B, g, V]
  const int* tokens;      // [B, g]
  const float* unif;      // [B, g+1]
  const Partial* part;    // [rows][nseg_rows] row-sweep partials
  int nseg_rows;
  const float* gathered;  // [rows] z[row][x] picked out by the sweep
  int B, g, V;
  int nseg;               // draw segments per row (one mass workgroup each)
  int seg_elems;          // elements per draw segment (kDrawSub sub-segments)
  TempConst tc;
  DrawInfo* info;         // [B]
  double* segsum;         // [B][nseg * kDrawSub] sub-segment masses
  int* accept_len;        // [B]
  int* out_tokens;        // [B, g+1]
};
// Each draw segment is summed as kDrawSub contiguous sub-segments, one per
// wave; the pick rescans one sub-segment.
constexpr int kDrawSub = 4;
// Draw segments per row for element type dt (DT_BF16 / DT_F32): 8192 bf16 or
// 4096 fp32 logits each.
int sample_draw_segments(int V, int dt, int* seg_elems);
hipError_t launch_sample(const SampleParams& p, int dt, hipStream_t s);

// ---------------------------------------------------------- greedy / tree
struct GreedyParams {
  const Partial* part;    // [B(g+1)][nseg] row-sweep partials (argmax)
  int nseg;
  const int* tokens;      // [B, g]
  int B, g;
  int* accept_len;
  int* out_tokens;        // [B, g+1]
};
hipError_t launch_greedy_finish(const GreedyParams& p, hipStream_t s);

struct TreeParams {
  const Partial* part;    // [B N][nseg] row-sweep partials (argmax)
  int nseg;
  const int* node_tokens; // [B, N]
  const int* parent;      // [N] or [B, N]
  int parent_stride;      // 0 or N
  int B, N;
  int* accept_len;
  int* out_path;          // [B, N]
  int* out_tokens;        // [B, N]
};
hipError_t launch_tree_finish(const TreeParams& p, hipStream_t s);

// ---------------------------------------------------------- probe
struct ProbeParams {
  const void* tgt;        // [rows, V]
  const void* drf;        // [rows, V] or null
  const float* row_max;   // [rows] target, then [rows] draft
  const double* row_sum;
  int rows, V;
  TempConst tc;
  double* out_p;
  double* out_q;
  double* out_resid;
};
hipError_t launch_probe(const ProbeParams& p, int dt, hipStream_t s);

// ---------------------------------------------------------- utilities
hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t s);
// Bandwidth probe: read [src, src + bytes) (bytes a multiple of 16) with the
// row sweep's load pattern, one XOR word per workgroup into sink.
long long stream_read_workgroups(long long bytes);
hipError_t launch_stream_read(const void* src, long long bytes, uint32_t* sink, hipStream_t s);

// ---------------------------------------------------------- LM head
// A row partial of the LM head's epilogue: m the max of its columns, K =
// fl(m c_hi), s the sum of 2^(z c - K) over them (m = -inf: no columns).
struct LmPartial {
  float m;
  float K;
  double s;
};

struct LmHeadParams {
  const uint16_t* A;      // [M, K] bf16 rows, 16-byte aligned (a_staged = 0), or the staged layout
  int M;
  const uint16_t* W;      // [K, N] bf16, N innermost (w_vd = 0) or [N, K], K innermost (w_vd = 1)
  int w_vd;
  int K, N;
  float* C;               // [M, N] fp32
  int a_staged;
  // optional row statistics of the logits as they leave the accumulators:
  // part[row][c] is the partial (max, K offset, sum of 2^(z c - K)) of
  // columns 128 c .. 128 c + 127 of the row, the row sweep's segment
  // statistics without the argmax; null: logits only
  LmPartial* part;
  int pstride;            // partials per row, lmhead_stat_parts(N)
  TempConst tc;
};
hipError_t launch_lmhead(const LmHeadParams& p, hipStream_t s);
// Partials per row of the GEMM's row statistics (one per 128 columns).
inline int lmhead_stat_parts(long long N) { return (int)(2 * ((N + 255) / 256)); }

// Merge of the GEMM's per-row partials into one partial per row (the form
// the sampling kernels merge, with nseg_rows = 1), plus the gather of the
// drafted token's logit for the accept test: row r < B(g+1) is target row
// (b, i) = (r / (g+1), r % (g+1)) (token tokens[b][i] when i < g), the rows
// after it draft rows (b, i) in order (token tokens[b][i]).
struct LmHeadMergeParams {
  const LmPartial* part;  // [M][nparts]
  int nparts;
  const float* C;         // [M, N] logits
  int M;
  long long N;
  const int* tokens;      // [B, g]
  int B, g;
  TempConst tc;
  Partial* out;           // [M]
  float* gathered;        // [M]
};
hipError_t launch_lmhead_merge(const LmHeadMergeParams& p, hipStream_t s);

// Staged feature rows: for every 256-row M tile mt and K step ks (32
// features) one contiguous 16 KB block, 256 rows x 64 bytes, at element
// offset (mt * K / 32 + ks) * 8192; rows past M are zero.  The GEMM then
// reads whole cache lines for its A operand.  Rows m < rows0 come from src0,
// the others from src1 (row m - rows0).
struct LmHeadStageParams {
  const uint16_t* src0;
  int rows0;
  const uint16_t* src1;
  int M, K;
  uint16_t* dst;
};
size_t lmhead_staged_bytes(long long M, long long K);
hipError_t launch_lmhead_stage(const LmHeadStageParams& p, hipStream_t s);

// ---------------------------------------------------------- KV compaction
struct KvParams {
  char* kv;                  // entry (b, p, s): entry_bytes at kv + b*seq_stride + p*plane_stride + s*entry_bytes
  int B, planes, S;
  long long entry_bytes, seq_stride, plane_stride;
  const int32_t* prefix_len; // [B]
  const int32_t* path;       // [B, path_stride] or null (linear drafts: nothing moves)
  int path_stride;
  const int32_t* accept_len; // [B]
  int32_t* new_len;          // [B] out
};
hipError_t launch_kv_compact(const KvParams& p, hipStream_t s);

// ---------------------------------------------------------- draft tree
constexpr int kTopkMax = 16;        // children per expanded node
constexpr int kFrontierMax = 64;    // frontier slots per depth
constexpr int kCandMax = 1024;      // children per sequence and depth
constexpr int kBuildMaxNodes = 2048;

// One (frontier row, segment) of the expansion sweep.
struct TopkPart {
  float m;                 // segment max
  float s;                 // sum of 2^((z - m) c) over the segment
  float v[kTopkMax];       // the segment's largest logits, best first
  int idx[kTopkMax];       // their token indices (INT_MAX: none)
};

struct TreeExpandParams {
  const void* logits;      // [B, K_in, V]
  int dt;
  const int32_t* frontier; // [B, K_in] table index or -1
  int B, K_in, V;
  TempConst tc;
  int k, K_out;
  int32_t* parent;         // node table [B, cap]
  int32_t* token;
  double* score;
  int32_t* depth;
  int cap, off;
  int32_t* next_frontier;  // [B, K_out]
  TopkPart* part;          // [B * K_in, nseg]
  int nseg, seg_elems;
};
int tree_expand_segments(int V, int* seg_elems);
hipError_t launch_tree_expand(const TreeExpandParams& p, hipStream_t s);

struct TreeBuildParams {
  const int32_t* parent;   // node table [B, cap]
  const int32_t* token;
  const double* score;
  const int32_t* depth;
  int B, cap, n_nodes, M;
  int32_t* out_n;          // [B]
  int32_t* out_parent;     // [B, M + 1]
  int32_t* out_token;
  int32_t* out_depth;
  int32_t* out_index;
  uint32_t* out_mask;      // [B, M + 1, W]
  int W;
};
hipError_t launch_tree_build(const TreeBuildParams& p, hipStream_t s);

// ---------------------------------------------------------- tree sampling
constexpr int kTreeMaxNodes = 4096;           // nodes per tree (verification calls)
constexpr int kTreeMaxRounds = 64;            // chip-wide pass rounds of one tree-sampling call
constexpr long long kMaxSampleVocab = 1LL << 25;

// The walk keeps each sequence's state in the workspace between its kernels.
// Passes over a node's rows after the row sweep (W passes, the final draw)
// work in segments of kTreeSeg elements, one 256-thread workgroup each, one
// 2048-element sub-segment per wave.
constexpr int kTreeSeg = 8192;
__host__ __device__ inline long long tree_segments(long long V) { return (V + kTreeSeg - 1) / kTreeSeg; }

struct TreeWalkState {
  int n, d, i, phase;      // current node, accepted depth, next child to test (index order), pending work
  int nk, mready;          // children of n (set with a pending row sweep); draw masses in place
  float Mt, Md;            // row statistics of n
  double St, Sd;
  double cc, W, Rk;        // the residual chain at n: p_i = max(0, p - cc q) / W, and R_i
  double cn, cfb;          // c of the pending W pass or draw, and of the law before it
  double pad2_;
};
static_assert(sizeof(TreeWalkState) == 96, "state layout");

struct TreeSampleParams {
  const void* tgt;         // [B, N, V] target rows of the nodes
  const void* drf;         // [B, N, V] draft rows (row n: the law n's children were drawn from)
  const int32_t* tokens;   // [B, N]
  const int32_t* parent;   // [N] or [B, N]
  int parent_stride;       // 0 or N
  const float* unif;       // [B, N]: u[b][n] tests node n, u[b][0] is the final draw
  int B, N, V;
  TempConst tc;
  int distinct;            // 1: siblings drawn without replacement (q_k excludes earlier siblings)
  int nseg;                // row sweep segments per row (row_sweep_shape)
  int seg_vecs;
  int n_pre;               // nodes 0 .. n_pre-1 have their rows swept before the walk
  int rounds;              // chip-wide rounds before the walks finish on their own CUs
  Partial* pre_part;       // [2 B n_pre][nseg]: target rows (b, n), then draft rows (b, n)
  Partial* ws_part;        // [2][B][2 nseg]: partials of a node swept during the walk (two buffers)
  TreeWalkState* state;    // [2][B] (two buffers)
  float* glog;             // [B][N][2]: node c's token logit in its parent's target and draft rows
  double* wpart;           // [2][B][tree_segments(V)][3]: W-pass segment sums (two buffers)
  double* ws_sub;          // [B][tree_segments(V) * kDrawSub] sub-segment masses of the final draw
  int32_t* accept_len;     // [B]
  int32_t* out_path;       // [B, N]
  int32_t* out_tokens;     // [B, N]
};
hipError_t launch_tree_sample(const TreeSampleParams& p, int dt, hipStream_t s);

}  // namespace sv
