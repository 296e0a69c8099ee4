/*
 * libspecverify -- batched draft verification for speculative decoding on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (sources: the web pages "EAGLE-3 speculative decoding review"
 * (6unoyunr.github.io), "EAGLE math" (aicassindra.com, transformer_math) and
 * "Speculative decoding" (addictedtoai.net wiki)):
 *
 *   A draft proposes gamma tokens x_0..x_{gamma-1}.  The target scores the
 *   prefix plus the drafts in one pass, giving gamma+1 rows of logits: row i
 *   is the target's distribution for drafted position i, and row gamma is the
 *   "bonus" row after the last draft.  Verification walks the drafts left to
 *   right, accepts x_i with probability min(1, p_i(x_i)/q_i(x_i)), stops at
 *   the first rejection j and resamples that position from
 *   norm(max(0, p_j - q_j)); if every draft is accepted it takes one more
 *   token from p_gamma.  Greedy decoding accepts a draft iff it equals the
 *   target's argmax.  Greedy tree verification accepts the longest
 *   root-to-node path whose tokens equal the target's argmax at their parent.
 *   EAGLE drafts features and reuses the target's LM head z = W h.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers: every array argument is DEVICE memory owned by the caller,
 *    row-major and contiguous with the vocabulary innermost.  Base pointers
 *    of logits, features and weights must be 16-byte aligned (SPEC_EALIGN).
 *    Integer and float side arrays must be 4-byte aligned.
 *  - Logits are float32 (SPEC_F32) or bf16 bit patterns (SPEC_BF16).  Each
 *    logit is finite or -inf, every row holds at least one finite logit and
 *    |logit| / temperature < 1e37; NaN inputs give undefined results.
 *  - Temperature: p = softmax(z_target / T), q = softmax(z_draft / T) with the
 *    same T > 0 (finite).  Greedy modes have their own calls.
 *  - Uniforms: u[b][i] for i < gamma is the accept test of drafted position
 *    i (accept iff u < p/q); u[b][gamma] is the single final draw.  Values
 *    must lie in [0, 1).
 *  - Final draw: inverse CDF over ascending token index: the first token
 *    whose cumulative mass exceeds u * total; zero-mass tokens are never
 *    drawn.
 *  - Argmax ties resolve to the lowest token index.
 *  - Calls are asynchronous on stream `s` (NULL = the default stream) and
 *    allocate nothing.  Outputs are valid once the stream has synchronised.
 *  - Workspace: `ws` is caller-owned device memory of at least
 *    spec_workspace_bytes(...) bytes, 256-byte aligned, holding per-row
 *    partial statistics between the kernels of one call.  It needs no
 *    initialisation: no output depends on a byte the call did not write
 *    (the early-exit call may read, and then discard, a skipped sequence's
 *    stale partials).  Calls that overlap in time must use distinct
 *    workspaces.
 *  - Errors: argument errors are reported synchronously, before anything is
 *    launched, as a non-zero spec_status.  A failed launch reports
 *    SPEC_EHIP.  Data-dependent conditions that can only be seen on the
 *    device (an out-of-range draft token, an invalid tree) are reported per
 *    sequence as accept_len[b] = -1 with every output token of b set to -1.
 *  - No C++ exception crosses this interface.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPEC_OK = 0,
  SPEC_EINVAL = 1,     /* a size, count, pointer or scalar argument is invalid */
  SPEC_EDTYPE = 2,     /* unknown dtype code */
  SPEC_EALIGN = 3,     /* a base pointer is not aligned as required */
  SPEC_EWORKSPACE = 4, /* workspace missing or smaller than required */
  SPEC_EHIP = 5        /* the HIP runtime reported an error */
} spec_status;

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

/* Layout of the LM-head weight W. */
typedef enum {
  SPEC_W_DV = 0,  /* W[d][V]: vocabulary innermost                             */
  SPEC_W_VD = 1   /* W[V][d]: feature dimension innermost, the layout in which
                     a linear layer's weight is usually stored (faster path)  */
} spec_wlayout;

/* How the children of one draft-tree node were drawn (sampling trees). */
typedef enum {
  SPEC_SIBLINGS_IID = 0,      /* independently from the node's draft law q  */
  SPEC_SIBLINGS_DISTINCT = 1  /* one after another from q without
                                 replacement (k distinct candidates, e.g. by
                                 the Gumbel-top-k trick)                   */
} spec_siblings;

typedef enum {
  SPEC_MODE_SAMPLE = 0,   /* spec_verify_sample: gamma_or_N = gamma        */
  SPEC_MODE_GREEDY = 1,   /* spec_verify_greedy: gamma_or_N = gamma        */
  SPEC_MODE_TREE = 2,     /* spec_verify_tree:   gamma_or_N = N (nodes)    */
  SPEC_MODE_LMHEAD = 3,   /* lmhead_verify:      gamma_or_N = gamma, d     */
  SPEC_MODE_ROWSTATS = 4, /* spec_row_stats / spec_probe_probs: B = rows   */
  SPEC_MODE_TREE_EXPAND = 5, /* spec_tree_expand:  gamma_or_N = K_in       */
  SPEC_MODE_TREE_SAMPLE = 6  /* spec_verify_tree_sample: gamma_or_N = N,
                                d = n_sweep                               */
} spec_mode;

/* Limits checked by every entry point. */
#define SPEC_MAX_GAMMA 63       /* one 64-wide wavefront lane per position   */
#define SPEC_MAX_TREE_NODES 4096
#define SPEC_MAX_TREE_ROUNDS 64   /* n_rounds limit of spec_verify_tree_sample */
#define SPEC_MAX_BATCH (1 << 20)
#define SPEC_MAX_SAMPLE_VOCAB (1 << 25)   /* V limit of the sampling calls */
#define SPEC_MAX_TOPK 16          /* children per expanded draft-tree node    */
#define SPEC_MAX_FRONTIER 64      /* frontier slots per expansion depth       */
#define SPEC_MAX_BUILD_NODES 2048 /* node-table entries and tree size (build) */

/* Bytes of workspace the call of the given mode needs for these sizes
 * (0 when an argument is out of range).  d is the feature width for
 * SPEC_MODE_LMHEAD and the call's n_sweep for SPEC_MODE_TREE_SAMPLE; other
 * modes ignore it.  The LMHEAD workspace holds the float32 logits of all
 * B(2*gamma+1) rows and 16 bytes of row statistics per 128 logits. */
size_t spec_workspace_bytes(int mode, int B, int gamma_or_N, int V, int d);

/* Zero-fill a workspace (a device fill kernel; graph-capture safe).  Not
 * required before use; offered for callers that poison-check buffers. */
spec_status spec_workspace_init(void* ws, size_t ws_bytes, hipStream_t s);

/* Human-readable name of a status code (static storage). */
const char* spec_status_str(spec_status st);

/*
 * spec_stream_read -- bandwidth probe (not a verification step): reads
 * [src, src + bytes) once with the row sweep's load pattern (32 KB per
 * workgroup, eight non-temporal 16-byte loads per lane in flight) and no
 * arithmetic, so its rate is the HBM read rate the verification kernels can
 * reach on this device.  sink [>= spec_stream_read_sink_words(bytes)] uint32
 * receives one XOR word per workgroup (meaningless; it keeps the loads live).
 * bytes a positive multiple of 16 (<= 2^40); src 16-byte aligned, sink
 * 4-byte aligned.
 */
long long spec_stream_read_sink_words(long long bytes);
spec_status spec_stream_read(const void* src, long long bytes, uint32_t* sink,
                             long long sink_words, hipStream_t s);

/*
 * spec_row_stats -- one pass over each logit row.
 * Pages: "EAGLE-3 speculative decoding review", "EAGLE: Predict Features, Not
 * Tokens" (logits z -> softmax -> next-token distribution) and "Does Using a
 * Small Model's Answer Reduce Quality?" (greedy takes the argmax).
 *
 * logits      [rows, V] in `dt`.
 * want        bit 0: max and sum statistics; bit 1: argmax.  At least one.
 * out_max     [rows] float32: max_v z[r][v]                  (want & 1 or 2)
 * out_sum     [rows] float64: sum_v exp((z[r][v]-max)/T)     (want & 1; may be
 *             NULL otherwise).  p[r][v] = exp((z[r][v]-max)/T) / out_sum[r].
 * out_argmax  [rows] int32: lowest index of the maximum       (want & 2; may be
 *             NULL otherwise).
 * temperature used only for the sum (ignored when !(want & 1)).
 * Workspace: spec_workspace_bytes(SPEC_MODE_ROWSTATS, rows, 0, V, 0).
 */
spec_status spec_row_stats(const void* logits, spec_dtype dt, int rows, int V,
                           float temperature, int want, float* out_max,
                           double* out_sum, int32_t* out_argmax, void* ws,
                           size_t ws_bytes, hipStream_t s);

/*
 * spec_row_partials -- the pass of spec_row_stats without its merge, for
 * callers that combine partial statistics themselves (for example the
 * vocabulary shards of one row held by several GPUs: shard records merge like
 * the segments of one row).  Pages: as spec_row_stats.
 *
 * Each row is cut into spec_row_segments(V, dt) segments; one 24-byte record
 * per (row, segment), row-major: float m (segment max); int32 arg (lowest
 * row-local index holding m, INT32_MAX without want & 2); float K; 4 unused
 * bytes; double s = sum over the segment of 2^(z c - K), c = log2(e)/T (K and
 * s are 0 without want & 1).  The row's statistics are M = max m,
 * out_sum = sum s * 2^(K - M c) (in double), argmax = min arg over the
 * segments whose m equals M.
 * partials   [rows][nseg] records, 8-byte aligned; partials_bytes must be at
 *            least rows * nseg * 24.  No workspace.
 * want, temperature: as in spec_row_stats.
 */
int spec_row_segments(int V, spec_dtype dt);
spec_status spec_row_partials(const void* logits, spec_dtype dt, int rows, int V,
                              float temperature, int want, void* partials,
                              size_t partials_bytes, hipStream_t s);

/*
 * spec_verify_sample -- speculative sampling verification of B sequences.
 * Pages: "EAGLE-3 speculative decoding review", "Speculative Decoding"
 * (3. Accept or Reject) and "Does Using a Small Model's Answer Reduce
 * Quality?" (A(x) = min(1, p(x)/q(x)); residual norm(max(0, p - q)));
 * "EAGLE math", "Vanilla speculative decoding" ((p - q)_+, the +1 bonus
 * token); "Speculative decoding" wiki, "The mechanism".
 *
 * target_logits [B, gamma+1, V]; draft_logits [B, gamma, V] (same dtype).
 * draft_tokens  [B, gamma] int32, each in [0, V).
 * uniforms      [B, gamma+1] float32 in [0, 1).
 * accept_len    [B] int32 out: j = number of accepted drafts (0..gamma).
 * out_tokens    [B, gamma+1] int32 out: x_0..x_{j-1}, then the resampled
 *               (j < gamma) or bonus (j = gamma) token, then -1 padding.
 * 1 <= gamma <= SPEC_MAX_GAMMA, 1 <= B <= SPEC_MAX_BATCH,
 * 1 <= V <= SPEC_MAX_SAMPLE_VOCAB.
 * Workspace: spec_workspace_bytes(SPEC_MODE_SAMPLE, B, gamma, V, 0).
 */
spec_status spec_verify_sample(const void* target_logits, const void* draft_logits,
                               spec_dtype dt, const int32_t* draft_tokens,
                               const float* uniforms, int B, int gamma, int V,
                               float temperature, int32_t* accept_len,
                               int32_t* out_tokens, void* ws, size_t ws_bytes,
                               hipStream_t s);

/*
 * spec_verify_sample_noalloc -- spec_verify_sample for callers that cannot
 * allocate device memory or hand over a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 *
 * Arguments, outputs and results as spec_verify_sample (bit-identical: the
 * same kernels run on the same layout), without ws / ws_bytes.  The
 * workspace is a static device array of SPEC_NOALLOC_SCRATCH_BYTES bytes in
 * the library, one per GPU, held until the process ends; its address is
 * looked up on the first call on each device.  The call allocates nothing.
 * Sizes whose workspace (spec_workspace_bytes(SPEC_MODE_SAMPLE, B, gamma, V,
 * 0)) exceeds SPEC_NOALLOC_SCRATCH_BYTES are rejected with SPEC_EWORKSPACE
 * before anything is launched (B = 64, gamma = 7, V = 128256 needs about
 * 0.50 MB; the limit holds about 2100 such sequences).  Every call on one GPU
 * shares that GPU's array and leaves its contents behind; the array needs no
 * clearing (each call writes every byte it reads), but calls that overlap in
 * time on the same GPU (several streams, several host threads) race on it
 * and give undefined results: serialise them, or use spec_verify_sample with
 * distinct workspaces.  A failed device lookup reports SPEC_EHIP.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES (16u << 20)
spec_status spec_verify_sample_noalloc(const void* target_logits, const void* draft_logits,
                                       spec_dtype dt, const int32_t* draft_tokens,
                                       const float* uniforms, int B, int gamma, int V,
                                       float temperature, int32_t* accept_len,
                                       int32_t* out_tokens, hipStream_t s);

/*
 * spec_verify_sample_early_exit -- spec_verify_sample with the rows swept in
 * position order: target and draft row i of a sequence are read only if its
 * positions before the block holding i were all accepted.
 * Pages: as spec_verify_sample; "EAGLE-3 speculative decoding review",
 * "Speculative Decoding" (3. Accept or Reject: stop at the first rejection
 * and discard every later draft token) -- the rows after a rejection cannot
 * change the outcome, so they need not be read.
 * Same arguments, workspace and outputs as spec_verify_sample, and the same
 * results bit for bit (the tests between blocks use the same merged
 * statistics and the same ratio as the final accept scan).
 * positions_per_launch  K: positions 0..gamma are swept in blocks of K, one
 *   launch per block; a sequence's next block is read only if every position
 *   of its earlier blocks was accepted.  K = gamma + 1 is one full sweep.
 *   Smaller K reads fewer rows and pays one launch latency (about 5 us) per
 *   block.  0 picks two blocks, position 0 then positions 1..gamma: a
 *   sequence whose first draft is rejected reads one position's rows, and
 *   the others read all of theirs in one more launch.  -1 picks blocks of
 *   1, 2, 4, ... positions: within twice the rows of K = 1 whatever the
 *   acceptance, in ceil(log2(gamma + 2)) launches.  -1 <= K <= gamma + 1.
 */
spec_status spec_verify_sample_early_exit(const void* target_logits, const void* draft_logits,
                                          spec_dtype dt, const int32_t* draft_tokens,
                                          const float* uniforms, int B, int gamma, int V,
                                          float temperature, int positions_per_launch,
                                          int32_t* accept_len, int32_t* out_tokens, void* ws,
                                          size_t ws_bytes, hipStream_t s);

/*
 * spec_verify_greedy -- greedy verification of B sequences.
 * Pages: "EAGLE-3 speculative decoding review", "Does Using a Small Model's
 * Answer Reduce Quality?" (accept iff the draft equals the target's argmax;
 * otherwise emit the target token and discard the rest; the result equals
 * target-only greedy decoding) and "Speculative Decoding" (the bonus token).
 *
 * target_logits [B, gamma+1, V]; draft_tokens [B, gamma] int32.
 * accept_len [B] out; out_tokens [B, gamma+1] out: x_0..x_{j-1}, argmax of
 * row j, then -1.  Draft tokens outside [0, V) never match.
 * Workspace: spec_workspace_bytes(SPEC_MODE_GREEDY, B, gamma, V, 0).
 */
spec_status spec_verify_greedy(const void* target_logits, spec_dtype dt,
                               const int32_t* draft_tokens, int B, int gamma,
                               int V, int32_t* accept_len, int32_t* out_tokens,
                               void* ws, size_t ws_bytes, hipStream_t s);

/*
 * spec_verify_tree -- greedy verification of a candidate tree per sequence.
 * Pages: "EAGLE-3 speculative decoding review", "EAGLE-2: Does Every Context
 * Need the Same Draft Tree?" (each node sees the shared prefix and its own
 * ancestors) and "The Complete EAGLE-3 Inference Process" (4. Strict
 * Acceptance: accept the longest prefix matching the target's choices);
 * "EAGLE math", "EAGLE-2: dynamic draft trees".
 *
 * target_logits [B, N, V]: row n is the target's distribution after node n.
 * node_tokens   [B, N] int32: token carried by node n (node 0 = the last
 *               committed token; it is not verified).
 * parent        [N] (parent_batch_stride = 0, shared) or [B, N]
 *               (parent_batch_stride = N): parent[0] = -1 and
 *               0 <= parent[n] < n.  A violation gives accept_len[b] = -1.
 * accept_len [B] out: depth of the accepted node n* (the deepest node whose
 *            whole root path matches; lowest index among equals).
 * out_path   [B, N] out: node indices of the accepted path, root excluded,
 *            root-to-leaf order, then -1.
 * out_tokens [B, N] out: the path's tokens, then the argmax of row n*
 *            (bonus), then -1.
 * 1 <= N <= SPEC_MAX_TREE_NODES.
 * Workspace: spec_workspace_bytes(SPEC_MODE_TREE, B, N, V, 0).
 */
spec_status spec_verify_tree(const void* target_logits, spec_dtype dt,
                             const int32_t* node_tokens, const int32_t* parent,
                             int parent_batch_stride, int B, int N, int V,
                             int32_t* accept_len, int32_t* out_path,
                             int32_t* out_tokens, void* ws, size_t ws_bytes,
                             hipStream_t s);

/*
 * spec_verify_tree_sample -- stochastic (sampling) verification of a draft
 * tree per sequence, lossless for the target distribution.
 * Pages: "EAGLE-3 speculative decoding review", "The Complete EAGLE-3
 * Inference Process" (4. Strict Acceptance: min(1, p/q) acceptance with
 * residual correction, on the tree) and "Does Using a Small Model's Answer
 * Reduce Quality?" (A(x) = min(1, p(x)/q(x)); resample from
 * norm(max(0, p - q))).
 *
 * p = softmax(target row / T), q = softmax(draft row / T).  From the root:
 * the children of the current node are tested in increasing index; child c,
 * the k-th (token x), is accepted iff uniforms[b][c] < p_k(x) / q_k(x), with
 * p_1 = p and p_{k+1} = norm(max(0, p_k - q_k)) after each rejection; an
 * accepted child becomes the current node.  q_k is the law child k was drawn
 * from: q itself for SPEC_SIBLINGS_IID; for SPEC_SIBLINGS_DISTINCT, q with
 * the tokens of children 1 .. k-1 removed and renormalised (a token repeated
 * among siblings then has q_k(x) = 0 and no residual mass: it is rejected).
 * If every child is rejected one token is drawn from the last residual; at a
 * node without children the bonus token is drawn from p.  The final draw
 * takes uniforms[b][0] (inverse CDF in vocabulary order, as in
 * spec_verify_sample).
 *
 * target_logits, draft_logits [B, N, V] (dt): row n of each belongs to node
 *               n; draft row n is the law n's children were drawn from.
 *               Only the rows of nodes the walk reaches are read: the target
 *               row of every visited node, the draft row of every visited
 *               node with children.
 * node_tokens   [B, N] int32 (node 0's token is not read).
 * parent        [N] (parent_batch_stride = 0) or [B, N] (= N): parent[0] = -1
 *               and 0 <= parent[n] < n.
 * uniforms      [B, N] float32 in [0, 1).
 * siblings      SPEC_SIBLINGS_IID or SPEC_SIBLINGS_DISTINCT (else EINVAL).
 * n_sweep       nodes 0 .. n_sweep-1 of every sequence have both rows swept
 *               across the whole GPU before the walk; deeper visited nodes
 *               are reduced when the walk reaches them.  -1 picks the prefix
 *               from B, N and V.  -1 <= n_sweep <= N.
 * n_rounds      the walk's passes over a node's rows (its row statistics on
 *               arrival, the residual mass W after a rejected sibling) run
 *               across the whole GPU in up to n_rounds rounds, two launches
 *               each; passes a walk still needs after them run on its
 *               sequence's own workgroup.  -1 picks a number from N;
 *               -1 <= n_rounds <= SPEC_MAX_TREE_ROUNDS.  Outputs depend on
 *               neither n_sweep nor n_rounds: every placement of a pass
 *               gives the same bits.
 * accept_len [B] out: number of accepted nodes; -1 when the tree is invalid
 *            or a token of a node n >= 1 lies outside [0, V) (outputs -1).
 * out_path   [B, N] out: accepted nodes (root excluded) in root-to-leaf
 *            order, then -1.
 * out_tokens [B, N] out: their tokens, then the drawn token, then -1.
 * 1 <= N <= SPEC_MAX_TREE_NODES, 1 <= V <= SPEC_MAX_SAMPLE_VOCAB.
 * Logit pointers 16-byte aligned, the others 4-byte aligned.
 * Workspace: spec_workspace_bytes(SPEC_MODE_TREE_SAMPLE, B, N, V, n_sweep).
 */
spec_status spec_verify_tree_sample(const void* target_logits, const void* draft_logits,
                                    spec_dtype dt, const int32_t* node_tokens,
                                    const int32_t* parent, int parent_batch_stride,
                                    const float* uniforms, int B, int N, int V,
                                    float temperature, spec_siblings siblings, int n_sweep,
                                    int n_rounds, int32_t* accept_len,
                                    int32_t* out_path, int32_t* out_tokens, void* ws,
                                    size_t ws_bytes, hipStream_t s);

/*
 * lmhead_project -- logits of feature rows through the LM head, z = h W.
 * Pages: "EAGLE-3 speculative decoding review", "EAGLE: Predict Features, Not
 * Tokens" (the LM head turns the top-layer feature into vocabulary logits;
 * the draft reuses the target's LM head); "EAGLE math", "EAGLE's move".
 *
 * feat [M, d] bf16 bits; W bf16 bits, [d, V] (wl = SPEC_W_DV) or [V, d]
 * (wl = SPEC_W_VD); out_logits [M, V] float32 (bf16 x bf16 products, float32
 * accumulation; both layouts give bit-identical logits).  feat, W and
 * out_logits 16-byte aligned.  d must be a multiple of 64; 1 <= M <= 2^22,
 * 1 <= V < 2^25.
 */
spec_status lmhead_project(const uint16_t* feat, int M, int d, const uint16_t* W,
                           spec_wlayout wl, int V, float* out_logits, hipStream_t s);

/*
 * lmhead_project_staged -- the same product as lmhead_project, bit for bit,
 * with the feature rows first copied into the workspace as contiguous 16 KB
 * blocks (256 rows x 32 features each), so that every GEMM load of them reads
 * whole cache lines; faster than lmhead_project, most for [V, d] weights.
 * Pages: as lmhead_project.
 *
 * Arguments as lmhead_project; ws is caller-owned device memory, 256-byte
 * aligned, of at least lmhead_project_workspace_bytes(M, d) bytes
 * (SPEC_EWORKSPACE otherwise), overwritten by the call.
 */
spec_status lmhead_project_staged(const uint16_t* feat, int M, int d, const uint16_t* W,
                                  spec_wlayout wl, int V, float* out_logits, void* ws,
                                  size_t ws_bytes, hipStream_t s);

/* Workspace bytes lmhead_project_staged needs; 0 for an invalid (M, d). */
size_t lmhead_project_workspace_bytes(int M, int d);

/*
 * lmhead_verify -- EAGLE-style verification: draft features are decoded
 * through the target's own, unchanged LM head, and the result is verified
 * like any draft.
 * Pages: "EAGLE-3 speculative decoding review", "EAGLE: Predict Features, Not
 * Tokens" (the LM head turns the top-layer feature into vocabulary logits;
 * the draft reuses the target's head); "EAGLE math", "EAGLE's move" and
 * "Why feature drafting lands a higher acceptance rate"; verification as in
 * spec_verify_sample.
 *
 * target_feat  [B*(gamma+1), d] bf16 bits: row b*(gamma+1)+i is the target's
 *              feature for position i of sequence b (i = gamma: bonus row).
 * draft_feat   [B*gamma, d] bf16 bits: row b*gamma+i is the drafted feature
 *              of position i.
 * W            [d, V] bf16 bits, vocabulary innermost (lmhead_verify_wvd
 *              takes the [V, d] layout).  No bias: z = h W.
 * draft_tokens, uniforms, temperature, accept_len, out_tokens: as in
 *              spec_verify_sample (p from the target rows, q from the draft
 *              rows, both float32 logits).
 * d a multiple of 64 (<= 2^20); 1 <= V < 2^25; gamma and B as in
 * spec_verify_sample.  Feature and weight pointers 16-byte aligned.
 * The feature rows (target rows, then draft rows) are first staged in the
 * workspace in the blocked layout of lmhead_project_staged, so one GEMM
 * streams W once for both; the logits stay in the workspace (float32, no
 * host round trip) for the verification kernels.  The GEMM's epilogue also
 * leaves each row's softmax statistics (max and sum of exp((z - max)/T)) as
 * one partial per 128 columns, computed from the accumulators before they are
 * stored; a merge of those gives the accept test its p and q normalisers, so
 * the logits are read back only for the rows the final draw needs.
 * Workspace: spec_workspace_bytes(SPEC_MODE_LMHEAD, B, gamma, V, d).  After
 * the call the logits are left in the last ceil256(B(2 gamma+1) V 4) bytes
 * of the workspace: B(gamma+1) target rows, then B gamma draft rows.
 * Errors: as spec_verify_sample; an invalid d gives SPEC_EINVAL.
 */
spec_status lmhead_verify(const uint16_t* target_feat, const uint16_t* draft_feat,
                          const uint16_t* W, const int32_t* draft_tokens,
                          const float* uniforms, int B, int gamma, int d, int V,
                          float temperature, int32_t* accept_len,
                          int32_t* out_tokens, void* ws, size_t ws_bytes,
                          hipStream_t s);

/*
 * lmhead_verify_wvd -- lmhead_verify with the LM-head weight stored [V, d]
 * (feature dimension innermost, the way a linear layer's weight is usually
 * kept).  Pages: as lmhead_verify.
 *
 * W_vd [V, d] bf16 bits, 16-byte aligned; every other argument, the
 * workspace and the outputs as in lmhead_verify.  For the same weights the
 * logits, and so the outputs, are bit-identical to lmhead_verify's with
 * W = W_vd^T: the GEMM feeds the MFMAs the same values in the same order.
 */
spec_status lmhead_verify_wvd(const uint16_t* target_feat, const uint16_t* draft_feat,
                              const uint16_t* W_vd, const int32_t* draft_tokens,
                              const float* uniforms, int B, int gamma, int d, int V,
                              float temperature, int32_t* accept_len,
                              int32_t* out_tokens, void* ws, size_t ws_bytes,
                              hipStream_t s);

/*
 * spec_probe_probs -- test probe: the full distributions the sampling path
 * works with, for `rows` pairs of target/draft rows, computed by the same
 * device statistics and element functions as spec_verify_sample's draw.
 * Pages: as spec_verify_sample.
 *
 * target_logits, draft_logits [rows, V] (draft may be NULL: then q and the
 * residual are not produced).
 * out_p, out_q, out_resid [rows, V] float64: p, q and the normalised
 * residual max(0, p - q) / sum(max(0, p - q)) (all zeros when p == q
 * everywhere).  out_q / out_resid may be NULL.
 * Workspace: spec_workspace_bytes(SPEC_MODE_ROWSTATS, 2*rows, 0, V, 0).
 */
spec_status spec_probe_probs(const void* target_logits, const void* draft_logits,
                             spec_dtype dt, int rows, int V, float temperature,
                             double* out_p, double* out_q, double* out_resid,
                             void* ws, size_t ws_bytes, hipStream_t s);

/*
 * spec_kv_compact -- keep only the accepted path's KV-cache entries.
 * Pages: "EAGLE-3 speculative decoding review", "The Complete EAGLE-3
 * Inference Process" (5. Update the KV Cache: keep the accepted path's
 * cache, discard rejected branches, resume drafting from the committed
 * prefix) and "Implementation Is More Complex Than a Simple Two-Model Setup"
 * (prune the KV cache to the accepted branch).
 *
 * kv: the cache, modified in place.  Entry (sequence b, plane p, slot s) is
 *     entry_bytes contiguous bytes at kv + b*seq_stride + p*plane_stride +
 *     s*entry_bytes (a plane is one layer's keys or values; slots of a plane
 *     are contiguous).  The B x planes blocks of S entries must not overlap:
 *     planes inside sequences ([B][planes][S]) or sequences inside planes
 *     ([planes][B][S]), padding allowed.
 * prefix_len [B]: L_b, entries cached before the verification forward; that
 *     forward wrote tree node n (node 0 = the last committed token) at slot
 *     L_b + n.
 * path [B, path_stride]: accepted nodes in depth order, as spec_verify_tree
 *     writes them (out_path, path_stride = N); NULL for linear drafts, whose
 *     accepted tokens already sit in place.
 * accept_len [B]: d_b from the verify call.
 * new_len [B] out: L_b + 1 + d_b, or -1 (nothing moved) when d_b < 0 or the
 *     path does not rise strictly from 1 or leaves the cache.
 * Effect: slot L_b + t receives the pre-call entry of slot L_b + path[t-1]
 * for t = 1..d_b, in every plane; all other slots are untouched.
 * kv, strides and entry_bytes 16-byte aligned (entry_bytes >= 16); the int
 * arrays 4-byte aligned.  No workspace.
 */
spec_status spec_kv_compact(void* kv, int B, int planes, int S, long long entry_bytes,
                            long long seq_stride, long long plane_stride,
                            const int32_t* prefix_len, const int32_t* path, int path_stride,
                            const int32_t* accept_len, int32_t* new_len, hipStream_t s);

/*
 * spec_tree_expand -- one depth of the EAGLE-2 dynamic draft tree.
 * Pages: "EAGLE math", "EAGLE-2: dynamic draft trees" (grow the tree by
 * expanding the nodes with the highest cumulative draft probability, prune,
 * re-rank); "EAGLE-3 speculative decoding review", "EAGLE-2: Does Every
 * Context Need the Same Draft Tree?" and "The Complete EAGLE-3 Inference
 * Process" (2. Generate a Draft Tree).
 *
 * Node table, per sequence b (row b of each [B, cap] array): parent (table
 * index, -1 for the root), token, score (float64 cumulative draft
 * log-probability, the root 0), depth (root 0).  The caller writes the root
 * at index 0 (parent -1, its token, score 0, depth 0) before the first call.
 * draft_logits [B, K_in, V]: the draft rows of the frontier nodes.
 * frontier [B, K_in]: their table indices; -1 (or an index >= off) marks an
 *     empty slot.  The first depth expands the root: K_in = 1, frontier 0.
 * For every frontier node: q = softmax(z / T); its k tokens with the largest
 * q (equal logits: lower index first) become children at table positions
 * off + f*k + r (slot f, rank r), score = parent score + log q(token),
 * depth = parent depth + 1.  Empty slots get placeholders (parent -1, token
 * -1, score -inf, depth -1).
 * next_frontier [B, K_out] out: the K_out children with the highest score
 *     (equal scores: lower table position first), -1 padded.  The next call
 *     takes it as its frontier with off += K_in * k.
 * 1 <= k <= SPEC_MAX_TOPK, K_in, K_out <= SPEC_MAX_FRONTIER, K_in * k <= 1024,
 * V >= k, off >= 1, off + K_in * k <= cap.  Every row of a non-empty slot
 * needs a finite logit.
 * Workspace: spec_workspace_bytes(SPEC_MODE_TREE_EXPAND, B, K_in, V, 0).
 */
spec_status spec_tree_expand(const void* draft_logits, spec_dtype dt, const int32_t* frontier,
                             int B, int K_in, int V, float temperature, int k, int K_out,
                             int32_t* node_parent, int32_t* node_token, double* node_score,
                             int32_t* node_depth, int cap, int off, int32_t* next_frontier,
                             void* ws, size_t ws_bytes, hipStream_t s);

/*
 * spec_tree_build -- re-rank the drafted nodes and lay out the tree with its
 * attention mask.
 * Pages: "EAGLE math", "EAGLE-2: dynamic draft trees" (re-rank which
 * candidates to keep; the verified node count stays fixed; a tree attention
 * mask scores every candidate in one pass); "EAGLE-3 speculative decoding
 * review", "EAGLE-2: Does Every Context Need the Same Draft Tree?" (a node
 * sees the shared prefix and its own ancestors only).
 *
 * Reads table entries 0 .. n_nodes-1 (the table spec_tree_expand fills).
 * Keeps the root and the M drafted nodes with the highest score (equal
 * scores: shallower first, then lower table index); a child never outscores
 * its parent, so the kept set is a tree.  Output node order: depth, then
 * score (higher first), then table index; parent[i] < i.
 * out_n [B]: 1 + min(M, drafted nodes), or -1 if the table breaks the
 *     expansion's invariants (root not at 0, a parent after its child, depth
 *     not parent depth + 1, a kept node whose parent is not kept).
 * out_parent, out_token, out_depth, out_index (table index) [B, M+1]: -1
 *     padded past out_n.
 * out_mask [B, M+1, W], W = ceil((M+1)/32) uint32 words: bit j of row i set
 *     iff node j is node i or one of its ancestors (what node i may attend to
 *     besides the committed prefix); zero rows past out_n.
 * n_nodes <= cap, n_nodes <= SPEC_MAX_BUILD_NODES, M + 1 <= SPEC_MAX_BUILD_NODES.
 * The outputs feed spec_verify_tree (parent and tokens).
 */
spec_status spec_tree_build(const int32_t* node_parent, const int32_t* node_token,
                            const double* node_score, const int32_t* node_depth, int B, int cap,
                            int n_nodes, int M, int32_t* out_n, int32_t* out_parent,
                            int32_t* out_token, int32_t* out_depth, int32_t* out_index,
                            uint32_t* out_mask, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
