/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) library for batched
 * speculative-sampling verification.
 *
 * The operation ("Speculative Decoding 的朴素思想", sections "一次 sampling 怎么执行",
 * "Correction 为什么用正残差" and "从单个 token 接到一段 draft"; "推测解码：接受规则、
 * 状态与收益边界", section "两模型精确采样"):
 *
 *   For each sequence b, a draft model proposed G tokens x_1..x_G, drawing x_i from
 *   q_i; the target gave G+1 distributions p_1..p_{G+1} for the same prefixes.  Both
 *   come in as logits and pass through the same policy (temperature T, optional
 *   top-k).  Positions are tested in order: x_i is accepted when U_i <= min(1,
 *   p_i(x_i)/q_i(x_i)) (and p_i(x_i) > 0).  At the first rejected position j a
 *   correction token is drawn from norm([p_j - q_j]_+) by inverse CDF with u_sample[b];
 *   if all G are accepted a bonus token is drawn from p_{G+1} the same way.  With
 *   T == 0 the policy is greedy (argmax, lowest index on ties): acceptance is exact
 *   match with the target argmax, and the correction / bonus is the target argmax
 *   ("tannlonggtaoo" note, section "Greedy Sampling").
 *
 * Conventions shared by every entry point:
 *   - All array arguments are DEVICE pointers to row-major, contiguous memory on the
 *     current HIP device; sizes are element counts.  Logit rows must be aligned to
 *     their element size (2 bytes for bf16, 4 for f32); rows whose byte length is a
 *     multiple of 16 with 16-byte-aligned bases take the vector-load path.
 *   - The caller owns every buffer.  The library allocates nothing, keeps no data
 *     between calls (only a process-wide counter that gives each call a distinct tag),
 *     and never synchronises: work is enqueued on `stream` (a hipStream_t; NULL is the
 *     default stream) and results are valid in stream order.
 *   - On any status other than SV_OK nothing has been enqueued and outputs are
 *     untouched.  Row-level data problems are not statuses: they are reported per
 *     sequence in accepted_len (codes below).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The two sentinels give the enumeration the range of int32_t, so any value a caller
 * passes (an unsupported one is answered with SV_ERR_DTYPE) is a valid value of the type. */
typedef enum { SV_DTYPE_INVALID = -1, SV_F32 = 0, SV_BF16 = 1, SV_DTYPE_LIMIT = 0x7fffffff } sv_dtype;

typedef enum {
  SV_OK = 0,
  SV_ERR_NULL = 1,        /* a required pointer is NULL                                  */
  SV_ERR_SHAPE = 2,       /* B < 1, G < 0, V < 1, or a size that overflows the launch    */
  SV_ERR_DTYPE = 3,       /* dtype is not SV_F32 / SV_BF16                               */
  SV_ERR_TEMPERATURE = 4, /* temperature negative, NaN or infinite                       */
  SV_ERR_WORKSPACE = 5,   /* workspace smaller than sv_workspace_bytes() or misaligned    */
  SV_ERR_ALIGN = 6,       /* a logit pointer is not aligned to its element size           */
  SV_ERR_LAUNCH = 7,      /* the HIP runtime refused a kernel launch                       */
  SV_ERR_PARAM = 8,       /* spec_typical_verify: epsilon or delta negative or not finite   */
  SV_ERR_SCRATCH = 9      /* spec_verify_noalloc: the arguments need more scratch memory    */
                          /* than SV_NOALLOC_SCRATCH_BYTES                                   */
} sv_status;

/* Row-level codes written into accepted_len[b] instead of a length; the whole row of
 * out_tokens is then -1.  They follow the checks of the single-position reference
 * ("推测解码：接受规则、状态与收益边界", section "单位置接受 reference"), tested in this
 * order over all G positions of the sequence, whether or not a position is reached: */
#define SV_ROW_BAD_TOKEN (-1)   /* a drafted token lies outside [0, V)                      */
#define SV_ROW_Q_ZERO (-2)      /* sampling: q_i(x_i) = 0 (logit -inf or cut by top-k), so   */
                                /* the draft cannot have proposed x_i                        */
#define SV_ROW_BAD_LOGITS (-3)  /* a row of the sequence holds NaN or +inf, or no finite logit */
#define SV_ROW_BAD_UNIFORM (-4) /* sampling: a u_accept or u_sample value outside [0, 1)    */
/* Not a data problem: a workgroup of the sampling kernel gave up waiting for results of
 * workgroups earlier in its grid (a bounded wait of about a second that ordinary
 * scheduling never reaches).  The sequence's out_tokens are then incomplete. */
#define SV_ROW_INTERNAL (-5)
/* spec_tree_verify: the parent array is not a tree in topological order (parent[0] must be
 * -1 and 0 <= parent[n] < n), or a node has more children than max_children. */
#define SV_ROW_BAD_TREE (-6)

/* Bytes of device workspace spec_verify needs for these arguments (0 never occurs). */
size_t sv_workspace_bytes(int32_t B, int32_t G, int32_t V, sv_dtype dtype, float temperature,
                          int32_t top_k);

/* Leading bytes of the workspace (words that workgroups hand to one another, each marked
 * with a tag unique to its kernel launch) that must be zero when a workspace is first
 * used with these arguments;
 * 0 for arguments spec_verify would reject.  A completed call leaves its own leading
 * sv_workspace_zero_bytes(...) bytes holding zeros and marks of completed calls, which
 * every later call treats as zero, and may overwrite everything after them.  So one
 * zero-fill serves any number of calls with the same arguments; before a call whose
 * zero prefix is longer than the previous call's on the same workspace, zero the longer
 * prefix again (a fill kernel on the same stream suffices).  Calls that share a
 * workspace must not overlap in time. */
size_t sv_workspace_zero_bytes(int32_t B, int32_t G, int32_t V, sv_dtype dtype,
                               float temperature, int32_t top_k);

/* Tag epoch: the process's tag count in units of 2^31.  Each kernel launch marks its
 * words with 32-bit tags taken from that count (one tag; a tree verification's draw
 * launch takes N + 1 consecutive ones, one per round of residual masses), and a tag value
 * comes back after 2^32 - 1 tags: a workspace word last written exactly that many tags
 * earlier would then pass for the current launch's.  A caller that keeps a workspace
 * across calls records this value whenever it zeroes the workspace's prefix, and zeroes
 * the prefix again (all of it ever used) before the first call after the value changed.
 * That happens once every 2^31 tags; no call is refused. */
uint32_t sv_tag_epoch(void);

/* Batched verification.
 *   target_logits [B, G+1, V] dtype   target logits for positions 1..G+1
 *   draft_logits  [B, G,   V] dtype   draft logits for positions 1..G; not read (may be
 *                                     NULL) when temperature == 0 or G == 0
 *   draft_tokens  [B, G]  int32       drafted tokens; may be NULL when G == 0
 *   u_accept      [B, G]  float32     acceptance uniforms in [0,1); not read when
 *                                     temperature == 0 (may then be NULL)
 *   u_sample      [B]     float32     one uniform per sequence for the correction or
 *                                     bonus draw; not read when temperature == 0
 *   temperature   T > 0 samples from softmax(z/T); T == 0 is greedy
 *   top_k         0 < top_k < V keeps every logit >= the top_k-th largest raw logit
 *                 (ties kept) in target and draft rows alike; otherwise no cut.
 *                 Ignored when temperature == 0.
 *   accepted_len  [B]     int32 out   0..G, or a negative row code
 *   out_tokens    [B, G+1] int32 out  accepted drafts, then the correction / bonus
 *                                     token at index accepted_len, then -1
 *   row_stats     [B, 2G+1, 2] float32 out, nullable: for each target row (0..G) then
 *                 draft row (0..G-1) of a sequence, (m, S) with m + ln S the natural
 *                 log-partition of the kept logits divided by T.  Not written when
 *                 temperature == 0.
 *   workspace     device buffer of at least sv_workspace_bytes(...) bytes, 256-byte
 *                 aligned, whose first sv_workspace_zero_bytes(...) bytes are zero.
 */
sv_status spec_verify(const void *target_logits, const void *draft_logits, sv_dtype dtype,
                      const int32_t *draft_tokens, const float *u_accept, const float *u_sample,
                      int32_t B, int32_t G, int32_t V, float temperature, int32_t top_k,
                      int32_t *accepted_len, int32_t *out_tokens, float *row_stats,
                      void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc: spec_verify with the library's own
 * scratch memory in place of the caller's workspace.  The arguments and results are those
 * of spec_verify; the kernels are the same.  The scratch is one array of
 * SV_NOALLOC_SCRATCH_BYTES bytes per GPU, a static device variable of the library that
 * each GPU holds from the first call on it until the process ends; the call allocates
 * nothing (no hipMalloc, no hipFree, no allocating library routine).
 *   - Arguments whose workspace (sv_workspace_bytes) exceeds SV_NOALLOC_SCRATCH_BYTES are
 *     refused with SV_ERR_SCRATCH; nothing is enqueued.
 *   - The first call on a device looks the array's device address up (hipGetSymbolAddress,
 *     on the current device) and keeps it; a failure of that lookup returns
 *     SV_ERR_LAUNCH.  Before a call whose leading words must be zero and are not known to
 *     be (the first call, a longer prefix than before, a new tag epoch), a fill kernel
 *     clears them on `stream`.
 *   - Every call on a GPU uses that GPU's one array, which keeps the last call's contents:
 *     calls that overlap in time on one GPU (on different streams, or from different host
 *     threads) race and must not be made.  Calls ordered on one stream are safe. */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
sv_status spec_verify_noalloc(const void *target_logits, const void *draft_logits, sv_dtype dtype,
                              const int32_t *draft_tokens, const float *u_accept,
                              const float *u_sample, int32_t B, int32_t G, int32_t V,
                              float temperature, int32_t top_k, int32_t *accepted_len,
                              int32_t *out_tokens, float *row_stats, void *stream);

/* spec_verify that also times each of its kernels with HIP events.
 * events: array of n_events hipEvent_t handles (created by the caller, with timing
 * enabled); kernel i is launched with events[2i] as its start event and events[2i+1]
 * as its stop event (hipExtLaunchKernel), so the pair brackets that dispatch alone.
 * *n_launched receives the number of kernels enqueued (at most SV_MAX_LAUNCHES);
 * kernels beyond n_events / 2 are launched untimed.  Otherwise identical to
 * spec_verify. */
#define SV_MAX_LAUNCHES 8
sv_status spec_verify_timed(const void *target_logits, const void *draft_logits, sv_dtype dtype,
                            const int32_t *draft_tokens, const float *u_accept,
                            const float *u_sample, int32_t B, int32_t G, int32_t V,
                            float temperature, int32_t top_k, int32_t *accepted_len,
                            int32_t *out_tokens, float *row_stats, void *workspace,
                            size_t workspace_bytes, void *stream, void *const *events,
                            int32_t n_events, int32_t *n_launched);

/* Names of the kernels spec_verify would launch for these arguments, in launch order,
 * as one string separated by ';' (static storage).  Used to match per-kernel timings
 * with profiler output. */
const char *sv_launch_plan(int32_t B, int32_t G, int32_t V, sv_dtype dtype, float temperature,
                           int32_t top_k);

/* ---- batched sampler (the step before verification, and plain decoding) ----
 *
 * One draw per row from the row's own distribution ("Speculative Decoding 的朴素思想",
 * section "一次 sampling 怎么执行", step 1: a uniform picks the token whose cumulative
 * interval holds it; this is the draft's own draw X ~ q, and plain decoding from p).
 * Row b's logits pass through the same policy as in spec_verify (temperature T, optional
 * top-k); tokens[b] is the first v, in index order, whose cumulative probability exceeds
 * u[b] times the total.  T == 0 takes the lowest-index argmax and reads no uniform.
 *   logits      [B, V] dtype
 *   u           [B] float32 in [0,1); may be NULL when temperature == 0
 *   tokens      [B] int32 out: the drawn token, or -1 when the row has a code
 *   row_status  [B] int32 out: 0, or SV_ROW_BAD_LOGITS (a NaN or +inf logit, or no finite
 *               kept logit), SV_ROW_BAD_UNIFORM (T > 0 and u[b] outside [0,1)), or
 *               SV_ROW_INTERNAL
 *   workspace   at least sv_workspace_bytes(B, 0, V, dtype, temperature, top_k) bytes,
 *               256-byte aligned, first sv_workspace_zero_bytes(B, 0, V, ...) bytes zero
 *               (the same rules as spec_verify's workspace).
 * The draw is spec_verify's bonus draw with G = 0 (p_1 = the row): the same kernels and
 * argument checks; statuses as for spec_verify. */
sv_status spec_sample(const void *logits, sv_dtype dtype, const float *u, int32_t B, int32_t V,
                      float temperature, int32_t top_k, int32_t *tokens, int32_t *row_status,
                      void *workspace, size_t workspace_bytes, void *stream);

/* spec_sample with each kernel dispatch bracketed by caller-owned HIP events, as in
 * spec_verify_timed. */
sv_status spec_sample_timed(const void *logits, sv_dtype dtype, const float *u, int32_t B,
                            int32_t V, float temperature, int32_t top_k, int32_t *tokens,
                            int32_t *row_status, void *workspace, size_t workspace_bytes,
                            void *stream, void *const *events, int32_t n_events,
                            int32_t *n_launched);

/* ---- overlap of target and draft at every drafted position ----
 *
 * For each sequence b and drafted position i, the two distributions the verification
 * compares there, p_i (target row i) and q_i (draft row i), after the same temperature
 * and top-k as in spec_verify:
 *   beta[b, i] = sum_v min(p_i(v), q_i(v))   the position's acceptance probability
 *                ("Speculative Decoding 的朴素思想", section "为什么接受概率恰好是这个比值";
 *                the overlap 1 - TV behind the LK loss -log beta and DSpark's label
 *                c* = 1 - ||p - q||_1 / 2 on "推测解码：接受规则、状态与收益边界")
 *   tv[b, i]   = sum_v max(p_i(v) - q_i(v), 0)  the rejection mass Z, summed from its own
 *                terms (not as 1 - beta) so that small distances keep their precision.
 *   target_logits [B, target_rows, V] dtype  target_rows = G + 1 (the verification's
 *                                            layout; row G is not read) or G
 *   draft_logits  [B, G, V] dtype
 *   temperature   T > 0 (T == 0 is SV_ERR_TEMPERATURE: greedy has no distribution)
 *   top_k         as in spec_verify
 *   beta, tv      [B, G] float64 out; NaN for a pair with a code
 *   pair_status   [B, G] int32 out: 0, SV_ROW_BAD_LOGITS (either row holds NaN or +inf,
 *                 or has no finite kept logit) or SV_ROW_INTERNAL
 *   workspace     at least sv_overlap_workspace_bytes(...) bytes, 256-byte aligned, first
 *                 sv_overlap_workspace_zero_bytes(...) bytes zero, under the same rules
 *                 as spec_verify's workspace (one workspace may serve both).
 * G == 0 returns SV_OK and enqueues nothing.  Other statuses as for spec_verify;
 * target_rows other than G or G + 1 is SV_ERR_SHAPE. */
size_t sv_overlap_workspace_bytes(int32_t B, int32_t G, int32_t V, sv_dtype dtype,
                                  float temperature, int32_t top_k);
size_t sv_overlap_workspace_zero_bytes(int32_t B, int32_t G, int32_t V, sv_dtype dtype,
                                       float temperature, int32_t top_k);
sv_status spec_overlap(const void *target_logits, const void *draft_logits, sv_dtype dtype,
                       int32_t B, int32_t G, int32_t V, int32_t target_rows, float temperature,
                       int32_t top_k, double *beta, double *tv, int32_t *pair_status,
                       void *workspace, size_t workspace_bytes, void *stream);

/* spec_overlap with each kernel dispatch bracketed by caller-owned HIP events, as in
 * spec_verify_timed. */
sv_status spec_overlap_timed(const void *target_logits, const void *draft_logits, sv_dtype dtype,
                             int32_t B, int32_t G, int32_t V, int32_t target_rows,
                             float temperature, int32_t top_k, double *beta, double *tv,
                             int32_t *pair_status, void *workspace, size_t workspace_bytes,
                             void *stream, void *const *events, int32_t n_events,
                             int32_t *n_launched);

/* Names of the kernels spec_overlap would launch, ';'-separated (static storage). */
const char *sv_overlap_launch_plan(int32_t B, int32_t G, int32_t V, sv_dtype dtype,
                                   float temperature, int32_t top_k);

/* ---- verification of a draft tree ----
 *
 * Each sequence proposes a tree of N nodes ("Speculative Decoding 的朴素思想", section
 * "Token Tree Verifier": SpecInfer's multi-step speculative sampling; the EAGLE page,
 * section 6.2: rejection node by node).  Node 0 is the committed context; node n >= 1 has
 * parent[b, n] < n and token tokens[b, n]; children of a node are drawn independently from
 * the node's draft distribution and are taken in index order.
 *   target_logits [B, N, V] dtype  p_u: the target's distribution after node u's path
 *   draft_logits  [B, N, V] dtype  q_u: the distribution u's children were drawn from
 *                                  (rows of leaves are not read; NULL allowed at T == 0)
 *   tokens, parent [B, N] int32    node tokens (node 0's unused) and parents (parent[b,0] = -1)
 *   u_accept [B, N] float32        the uniform of node n's test (node 0's unused)
 *   u_sample [B] float32           the uniform of the final draw
 *   max_children                   the most children any node has (0 <= it <= N - 1).
 *                                  At T > 0 with max_children >= 2 a row may span at most
 *                                  32 chunks of 32 KiB (V <= 524288 bf16, 262144 f32):
 *                                  the residual masses are formed by one workgroup per
 *                                  chunk of the tree, which wait for one another.
 *                                  Longer rows are SV_ERR_SHAPE there.
 * The walk starts at the root and tests the node's children in order: the first child
 * against p_u by U <= min(1, p_u(x)/q_u(x)); each rejection replaces the current
 * distribution by norm([cur - q_u]_+) and the next child is tested against it.  An
 * accepted child becomes the node; if every child is rejected the token is drawn from the
 * current distribution by inverse CDF with u_sample, at a leaf the bonus is drawn from p_u.
 * T == 0: the first child whose token is argmax p_u is accepted, else argmax p_u ends the
 * round; draft logits and uniforms are not read.
 *   accepted_len [B] int32 out    the depth reached (accepted tokens), or a negative code
 *   out_tokens   [B, N] int32 out the accepted tokens, then the final token, then -1
 *   path_nodes   [B, N] int32 out the accepted nodes, then -1 (nullable)
 * Row codes (tested in this order): SV_ROW_INTERNAL, SV_ROW_BAD_TREE, SV_ROW_BAD_TOKEN (a
 * token of node n >= 1 outside [0, V)), SV_ROW_BAD_LOGITS (any target row, or the draft row
 * of a node with children), SV_ROW_BAD_UNIFORM, SV_ROW_Q_ZERO (q_parent(n)(x_n) = 0).
 * Workspace: sv_tree_workspace_bytes(...) bytes, 256-byte aligned, first
 * sv_tree_workspace_zero_bytes(...) bytes zero, under the rules of spec_verify's workspace.
 * N is at most 1024. */
size_t sv_tree_workspace_bytes(int32_t B, int32_t N, int32_t V, int32_t max_children,
                               sv_dtype dtype, float temperature, int32_t top_k);
size_t sv_tree_workspace_zero_bytes(int32_t B, int32_t N, int32_t V, int32_t max_children,
                                    sv_dtype dtype, float temperature, int32_t top_k);
sv_status spec_tree_verify(const void *target_logits, const void *draft_logits, sv_dtype dtype,
                           const int32_t *tokens, const int32_t *parent, const float *u_accept,
                           const float *u_sample, int32_t B, int32_t N, int32_t V,
                           int32_t max_children, float temperature, int32_t top_k,
                           int32_t *accepted_len, int32_t *out_tokens, int32_t *path_nodes,
                           void *workspace, size_t workspace_bytes, void *stream);

/* spec_tree_verify with each kernel dispatch bracketed by caller-owned HIP events, as in
 * spec_verify_timed. */
sv_status spec_tree_verify_timed(const void *target_logits, const void *draft_logits,
                                 sv_dtype dtype, const int32_t *tokens, const int32_t *parent,
                                 const float *u_accept, const float *u_sample, int32_t B,
                                 int32_t N, int32_t V, int32_t max_children, float temperature,
                                 int32_t top_k, int32_t *accepted_len, int32_t *out_tokens,
                                 int32_t *path_nodes, void *workspace, size_t workspace_bytes,
                                 void *stream, void *const *events, int32_t n_events,
                                 int32_t *n_launched);

/* Names of the kernels spec_tree_verify would launch, ';'-separated (static storage). */
const char *sv_tree_launch_plan(int32_t B, int32_t N, int32_t V, int32_t max_children,
                                sv_dtype dtype, float temperature, int32_t top_k);

/* ---- typical acceptance ----
 *
 * Medusa's typical acceptance ("Speculative Decoding 的朴素思想", section "Medusa-1 与
 * typical acceptance"): drafted token x_i is accepted when
 *   p_i(x_i) > min(epsilon, delta * exp(-H(p_i))),
 * with p_i the target's distribution at position i after temperature and top-k (as in
 * spec_verify) and H its entropy in nats.  The accepted prefix is the longest run of
 * accepted positions; the token after it is the target's greedy choice argmax p_{j+1}
 * (lowest index on ties).  Not distribution-preserving; reads no draft logits and no
 * uniforms.
 *   target_logits [B, G+1, V] dtype
 *   draft_tokens  [B, G] int32 (may be NULL when G == 0)
 *   temperature   T > 0 (T == 0 is SV_ERR_TEMPERATURE: use spec_verify's greedy mode)
 *   epsilon, delta >= 0 and finite (else SV_ERR_PARAM); epsilon = 0 accepts every token
 *                 with p > 0
 *   accepted_len  [B] int32 out: 0..G, or SV_ROW_BAD_TOKEN / SV_ROW_BAD_LOGITS (any of
 *                 the G+1 rows) / SV_ROW_INTERNAL
 *   out_tokens    [B, G+1] int32 out: accepted drafts, then argmax p_{j+1}, then -1
 * G is at most 256.  Workspace: sv_typical_workspace_bytes(...) bytes, 256-byte aligned,
 * first sv_typical_workspace_zero_bytes(...) bytes zero, under spec_verify's rules. */
size_t sv_typical_workspace_bytes(int32_t B, int32_t G, int32_t V, sv_dtype dtype,
                                  float temperature, int32_t top_k);
size_t sv_typical_workspace_zero_bytes(int32_t B, int32_t G, int32_t V, sv_dtype dtype,
                                       float temperature, int32_t top_k);
sv_status spec_typical_verify(const void *target_logits, sv_dtype dtype,
                              const int32_t *draft_tokens, int32_t B, int32_t G, int32_t V,
                              float temperature, int32_t top_k, float epsilon, float delta,
                              int32_t *accepted_len, int32_t *out_tokens, void *workspace,
                              size_t workspace_bytes, void *stream);

/* spec_typical_verify with each kernel dispatch bracketed by caller-owned HIP events, as in
 * spec_verify_timed. */
sv_status spec_typical_verify_timed(const void *target_logits, sv_dtype dtype,
                                    const int32_t *draft_tokens, int32_t B, int32_t G,
                                    int32_t V, float temperature, int32_t top_k, float epsilon,
                                    float delta, int32_t *accepted_len, int32_t *out_tokens,
                                    void *workspace, size_t workspace_bytes, void *stream,
                                    void *const *events, int32_t n_events,
                                    int32_t *n_launched);

/* Names of the kernels spec_typical_verify would launch, ';'-separated (static storage). */
const char *sv_typical_launch_plan(int32_t B, int32_t G, int32_t V, sv_dtype dtype,
                                   float temperature, int32_t top_k);

/* Human-readable text of a status (static storage). */
const char *sv_status_string(sv_status status);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
