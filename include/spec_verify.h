/*
 * spec_verify.h -- C ABI of libspec_verify.so: batched target-side verification for
 * exact speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * Four verification rules, each one entry point (the chain and greedy rules also have a
 * *_stop variant that applies stop tokens and an output budget inside the round, and an
 * *_ex variant that adds target logit processors -- bias, grammar mask, top-k, top-p):
 *   spec_verify_chain          rejection-sampling verification of a draft chain
 *   spec_verify_greedy         argmax-match verification of a draft chain
 *   spec_verify_tree           tree verification by target-sample membership (and
 *                              spec_verify_tree_greedy, its temperature-0 form)
 *   spec_verify_tree_residual  multi-candidate tree verification with residual updates
 *
 * Pages that define the operations (cited by title and section):
 *   [M7.1]  "M7.1 - Speculative Decoding: Draft, Verify, Accept, Reject"
 *   [M7.7]  "M7.7 - Draft Sources, Dependent Heads, and Hardware-Aware Trees"
 *   [Atlas] "Speculative decoding: proposals and verified output" (AI-atlas lesson data)
 *   [M16]   "Module 16: Speculative Decoding"
 *   [Tiny]  "Exact Speculative and Assisted Decoding for TinyRustLM"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every array pointer is a DEVICE pointer, owned by the caller, in dense
 *           row-major layout with the vocabulary innermost.  The library never
 *           allocates, never frees and never synchronizes; all work is enqueued on
 *           `stream`, and outputs are valid once that stream reaches the call.
 * Graphs.   A call enqueues kernel launches only (one, or two with top-k / top-p), so
 *           it may be captured in a HIP graph and replayed: each replay reads the
 *           buffers' contents at replay time.  Make one eager call with the same
 *           sizes and dtypes before capturing: the first launch of a kernel
 *           configuration on a device queries its occupancy.
 * Workspace. Each entry point takes a caller-owned device workspace of at least the
 *           size its query function returns, aligned to 256 bytes.  It must be
 *           zero-filled before its first use, and every call leaves it entirely
 *           zero again (the blocks that consume counters and intermediate results
 *           clear them), so one workspace serves any sequence of calls -- any entry
 *           point, any sizes that fit it -- issued in order on one stream.  Calls
 *           that overlap in time must use different workspaces.
 * Host status.  The return value reports only what the host can check before
 *           launching: null pointers, sizes outside the documented limits, a
 *           temperature outside its range, an unknown dtype, a workspace that is too
 *           small or misaligned, and a HIP launch failure.  Sizes are also refused
 *           (SPEC_EINVAL, and a workspace query returns 0) when the launch would need
 *           more than (2^32 - 1) / 256 = 16777215 blocks of 256 threads (a dispatch
 *           counts work-items in 32 bits).  A launch has at least one block per row
 *           (or tree request), so this happens once the rows near 2^24, or once the
 *           logits near 2^40 elements.  On any non-SPEC_OK
 *           return nothing has been enqueued (except SPEC_EHIP, where a launch failed).
 * Request status.  Data errors are reported per request in req_status[b] (SPEC_REQ_*).
 *           A request with a non-zero status emits nothing: accepted_len[b] = -1 and
 *           its out_tokens row is all -1 (the round is aborted without emitting, as
 *           [Tiny] "Normative stochastic pseudocode" does on a NaN row or an empty
 *           residual).  Checks apply to what the round actually reaches, in the
 *           order it reaches it: row i, then draft token i, then q_i(x_i), then
 *           uniform i, for i = 0, 1, ...
 * Uniforms. The caller supplies every random number as fp32 in [0, 1) ([Tiny]
 *           "Normative edge-case behavior": counter-based, per-purpose draws).  Given
 *           the same inputs the outputs are bitwise reproducible.
 * Exactness. Tokens are exact functions of the inputs except for uniforms that fall
 *           within ~1e-6 of an acceptance threshold or of a CDF boundary, where fp32
 *           rounding of the probabilities may decide either way.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 2

/* Limits checked on the host. */
#define SPEC_MAX_BATCH  (1 << 22)   /* B */
#define SPEC_MAX_GAMMA  63          /* gamma: draft tokens per request */
#define SPEC_MAX_VOCAB  (1 << 28)   /* V */
#define SPEC_MAX_NODES  4096        /* N: tree nodes per request */
#define SPEC_MAX_STOP   256         /* n_stop: stop tokens of the *_stop entry points */
#define SPEC_MAX_SPARSE_K 65536     /* q_k: entries of a sparse draft row */
#define SPEC_MIN_TEMPERATURE 0x1p-20f
#define SPEC_MAX_TEMPERATURE 0x1p+20f

typedef enum {
  SPEC_OK = 0,
  SPEC_EINVAL = 1,      /* null pointer, size out of range, bad temperature */
  SPEC_EDTYPE = 2,      /* unknown spec_dtype */
  SPEC_EWORKSPACE = 3,  /* workspace missing, too small or not 256-byte aligned */
  SPEC_EHIP = 4,        /* a kernel launch failed (hipGetLastError) */
  SPEC_ESCRATCH = 5     /* spec_verify_chain_static: the sizes need more than its scratch */
} spec_status;

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

/* Per-request status codes written to req_status[b]. */
enum {
  SPEC_REQ_OK = 0,
  SPEC_REQ_NONFINITE = 1,       /* a reached logits row has NaN or +inf, or is all -inf */
  SPEC_REQ_BADTOKEN = 2,        /* a reached draft token is outside [0, V) */
  SPEC_REQ_BADUNIFORM = 3,      /* a consumed uniform is outside [0, 1) */
  SPEC_REQ_QZERO = 4,           /* q_i(x_i) is not a positive finite number ([M7.1] §0x03D:
                                   a token the draft gives no mass cannot be proposed) */
  SPEC_REQ_RESIDUAL_EMPTY = 5,  /* terminal mass W is not positive and finite, or the q row
                                   read at the rejected position has a negative or
                                   non-finite entry ([Tiny] residual invariant) */
  SPEC_REQ_BADTREE = 6,         /* parents[0] != -1, a parents[v] outside [0, v), or a
                                   non-root node token outside [0, V) ([M7.7] §0x0F) */
  SPEC_REQ_INTERNAL = 7         /* an internal wait between blocks hit its bound (not
                                   expected; the request's outputs are not valid).  A word
                                   published late may be left in the workspace: a chain
                                   call zeroes its failed requests' words itself; a greedy
                                   or tree call marks the workspace dirty (word 0), and
                                   every later call on a dirty workspace, of any entry
                                   point, reports SPEC_REQ_INTERNAL for all its requests
                                   until the caller zero-fills the workspace */
};

/* How a request's round ended (the finish output of the *_stop entry points). */
enum {
  SPEC_FINISH_NONE = 0,     /* the request goes on */
  SPEC_FINISH_STOP = 1,     /* the last emitted token is a stop token */
  SPEC_FINISH_BUDGET = 2    /* the emitted tokens used up the remaining budget (or it was
                               already 0); a stop token wins a tie */
};

/* ------------------------------------------------------------------ chain ---
 * Rejection-sampling verification of B independent draft chains.
 *
 * Defined by [M7.1] §0x03-§0x03H and §0x04 "Loop Pseudocode", [M16] "The Math:
 * Speculative Sampling" and "Code: Verify a Draft", [Atlas] mechanism:
 *   p_i = softmax(l_i / T) for rows i = 0..gamma  (temperature is applied to the
 *         target logits only; q is used exactly as given);
 *   for i = 0..gamma-1: accept x_i iff u_i < a_i = min(1, p_i(x_i) / q_i(x_i));
 *         stop at the first rejection, A = its index (A = gamma if none);
 *   terminal weights w = max(p_A - q_A, 0) if A < gamma ([M7.1] §0x03C), else
 *         w = p_gamma (the bonus row, [M7.1] §0x03H);
 *   terminal token k = first index (vocabulary order) whose running sum of w
 *         exceeds u_gamma * sum(w);
 *   emitted tokens: x_0..x_{A-1}, k  (A + 1 tokens, [M16]).
 *
 * target_logits  [B, gamma+1, V] in logit_dtype.  Row i < gamma scores draft token i;
 *                row gamma is the bonus row ([M7.1] §0x04A, replayed-frontier layout).
 * draft_probs    [B, gamma, V] in q_dtype: the distribution each draft token was drawn
 *                from, after the drafter's processors.  Only q_i(x_i) for reached rows
 *                and the full row q_A of a rejecting request are read.
 * draft_tokens   [B, gamma] int32.
 * uniforms       [B, gamma+1] fp32: u[b, i] for the accept test of draft i, u[b, gamma]
 *                for the single terminal draw (correction or bonus).
 * temperature    in [SPEC_MIN_TEMPERATURE, SPEC_MAX_TEMPERATURE].
 * accepted_len   [B] int32 out: A in [0, gamma], or -1.
 * out_tokens     [B, gamma+1] int32 out: A + 1 tokens, then -1.
 * req_status     [B] int32 out: SPEC_REQ_*.
 * stats          [B, gamma+1, 4] fp32 out, may be NULL.  For each reached row i < gamma:
 *                (m_i, log Z_i, p_i(x_i), a_i), with m_i = max_x l_{i,x} / T and
 *                Z_i = sum_x exp(l_{i,x} / T - m_i).  Row gamma: (m_gamma, log Z_gamma)
 *                when the bonus row is reached, W = sum(w) in column 2, NaN in column 3.
 *                Every other entry (and every entry of a failed request) is NaN.
 * gamma may be 0 (a plain target draw from row 0); then draft_probs and draft_tokens
 * may be NULL.  B may be 0 (nothing is enqueued).
 */
size_t spec_chain_workspace_bytes(int B, int gamma, int V);

spec_status spec_verify_chain(const void* target_logits, int logit_dtype,
                              const void* draft_probs, int q_dtype,
                              const int32_t* draft_tokens, const float* uniforms,
                              int B, int gamma, int V, float temperature,
                              int32_t* accepted_len, int32_t* out_tokens, int32_t* req_status,
                              float* stats, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): spec_verify_chain with the same
 * arguments, results and errors, minus the workspace, which it takes from a device array
 * of SPEC_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on until the
 * process ends.  It calls no allocating routine.  Sizes whose spec_chain_workspace_bytes
 * exceeds SPEC_STATIC_SCRATCH_BYTES return SPEC_ESCRATCH; invalid sizes SPEC_EINVAL.  Each
 * call first zero-fills the part of the array it uses (a kernel on `stream`), so a failed
 * call leaves nothing behind.  All calls on one GPU share its array: calls that may overlap
 * on one GPU (different streams without ordering) race and must not be issued. */
#define SPEC_STATIC_SCRATCH_BYTES (4u << 20)
spec_status spec_verify_chain_static(const void* target_logits, int logit_dtype,
                                     const void* draft_probs, int q_dtype,
                                     const int32_t* draft_tokens, const float* uniforms,
                                     int B, int gamma, int V, float temperature,
                                     int32_t* accepted_len, int32_t* out_tokens,
                                     int32_t* req_status, float* stats, hipStream_t stream);

/* Chain verification with stop tokens and an output budget ([M7.1] §0x05B "Round
 * Progress Includes Correction Or Bonus": progress is min(A + 1, H), H the distance to
 * the first emitted stop token or the remaining budget; §0x06 "KV Commit And Rollback":
 * stopping is applied before anything is published; [Tiny] "Normative stochastic
 * pseudocode"):
 *   budget[b] <= 0: no round -- nothing is read or checked, nothing is emitted,
 *         accepted_len 0, finish SPEC_FINISH_BUDGET;
 *   otherwise the tests run as in spec_verify_chain, and an ACCEPTED draft x_i that is a
 *         stop token, or with i + 1 == budget[b], ends the round after itself: the
 *         emitted tokens are x_0..x_i (accepted_len = i + 1), no terminal token is drawn,
 *         and nothing after draft i is read or checked (row gamma and u_gamma included);
 *   otherwise the terminal token is emitted as usual, and finish reports whether it is a
 *         stop token, or whether A + 1 == budget[b].
 * stop_tokens  [n_stop] int32 device array, 0 <= n_stop <= SPEC_MAX_STOP (may be NULL
 *              when n_stop = 0); an entry outside [0, V) never matches.
 * budget       [B] int32 device array of remaining output budgets, or NULL (no limit).
 * finish       [B] int32 out (SPEC_FINISH_*; 0 for a failed request), or NULL.
 * stats        rows tested by a round that ended on a draft keep their statistics; the
 *              bonus row and W stay NaN.
 * Every other argument is as for spec_verify_chain, whose workspace it uses; with
 * n_stop = 0 and budget = NULL the outputs are those of spec_verify_chain.
 */
spec_status spec_verify_chain_stop(const void* target_logits, int logit_dtype,
                                   const void* draft_probs, int q_dtype,
                                   const int32_t* draft_tokens, const float* uniforms,
                                   int B, int gamma, int V, float temperature,
                                   const int32_t* stop_tokens, int n_stop, const int32_t* budget,
                                   int32_t* accepted_len, int32_t* out_tokens, int32_t* req_status,
                                   int32_t* finish, float* stats, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* Options of spec_verify_chain_ex and spec_verify_greedy_ex: stop tokens, an output
 * budget, and target logit processors.  Every pointer is a device pointer or NULL (that
 * option off); a zero-initialized struct (or a NULL options pointer) gives the plain call.
 *
 * Processors ([M7.1] §0x06J: the verified p_i is the processed row, not the raw softmax;
 * §0x04G: ordered temperature and additive-bias processors; [Tiny] "Grammar and
 * deterministic opportunities": a grammar mask renormalizes over the valid tokens):
 *   s_x = l_x + bias_x in fp32;  p is proportional to exp(s_x / T) over the kept tokens;
 *   a token is kept when it is allowed, and s_x is at least the k-th largest allowed s
 *   (top-k, ties kept), and the probability mass (over the tokens left so far) of the tokens
 *   with strictly larger s is below top_p (top-p: the smallest tie-closed set of top tokens
 *   whose mass reaches top_p).  NaN or +inf in l + bias anywhere in a reached row makes the
 *   request SPEC_REQ_NONFINITE, masked or not; so does a reached row with no kept token.
 *   Sparse draft rows ([Tiny] "Logit and residual scratch": exact only when the omitted
 *   proposal probabilities are known to be zero): q_i(x) is the sum of the values listed at
 *   index x (0 if none); the residual uses the row densified the same way.  An entry whose
 *   index is outside [0, V), or whose value is negative or not finite, makes the row
 *   invalid when it is read as a whole (SPEC_REQ_RESIDUAL_EMPTY at a rejection there).
 *   Top-k and top-p run a threshold pass over every row first (a second launch, about 17
 *   reads of each row from cache); bias and the mask are applied where the verifier reads
 *   logits, at no extra pass.  The greedy verifier applies bias and the mask (truncations
 *   never move the argmax) and ignores top_k and top_p.
 * Lazy rows ([M7.1] §0x03G: the round stops at the first rejection, and every later row
 * is discarded): with lazy_rows = k >= 1, rows 0..k-1 of every request are read (none when
 * the budget is 0), and rows jk..jk+k-1 (j >= 1) only when drafts 0..jk-1 were all
 * accepted without a stop or budget end (greedy: matched the target argmax).  The outputs
 * equal those of lazy_rows = 0 (statistics are only reported for reached rows either way);
 * fewer bytes are read when rejections come early, at the cost of one dependent wait per
 * group.  Negative values are SPEC_EINVAL; k >= gamma + 1 is one group (every row).
 */
typedef struct {
  const int32_t* stop_tokens;   /* [n_stop] stop tokens (as for spec_verify_chain_stop) */
  int32_t n_stop;               /* 0 .. SPEC_MAX_STOP */
  const int32_t* budget;        /* [B] remaining output budgets */
  int32_t* finish;              /* [B] out: SPEC_FINISH_* */
  const float* bias;            /* [V] additive logit bias, fp32 */
  const uint32_t* allowed;      /* [B, gamma+1, ceil(V/32)] allowed-token bitmask of each
                                   row: bit x % 32 of word x / 32 set = token x allowed */
  const int32_t* top_k;         /* [B] top-k per request; 0 (or negative): off */
  const float* top_p;           /* [B] top-p per request; outside (0, 1): off */
  const int32_t* q_index;       /* chain only: [B, gamma, q_k] token indices of sparse draft
                                   rows; draft_probs then holds [B, gamma, q_k] fp32 values
                                   (q_dtype SPEC_F32) and every token not listed has q = 0 */
  int32_t q_k;                  /* 1 .. SPEC_MAX_SPARSE_K when q_index is given */
  int32_t lazy_rows;            /* 0 reads every row; k >= 1 reads the rows in groups of
                                   k, a group only when every draft before it was
                                   accepted (see above) */
} spec_verify_options;

/* Chain verification with options (spec_verify_options); every other argument and the
 * workspace are those of spec_verify_chain, whose outputs it gives for opt = NULL. */
spec_status spec_verify_chain_ex(const void* target_logits, int logit_dtype,
                                 const void* draft_probs, int q_dtype,
                                 const int32_t* draft_tokens, const float* uniforms,
                                 int B, int gamma, int V, float temperature,
                                 const spec_verify_options* opt,
                                 int32_t* accepted_len, int32_t* out_tokens, int32_t* req_status,
                                 float* stats, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* ----------------------------------------------------------------- greedy ---
 * Argmax-match verification ([M7.1] §0x02D: longest-prefix validation is exact for
 * greedy decoding; [Tiny] "Normative greedy pseudocode"):
 *   t_i = argmax_x l_{i,x}, lowest index on ties;  A = first i < gamma with x_i != t_i,
 *   else gamma;  emitted tokens x_0..x_{A-1}, t_A.
 * target_logits [B, gamma+1, V]; draft_tokens [B, gamma]; outputs as for the chain.
 * No temperature: a positive temperature does not move an argmax.
 */
size_t spec_greedy_workspace_bytes(int B, int gamma, int V);

spec_status spec_verify_greedy(const void* target_logits, int logit_dtype,
                               const int32_t* draft_tokens, int B, int gamma, int V,
                               int32_t* accepted_len, int32_t* out_tokens, int32_t* req_status,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Greedy verification with stop tokens and an output budget ([Tiny] "Normative greedy
 * pseudocode": a matching draft that is an active stop token, or that uses up the
 * remaining budget, ends the round after itself; a budget of 0 emits nothing).  The
 * rules, stop_tokens, budget and finish are those of spec_verify_chain_stop; the
 * workspace is that of spec_verify_greedy.
 */
spec_status spec_verify_greedy_stop(const void* target_logits, int logit_dtype,
                                    const int32_t* draft_tokens, int B, int gamma, int V,
                                    const int32_t* stop_tokens, int n_stop, const int32_t* budget,
                                    int32_t* accepted_len, int32_t* out_tokens, int32_t* req_status,
                                    int32_t* finish, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Greedy verification with options (stop tokens, budget, bias and mask, lazy rows; top_k,
 * top_p and q_index are ignored); the workspace is that of spec_verify_greedy. */
spec_status spec_verify_greedy_ex(const void* target_logits, int logit_dtype,
                                  const int32_t* draft_tokens, int B, int gamma, int V,
                                  const spec_verify_options* opt,
                                  int32_t* accepted_len, int32_t* out_tokens, int32_t* req_status,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------- tree ---
 * Tree verification by target-sample membership ([M7.7] §0x04B and §0x09: accept a
 * candidate child when it equals the token the target samples; [M16] "Verify the
 * Tree": walk down from the root until no child matches, then emit one target token).
 *   v = 0 (the frontier root);
 *   repeat: y = inverse-CDF draw of softmax(l_v / T) with u[b, v];
 *           if a child c of v (parents[c] == v) has node_tokens[c] == y (the lowest
 *           such c if siblings repeat a token): accept c, v = c;  else stop.
 *   emitted tokens: tokens of the accepted nodes, then the last draw y.
 * Row v of node_logits scores the children of node v ([M7.7] §0x07E: a node's row
 * predicts its children, never itself).  Only rows on the walked path are read.
 *
 * node_logits   [B, N, V]; node_tokens [B, N] int32 (node 0's entry is ignored);
 * parents       [B, N] int32 with parents[0] = -1 and 0 <= parents[v] < v;
 * uniforms      [B, N] fp32, u[b, v] used for the draw at node v;
 * accepted_len  [B]: number of accepted non-root nodes (path length), or -1;
 * out_tokens    [B, N]: accepted_len + 1 tokens, then -1;
 * out_nodes     [B, N]: the accepted node ids in path order, then -1.
 */
size_t spec_tree_workspace_bytes(int B, int N, int V);

spec_status spec_verify_tree(const void* node_logits, int logit_dtype,
                             const int32_t* node_tokens, const int32_t* parents,
                             const float* uniforms, int B, int N, int V, float temperature,
                             int32_t* accepted_len, int32_t* out_tokens, int32_t* out_nodes,
                             int32_t* req_status, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Greedy tree verification, the temperature-0 form of spec_verify_tree ([M16] "Verify the
 * Tree -- and Why It's Exact": follow the child whose token is the target's greedy next
 * token; the output equals plain greedy decoding of the target):
 *   y = argmax_x l_{v,x} (lowest index on ties) in place of the draw; the walk, the
 *   outputs and the workspace (spec_tree_workspace_bytes) are those of spec_verify_tree.
 * No uniforms and no temperature.  Request statuses: SPEC_REQ_BADTREE, then
 * SPEC_REQ_NONFINITE for a reached row holding NaN or +inf, or entirely -inf.
 */
spec_status spec_verify_tree_greedy(const void* node_logits, int logit_dtype,
                                    const int32_t* node_tokens, const int32_t* parents,
                                    int B, int N, int V,
                                    int32_t* accepted_len, int32_t* out_tokens, int32_t* out_nodes,
                                    int32_t* req_status, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* -------------------------------------------------------- residual tree ---
 * Multi-candidate tree verification with residual updates ([M7.7] §0x09A, "Stochastic
 * residual update"; §0x08B: testing every candidate against the original target would
 * duplicate mass).  Same tree layout as spec_verify_tree (node 0 = frontier root, row v of
 * node_logits scores v's children), plus the proposal distribution of every node:
 *   v = 0;
 *   repeat: res = softmax(l_v / T);
 *           for each child c of v in increasing index order (token x_c, drawn from q_c):
 *               accept c iff u_acc[b, c] < min(1, res(x_c) / q_c(x_c)): emit x_c, v = c,
 *               and continue the walk from c;
 *               else res = [res - q_c]_+ / sum([res - q_c]_+);
 *           no child accepted (or no children): emit the inverse-CDF draw of res with
 *           u_draw[b, v] (vocabulary order, as spec_verify_chain) and stop.
 * The emitted sequence follows the target's own law for any proposals ([M7.7] §0x09A).
 *
 * node_logits   [B, N, V] logit_dtype; draft_probs [B, N, V] q_dtype: row c (c >= 1) is the
 *               distribution node c's token was drawn from (row 0 is not read; siblings
 *               drawn i.i.d. repeat one row).  Only q_c(x_c) of tested children and the
 *               full rows of rejected children are read.
 * node_tokens, parents [B, N] int32 as for spec_verify_tree.
 * accept_uniforms [B, N] fp32 (entry c for the test of child c; entry 0 is not read);
 * draw_uniforms   [B, N] fp32 (entry v for the terminal draw at node v).
 * Outputs as for spec_verify_tree.  Statuses: SPEC_REQ_BADTREE (checked first), then in
 * reached order SPEC_REQ_NONFINITE (a row), SPEC_REQ_QZERO (q_c(x_c) not positive and
 * finite), SPEC_REQ_BADUNIFORM, SPEC_REQ_RESIDUAL_EMPTY (a rejected child's q row has a
 * negative or non-finite entry, or the residual has no mass).
 * V is limited to 2^21 here (a row's 2048-element chunk masses are staged on chip).
 */
size_t spec_tree_residual_workspace_bytes(int B, int N, int V);

spec_status spec_verify_tree_residual(const void* node_logits, int logit_dtype,
                                      const void* draft_probs, int q_dtype,
                                      const int32_t* node_tokens, const int32_t* parents,
                                      const float* accept_uniforms, const float* draw_uniforms,
                                      int B, int N, int V, float temperature,
                                      int32_t* accepted_len, int32_t* out_tokens, int32_t* out_nodes,
                                      int32_t* req_status, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* ------------------------------------------------------------------ misc --- */
const char* spec_status_string(int code);     /* static string, never NULL */
const char* spec_req_status_string(int code); /* static string, never NULL */
int spec_abi_version(void);                   /* SPEC_ABI_VERSION */

/* Timeline trace, for profiling (not for the calls' results).  In a library built with
 * tracing (python -m exact_rejection_sampling_amd.build --trace, which writes
 * libspec_verify_trace.so), every later call records, for each block of its kernels, a tag
 * and stamps of the GPU's 100 MHz real-time counter into `buffer`: a device allocation of
 * 5 * records_per_kernel * 16 uint64 words, which the caller owns and keeps alive while traced
 * calls run; block x of kernel slot k (0 chain, 1 chain exact redraw, 2 tree, 3 residual tree,
 * 4 the top-k / top-p threshold pass)
 * writes words [(k * records_per_kernel + x) * 16, + 16) with plain stores on the call's stream,
 * and blocks at or past records_per_kernel write nothing.  buffer == NULL turns tracing off.
 * Returns SPEC_EINVAL in a library built without tracing, or for a non-null buffer with
 * records_per_kernel == 0.  Not thread-safe: set it while no call is being issued. */
spec_status spec_trace_set(void* buffer, size_t records_per_kernel);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
