/*
 * libspecverify: batched speculative-sampling verifier for MI355X (gfx950).
 *
 * The operation is the verification half of one speculative-decoding round
 * (page "초안 모델로 생성 속도를 높이는 추측 디코딩", section "방법",
 * Algorithm 1; page "vLLM speculative decoding이 기각 토큰을 다시 뽑는 이유",
 * section "드래프트가 제안하고 타깃이 판정한다").  For each request b the
 * target model scored G+1 positions and the drafter proposed G tokens x_j:
 *
 *   p_j = softmax(topk(target_logits[b, j, :] / T))   j = 0..G
 *   q_j = softmax(topk(draft_logits[b, j, :] / T))    j = 0..G-1
 *   accept x_j iff u_j <= p_j(x_j) / q_j(x_j)          (q_j(x_j) > 0)
 *   n   = first rejected position, or G
 *   out[0..n-1] = x_0..x_{n-1}
 *   out[n]      = a draw from norm(max(0, p_n - q_n))  if n < G (recovered)
 *               = a draw from p_G                     if n = G (bonus)
 *   out[n+1..G] = -1
 *
 * The recovered/bonus draw is the Exp(1) race argmax_y w_y / E_y (page on
 * vLLM's kernel, section "vLLM 커널은 이 규칙을 어떻게 옮겼나"), so the
 * residual is never normalised.  Temperature and top-k are applied to the
 * logits first, to p and to q alike (same section: p is the adjusted law).
 *
 * Random numbers: a counter-based Philox4x32-10 keyed by sv_params.seed.
 * The accept uniform of (b, j) comes from counter (0, j, b, 0), words 0 and
 * 1; the race uniform of token y at position j from counter (y>>1, j, b, 1),
 * words (0,1) for even y and (2,3) for odd y.  Two words (lo, hi) map to
 * u = ((hi:lo >> 11) + 1) * 2^-53 in (0, 1], in fp64, so u is never 0.
 * E = -ln(u).  Results are a pure function of the inputs and the seed.
 *
 * Ties: every argmax (greedy target token, race winner) goes to the lowest
 * index; top-k keeps exactly k tokens ranked by (logit desc, index asc).
 *
 * Conventions shared by every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller; the
 *    library never allocates or frees device memory.  Rows are contiguous
 *    (row stride = vocab); logits are fp32 or bf16 (sv_params.dtype), aligned
 *    to their element size.
 *  - workspace: caller-owned device scratch of at least
 *    sv_workspace_bytes(params) bytes, 256-byte aligned.  Its contents on
 *    entry are ignored; calls that share a workspace must not overlap.
 *  - stream: a hipStream_t passed as void* (NULL = the default stream).  Calls
 *    only enqueue work: there is no host synchronisation and no readback.
 *  - Argument errors and launch errors are returned synchronously as an
 *    sv_status; nothing is enqueued after an argument error.
 *  - A draft token outside [0, vocab) is treated as rejected at its
 *    position (q(x) := 0, a greedy mismatch) and sets a sticky code in the
 *    workspace that sv_read_device_error reports.
 *  - A row whose logits are all -inf, or that holds NaN or +inf, has no
 *    defined law: results for it are unspecified (no fault).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_ERR_INVALID_ARG = 1,  /* bad size, temperature, top_k or null pointer */
  SV_ERR_DTYPE = 2,        /* dtype not SV_F32 / SV_BF16, or misaligned logits */
  SV_ERR_WORKSPACE = 3,    /* workspace null, misaligned or too small */
  SV_ERR_HIP = 4,          /* a HIP runtime call or kernel launch failed */
  SV_ERR_UNSUPPORTED = 5,  /* gamma > 16384; spec_verify_prob_noalloc: top_k > 1024 */
  SV_ERR_SCRATCH = 6       /* spec_verify_prob_noalloc: the call needs more than
                              SV_NOALLOC_SCRATCH_BYTES of device scratch */
} sv_status;

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

typedef struct {
  int32_t batch;       /* B >= 1 requests */
  int32_t gamma;       /* 1 <= G <= 16384 draft positions per request */
  int32_t vocab;       /* V >= 1 */
  int32_t dtype;       /* sv_dtype of every logit array */
  float temperature;   /* T > 0 (finite) for prob/onehot; ignored by greedy */
  int32_t top_k;       /* 0 or >= vocab: off; else keep exactly k tokens.  k <= 1024:
                          kept as candidates in one read of each row; larger k:
                          a cut at the k-th key of each full row (a radix select,
                          two to six more reads of the rows of such requests) */
  uint64_t seed;       /* Philox key */
} sv_params;

/* Bytes of workspace any entry point needs for these parameters (0 if the
 * parameters are invalid). */
size_t sv_workspace_bytes(const sv_params* params);

/* Static, human-readable text of a status code. */
const char* sv_status_string(sv_status status);

/* Probabilistic draft ("probabilistic" draft sampling on the vLLM page,
 * section "기본값 greedy 드래프트에서도 분포가 지켜질까"; the residual rule
 * of section "왜 하필 max(p − q, 0)인가").
 *   target_logits [B][G+1][V], draft_logits [B][G][V], draft_tokens [B][G]
 *   out_tokens [B][G+1] (-1 after the emitted token), num_accepted [B] = n
 *   p_draft, q_draft [B][G]: p_j(x_j), q_j(x_j) for every j (may be NULL). */
sv_status spec_verify_prob(const sv_params* params, const void* target_logits, const void* draft_logits,
                           const int32_t* draft_tokens, int32_t* out_tokens, int32_t* num_accepted,
                           float* p_draft, float* q_draft, void* workspace, size_t workspace_bytes,
                           void* stream);

/* One-hot draft (a greedy drafter, vLLM's default; same page, section
 * "기본값 greedy 드래프트에서도 분포가 지켜질까"): q(x) = 1, accept iff
 * u <= p(x), the residual is p with x masked.  Arguments as spec_verify_prob
 * without draft logits; p_draft [B][G] may be NULL. */
sv_status spec_verify_onehot(const sv_params* params, const void* target_logits, const int32_t* draft_tokens,
                             int32_t* out_tokens, int32_t* num_accepted, float* p_draft, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Temperature 0 (page "초안 모델로 생성 속도를 높이는 추측 디코딩", section
 * "방법": at T = 0 a draft token is accepted only if it is the target's
 * argmax; the vLLM page's greedy kernel).  Accept iff x_j == argmax_y
 * target_logits[b, j, y]; the target argmax replaces the first mismatch and
 * is the bonus after G matches.  temperature and top_k are ignored; seed is
 * unused.  target_argmax [B][G+1] may be NULL. */
sv_status spec_verify_greedy(const sv_params* params, const void* target_logits, const int32_t* draft_tokens,
                             int32_t* out_tokens, int32_t* num_accepted, int32_t* target_argmax,
                             void* workspace, size_t workspace_bytes, void* stream);

/* spec_verify_prob for callers that cannot allocate device memory or pass a
 * workspace: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and Philox
 * streams as spec_verify_prob (bit-identical outputs), with the library's
 * own device scratch in place of `workspace`: a static device array of
 * SV_NOALLOC_SCRATCH_BYTES in the library's code object, one per GPU, held
 * until the process ends.  Its address is looked up on the first call on
 * each device; no call allocates or frees anything.
 *   error_word: DEVICE int32 (may be NULL) that receives the call's error
 *     word, bits as sv_read_device_error.
 * Limits: the call must need at most SV_NOALLOC_SCRATCH_BYTES of scratch
 * (sv_workspace_bytes(params) bytes; the B=1024, gamma=8, V=256000 top-64
 * call needs about 9 MB), else SV_ERR_SCRATCH; a top_k above 1024 (below
 * vocab) returns SV_ERR_UNSUPPORTED.  Nothing is enqueued after an error.
 * Every call on one GPU uses that GPU's single scratch array: calls that
 * overlap on one GPU (different streams, or host threads) race and must be
 * ordered by the caller.  The kernels clear what must start at zero, so the
 * array's contents left by an earlier call do not matter. */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
sv_status spec_verify_prob_noalloc(const sv_params* params, const void* target_logits, const void* draft_logits,
                                   const int32_t* draft_tokens, int32_t* out_tokens, int32_t* num_accepted,
                                   float* p_draft, float* q_draft, int32_t* error_word, void* stream);

/* Form of the draft in spec_verify_batch. */
typedef enum {
  SV_DRAFT_LOGITS = 0, /* draft logits, same dtype and rules as the target's */
  SV_DRAFT_ONEHOT = 1, /* no draft rows: a greedy drafter, q one-hot at x_j */
  SV_DRAFT_PROBS = 2,  /* fp32 draft probabilities q, used as given (vLLM's
                          "probabilistic" draft_probs): no temperature, top-k,
                          top-p or renormalisation is applied to them */
  SV_DRAFT_MATCH = 3   /* token-only drafts (prompt lookup, n-grams, tree
                          drafts) verified by sampler-match (page "투기적
                          디코딩" (mlxcel manual), section "mlxcel의 프롬프트
                          조회"): see spec_verify_batch */
} sv_draft_kind;

/* Where the rows of a spec_verify_batch call live.  Strides are in elements
 * (0 = vocab; otherwise >= vocab, e.g. a vocabulary padded for the LM head).
 * cu_draft (DEVICE array [B+1], may be NULL): request b owns draft positions
 * cu_draft[b] .. cu_draft[b+1]-1, g_b of them, 0 <= g_b <= gamma, with
 * cu_draft[0] = 0 (vLLM's cu_num_draft_tokens).  Rows are then packed:
 * request b's g_b + 1 target rows start at row cu_draft[b] + b; its g_b
 * draft rows, draft tokens and p_draft / q_draft entries at cu_draft[b].
 * out_tokens stays [B][gamma+1].  With cu_draft NULL every request has gamma
 * positions, rows [B][gamma+1] and [B][gamma].  A cu_draft array that breaks
 * these rules makes every request invalid: out_tokens -1, num_accepted 0,
 * p_draft / q_draft not written; the sticky error word gets bit 2 (value 4).
 * A ragged call whose every draft length is 0 (cu_draft[B] = 0) has no draft
 * tokens or draft rows: draft_tokens and draft may then be NULL (if they are
 * NULL and cu_draft[B] != 0, the layout is invalid as above). */
typedef struct {
  int32_t draft_kind;      /* sv_draft_kind */
  int32_t reserved;        /* 0 */
  int64_t target_stride;
  int64_t draft_stride;
  const int32_t* cu_draft;
  const int32_t* parents;  /* SV_DRAFT_MATCH only (may be NULL: chains): DEVICE
                              array laid out like draft_tokens; the draft token
                              of position j is node j + 1 of a tree whose root
                              (node 0) is the last context token, and
                              parents[.] of node i is its parent node, in
                              0..i-1.  Target row i is the law after node i's
                              path.  A request whose parents break this rule
                              emits nothing; the sticky error word gets bit 1
                              (value 2). */
} sv_layout;

/* Per-request sampling settings of spec_verify_batch: DEVICE arrays of
 * length batch, owned by the caller and read by the kernels (the host never
 * reads them).  The adjusted laws are temperature, then top-k, then top-p,
 * applied alike to p and q (page "vLLM speculative decoding이 기각 토큰을 다시
 * 뽑는 이유", section "vLLM 커널은 이 규칙을 어떻게 옮겼나": temperature,
 * top_k and top_p are applied before the test, in that order).
 *   temperature[b]  T_b >= 0, finite.  T_b == 0: a greedy request, decided by
 *                   argmax matching (section "기본값 greedy 드래프트에서도
 *                   분포가 지켜질까"); its top_k and top_p are ignored.
 *   top_k[b]        0 or >= vocab: off; else 1..max_top_k.  NULL: all off.
 *   top_p[b]        in (0, 1]; 1: off.  The nucleus is the shortest prefix,
 *                   in (logit desc, index asc) order, of the law left by
 *                   top-k whose probability reaches top_p (at least one
 *                   token); the law is renormalised over it.  NULL: all off.
 *   max_top_k       host-side bound, >= 0: every top_k[b] below vocab is at
 *                   most this (it sizes the workspace and the kernels).  A
 *                   top_k[b] up to min(max_top_k, 1024) is kept as candidates;
 *                   a larger one is a cut at the k-th key of each full row.
 * A request whose settings break these rules (T negative, NaN or infinite;
 * top_k negative or in (max_top_k, vocab); top_p NaN, <= 0 or > 1) emits
 * nothing: out_tokens all -1, num_accepted 0, p_draft and q_draft 0; the
 * sticky error word gets bit 1 (value 2).  Other requests are unaffected. */
typedef struct {
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  int32_t max_top_k;
  int32_t reserved; /* 0 */
} sv_sampling;

/* Outputs of spec_verify_batch (DEVICE arrays owned by the caller).
 *   out_tokens [B][G+1], num_accepted [B]: required, as spec_verify_prob.
 *   p_draft, q_draft: p_j(x_j), q_j(x_j) per draft position (laid out like
 *     draft_tokens); may be NULL.
 *   beta: per draft position, sum_y min(p_j(y), q_j(y)), the probability
 *     that position j's draft is accepted (page "초안 모델로 생성 속도를
 *     높이는 추측 디코딩", section "수락률 α와 기대 속도 향상": alpha is its
 *     expectation, Theorem 3.5); p_j(x_j) for one-hot drafts, 1 or 0 (argmax
 *     match) for greedy requests; laid out like draft_tokens; may be NULL.
 *     0 for requests that are not verified.  For requests without top-k and
 *     with draft logits or probabilities it costs one more read of their
 *     target and draft rows.
 *   counters [B][3] int64: per request, += (draft positions verified, drafts
 *     accepted, 1) on every call that verifies it (the manual page's
 *     draft_n, draft_n_accepted, draft_rounds: the mean accepted length is
 *     counters[b][1] / counters[b][2]); never cleared by the library; may be
 *     NULL.  Requests that are not verified (invalid) are not counted. */
typedef struct {
  int32_t* out_tokens;
  int32_t* num_accepted;
  float* p_draft;
  float* q_draft;
  float* beta;
  int64_t* counters;
  int32_t* path_nodes;  /* SV_DRAFT_MATCH: [B][G+1], the accepted nodes in order,
                           -1 after; may be NULL */
} sv_outputs;

/* Workspace bytes of spec_verify_batch for these parameters (0 if invalid).
 * With sampling != NULL, params->temperature and params->top_k are not
 * used. */
size_t sv_workspace_bytes_batch(const sv_params* params, const sv_sampling* sampling);

/* Verification with per-request settings: greedy, top-k, top-p and plain
 * requests mixed in one call (vLLM's rejection sampler takes such a batch,
 * same section), any draft form, dense or ragged rows.  Sampled requests
 * follow spec_verify_prob (draft logits), spec_verify_onehot (no draft rows)
 * or, with draft probabilities, the same test and residual with q as given,
 * each with its own T, top-k and top-p on the target (and on draft logits);
 * they draw from the same Philox streams (keyed by params->seed and the
 * request's (b, j)): a dense batch whose requests all share one setting
 * gives bit-identical results to the single-setting entry point.  Greedy
 * requests follow spec_verify_greedy; for them p_draft is the temperature-0
 * law (1 if x_j is the target argmax, else 0) and q_draft = 1.  Draft rows
 * of greedy requests are not read.  q_draft is 1 for valid one-hot drafts.
 *   params: batch, gamma (the largest draft length), vocab, dtype, seed;
 *           with sampling == NULL also the one temperature (0: greedy) and
 *           top_k of every request (top-p off)
 *   sampling: per-request settings, or NULL
 *   layout: draft form, strides, ragged offsets; NULL = dense rows with
 *           draft logits if `draft` is not NULL, else one-hot drafts
 *   target_logits, draft (logits or fp32 probabilities; NULL for one-hot),
 *   draft_tokens: as described by layout;
 *   outputs: see sv_outputs.
 * Sampler-match (layout->draft_kind SV_DRAFT_MATCH): every node gets a fresh
 * sample from its row's adjusted law (temperature 0: the argmax), drawn by
 * the Exp(1) race over the law's kept tokens on the race stream of (request,
 * node): the draw of the recovered and bonus tokens, with the node in place
 * of the position.  From the root the walk follows
 * the child whose token equals the sample (the lowest-indexed one if several
 * do) and emits the sample where no child matches: out_tokens holds the
 * accepted tokens and that sample, num_accepted the accepted depth.  Lossless
 * for token-only proposals.  p_draft of node i is p_parent(x_i), its
 * acceptance probability once its parent is reached (also beta); q_draft is
 * 1 for valid tokens.
 * Workspace: sv_workspace_bytes_batch(params, sampling) bytes.
 * Streams: the row passes of the different kinds of request run side by
 * side.  The call records an event on `stream`, the top-k rows and the
 * temperature-0 rows are streamed on two library-owned streams of the current
 * device that wait for it (created on the first batch call on that device
 * that is not being captured into a graph, non-blocking, default priority,
 * kept until the process ends; until then the row passes run on `stream`
 * one after another), and `stream` waits for both at the end of the call
 * (sampler-match calls, and calls while kernel timing is enabled, before
 * their accept passes): stream order is unchanged, and a capture of
 * `stream` takes the two streams in.  Calls from several host threads are
 * serialised while they enqueue this fork and join. */
sv_status spec_verify_batch(const sv_params* params, const sv_sampling* sampling, const sv_layout* layout,
                            const void* target_logits, const void* draft, const int32_t* draft_tokens,
                            const sv_outputs* outputs, void* workspace, size_t workspace_bytes, void* stream);

/* Synchronises `stream`, then copies the sticky device error word of the
 * last call that used `workspace` to *host_code: bit 0 (value 1) = a draft
 * token was out of range; bit 1 (value 2) = a request of spec_verify_batch
 * had invalid settings or tree parents; bit 2 (value 4) = its cu_draft array
 * broke the layout rules. */
sv_status sv_read_device_error(const void* workspace, int32_t* host_code, void* stream);

/* Per-kernel timing for measurement.  While enabled, every launch of the
 * library is bracketed by a pair of HIP events on the caller's stream (in a
 * spec_verify_batch call the row passes are bracketed as one span, from the
 * fork to the join);
 * sv_kernel_timing_read synchronises on the recorded events and returns the
 * summed device time (ms) and launch count of one kernel family:
 *   0 = row pass (softmax / top-k / argmax over every logit row),
 *   1 = per-request accept + scan (+ race over top-k candidates),
 *   2 = residual / bonus race over a full row.
 * Process-global; not thread-safe; at most 65536 launches per family are
 * recorded between resets. */
sv_status sv_kernel_timing_enable(int enable);
sv_status sv_kernel_timing_reset(void);
sv_status sv_kernel_timing_read(int family, double* total_ms, int64_t* launches);

/* Measurement only: enqueues one read of `bytes` (a multiple of 16) of the
 * DEVICE buffer `buf` (16-byte aligned), with the 16-byte nontemporal loads
 * of the row passes and nothing else, one workgroup per 512 KB: the
 * streaming-read ceiling the row passes' bandwidth is compared with.  `sink`
 * (DEVICE, 256 uint32, 4-byte aligned) is written only by a data-dependent
 * test that keeps the loads alive.  Asynchronous on `stream`. */
sv_status sv_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
