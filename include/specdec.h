/*
 * specdec.h -- C ABI of the MI355X (gfx950) batched speculative-decoding verify step.
 *
 * The operation (one "round" per sequence) is the draft-then-verify rule that all three
 * source pages state:
 *   - "Decodificação especulativa explicada: rascunhe barato, verifique numa passada"
 *     (gsantana.dev), sections "O ciclo de rascunho e verificação" and
 *     "A regra de amostragem por rejeição";
 *   - "ch15 · Speculative Decoding" (snowch.github.io, LLM serving from scratch), section
 *     "Why the result is exactly the target model" (its accept_sampled interface:
 *     target logits, draft probabilities, proposed ids, sampling parameters, a random
 *     generator -> emitted tokens and the number accepted);
 *   - "Speculative decoding: el secretario que adelanta lo que va a decir el jefe"
 *     (blog.lo0.es), section "El mecanismo desnudo", step 3.
 *
 * For sequence b with k = k_b drafts x_0..x_{k-1}, target logit rows z_0..z_k and drafter
 * distributions q_0..q_{k-1}:
 *   p_i = softmax(z_i / T_b)                       (T_b = 0: greedy, p_i = point mass on argmax)
 *   for i = 0..k-1, left to right:
 *     accept x_i  iff  u[b,i] * q_i(x_i) < p_i(x_i)          (probability min(1, p/q))
 *     on the first rejection: emit y ~ norm(max(0, p_i - q_i)) drawn with u[b,K]; stop
 *   if all k are accepted: emit a bonus y ~ p_k drawn with u[b,K]
 *   accept_len[b] = number of accepted drafts A in [0, k]; the round emits A + 1 tokens.
 * Greedy rows accept x_i iff x_i is the lowest-index argmax of z_i and emit that argmax at
 * the first mismatch (or as the bonus).  Sampling is inverse-CDF over ascending token id:
 * the first token whose running weight sum exceeds u times the total.  One-hot rows
 * (n-gram / prompt-lookup drafters, q_i = onehot(x_i)) accept iff u < p_i(x_i) and redraw
 * from p_i with x_i removed.  A rejection whose residual max(0, p_i - q_i) has no mass (only
 * possible when q_i is not a probability distribution) draws from p_i itself.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is DEVICE memory on the current HIP device, except where
 *     noted.  The caller owns every buffer; the library allocates nothing, keeps no
 *     per-call state and never synchronises: work is enqueued on `stream` (a hipStream_t;
 *     NULL = the default stream) and the call returns immediately.
 *   - Layouts are dense row-major, innermost dimension contiguous.
 *   - The returned status covers what the host can check (NULL pointers, sizes, dtype,
 *     element alignment, workspace size) plus launch errors.  Data errors are found on the
 *     device and poison only their sequence: accept_len[b] = -1, every out_tokens slot
 *     -1, every out_probs slot 0.  A sequence is invalid when k_b is outside [0, K]; T_b is
 *     negative, NaN, infinite or in (0, SPECDEC_TEMPERATURE_MIN); a used logit row
 *     (rows 0..k_b) holds a NaN or +inf or is all -inf; a proposed id in slots < k_b is
 *     outside [0, V); for a sampled row a used uniform (columns < k_b and column K) is
 *     outside [0, 1); or for a sampled model-draft row a gathered q_i(x_i) is negative or
 *     not finite, draft_probs is NULL, or -- at a rejection -- the rejected slot's draft row
 *     q_j (the one row the residual draw reads) holds an entry that is negative or not
 *     finite.
 *   - Padded rows and slots never influence a result: draft rows k_b..K-1 are never read;
 *     logit rows k_b+1..K (the small-vocabulary path loads rows 0..K together when K < 8) and
 *     proposed and uniform columns k_b..K-1 may be loaded (they lie inside the [B, K+1, V],
 *     [B, K] and [B, K+1] buffers) but their values, NaN included, are ignored.
 *   - Results are deterministic: the same inputs give bit-identical outputs on every run.
 */
#ifndef SPECDEC_H_
#define SPECDEC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPECDEC_OK = 0,
  SPECDEC_ERR_NULL = -1,      /* a required pointer is NULL                               */
  SPECDEC_ERR_SHAPE = -2,     /* B < 0, K < 0, K > SPECDEC_MAX_K, V < 1, or                */
                              /* B*(K+1)*ceil(V/8192) >= 2^31                               */
  SPECDEC_ERR_DTYPE = -3,     /* logits_dtype is not a specdec_dtype                      */
  SPECDEC_ERR_ALIGN = -4,     /* a tensor base is not aligned to its element size         */
  SPECDEC_ERR_WORKSPACE = -5, /* workspace NULL or smaller than specdec_workspace_size()  */
  SPECDEC_ERR_LAUNCH = -6,    /* a kernel launch or event record failed                   */
  SPECDEC_ERR_SCRATCH = -7    /* specdec_verify_noalloc: the sizes need more workspace    */
                              /* than its built-in scratch (SPECDEC_NOALLOC_SCRATCH_BYTES) */
} specdec_status;

typedef enum {
  SPECDEC_F32 = 0,            /* IEEE binary32 logits                                     */
  SPECDEC_BF16 = 1            /* bfloat16 logits (upper 16 bits of a binary32)            */
} specdec_dtype;

#define SPECDEC_MAX_K 63                  /* drafts per sequence (K+1 rows fit one wave64) */
#define SPECDEC_TEMPERATURE_MIN 1e-6f     /* smallest non-zero temperature accepted       */

/* Bytes of device workspace specdec_verify / specdec_verify_greedy / specdec_verify_match need
 * for these sizes (a pure function of B, K, V; 0 for B == 0 or invalid sizes).  The workspace
 * holds per-row partial statistics, the gathered drafted ids / logits / draft probabilities,
 * per-sequence draw state and per-segment weight sums; it needs no initialisation and its
 * contents are meaningless after the call.  Calls that overlap in time (different streams) need
 * separate workspaces. */
size_t specdec_workspace_size(int32_t B, int32_t K, int32_t V);

/* Batched rejection-sampling verify (sampled and greedy rows mixed by temperature).
 *
 * target_logits  [B, K+1, V]  logits_dtype; row i of sequence b is the target's
 *                             next-token logits after the prefix and drafts x_0..x_{i-1}.
 * draft_probs    [B, K, V]    float32 drafter probabilities q_i, used exactly as given
 *                             (never renormalised).  Only the gathered q_i(x_i) and, for a
 *                             rejected model-draft row, the one row q_j are read.  May be
 *                             NULL when no sampled row is a model-draft row.
 * draft_onehot   [B]          uint8, nonzero = one-hot (n-gram) row.  NULL = none.
 * proposed       [B, K]       int32 drafted ids x_i.  May be NULL when K == 0.
 * num_draft      [B]          int32 k_b in [0, K].  NULL = every sequence has K drafts.
 * temperature    [B]          float32; 0 = greedy row (reads neither q nor u).
 * uniforms       [B, K+1]     float32 in [0, 1): column i < K is accept test i, column K
 *                             the one correction-or-bonus draw.
 * accept_len     [B]    out   int32 A_b in [0, k_b], or -1 for an invalid sequence.
 * out_tokens     [B, K+1] out int32: slots 0..A_b hold the emitted tokens (accepted drafts,
 *                             then the correction or bonus token); other slots -1.
 * out_probs      [B, K+1] out float32 or NULL: the target probability p_i(token) of each
 *                             emitted token (greedy rows report softmax at T = 1); other
 *                             slots 0.
 * workspace                   device scratch of at least workspace_bytes >=
 *                             specdec_workspace_size(B, K, V) bytes, 16-byte aligned.
 * stream                      hipStream_t (NULL = default stream).
 * The caller rolls both KV caches back to prefix + accept_len[b] + 1 tokens.
 * On the streaming path the draw of a sequence is picked by one workgroup that waits, with a
 * bound (2^20 polls, about a second), for the other workgroups of its sequence; they come right
 * after it in dispatch order and none of them waits, so the wait ends, but if it ever gave up
 * (those workgroups unable to run for that long) the sequence would be reported invalid rather
 * than the call hanging.
 */
specdec_status specdec_verify(const void* target_logits, int32_t logits_dtype,
                              const float* draft_probs, const uint8_t* draft_onehot,
                              const int32_t* proposed, const int32_t* num_draft,
                              const float* temperature, const float* uniforms,
                              int32_t B, int32_t K, int32_t V,
                              int32_t* accept_len, int32_t* out_tokens, float* out_probs,
                              void* workspace, size_t workspace_bytes, void* stream);

/* specdec_verify without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP-graph capture, tight serving loops, harnesses that forbid allocation).  The
 * workspace is a file-scope device array of SPECDEC_NOALLOC_SCRATCH_BYTES (32 MiB) that each
 * device holds for the life of the process; its address is looked up once per device, on the
 * first call whose stream belongs to that device (the null stream: the current device), the
 * caller's current device being left as it was.  The call allocates nothing (no hipMalloc, no
 * library allocation).  Arguments, outputs, data errors and results are those of
 * specdec_verify (automatic path) with the same inputs.  Its argument checks (sizes, dtype,
 * NULL and misaligned pointers, with specdec_verify's status codes) run on the host before any
 * HIP call; after them it returns SPECDEC_ERR_SCRATCH, still before any HIP call, when
 * specdec_workspace_size(B, K, V) exceeds the scratch (for example B = 64,
 * K = 5, V = 128256 needs about 1.0 MB; B = 512, K = 8, V = 128256 about 11 MB).  Every call
 * on one device shares that device's scratch: calls that overlap in time on one device (other
 * streams, other threads) race; consecutive calls on one stream do not. */
#define SPECDEC_NOALLOC_SCRATCH_BYTES (32u << 20)

size_t specdec_noalloc_scratch_bytes(void);

specdec_status specdec_verify_noalloc(const void* target_logits, int32_t logits_dtype,
                                      const float* draft_probs, const uint8_t* draft_onehot,
                                      const int32_t* proposed, const int32_t* num_draft,
                                      const float* temperature, const float* uniforms,
                                      int32_t B, int32_t K, int32_t V,
                                      int32_t* accept_len, int32_t* out_tokens, float* out_probs,
                                      void* stream);

/* Greedy-only verify: every row is treated as temperature 0 (accept x_i iff it is the
 * lowest-index argmax of z_i; emit the argmax at the first mismatch or as the bonus).
 * Arguments as for specdec_verify; no q, T or u is read.  out_probs may be NULL; when
 * given it receives softmax at T = 1 of each emitted token. */
specdec_status specdec_verify_greedy(const void* target_logits, int32_t logits_dtype,
                                     const int32_t* proposed, const int32_t* num_draft,
                                     int32_t B, int32_t K, int32_t V,
                                     int32_t* accept_len, int32_t* out_tokens, float* out_probs,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* Execution paths.  Rows of at most SPECDEC_SMALL_V_MAX tokens fit one wavefront's registers,
 * so by default such calls run one kernel in which a group of lanes handles each sequence (a
 * whole wave64, or 16 or 8 lanes of one for rows of at most 64 or 32 tokens; every row read once,
 * the draw taken from registers); larger vocabularies run the streaming kernels: one 256-thread
 * workgroup per 8192-logit chunk of each row, then one launch for the accept scan, the draw and
 * its pick (when B times the number of chunks exceeds 1536, three: a scan pass, the draw pass and a
 * pick kernel).  SPECDEC_PATH_STREAMING forces the streaming kernels at any V,
 * SPECDEC_PATH_SMALL_VOCAB the small-vocabulary kernel (an error, SPECDEC_ERR_SHAPE, when
 * V > SPECDEC_SMALL_V_MAX), and SPECDEC_PATH_ONE_LAUNCH the same streaming work in a single launch
 * whose workgroups hand partial results to each other through the workspace (plus a small
 * zero-fill launch before it); it is slower on MI355X and kept for comparison.
 * SPECDEC_PATH_QUAD runs one launch of four 1024-thread workgroups per sequence, each streaming a
 * quarter of every row and exchanging quarter statistics and draw sums with the others through
 * tagged words in the workspace (no initialisation needed; each sequence keeps a counter there
 * that every call advances); it takes rows of whole 8-token groups (V a multiple of 8), 16-byte
 * aligned logits and draft rows, at most 32 2048-token segments per quarter (V <= 262144), no
 * sample-and-match mode, and no more sequences than leave all 4 B workgroups resident on the
 * device at once (B <= 64 on MI355X), else SPECDEC_ERR_SHAPE.  It measured even with the default
 * at B = 64, k = 5, V = 128256 and slower on smaller or ragged batches, and is kept for
 * comparison.  Every path implements the same rule and passes the same parity tests.
 * specdec_verify_greedy and specdec_verify_match take the automatic choice. */
#define SPECDEC_SMALL_V_MAX 1024
#define SPECDEC_PATH_AUTO 0
#define SPECDEC_PATH_STREAMING 1
#define SPECDEC_PATH_SMALL_VOCAB 2
#define SPECDEC_PATH_ONE_LAUNCH 3
#define SPECDEC_PATH_QUAD 4

/* Options of specdec_verify_ex.
 *   hot_event_begin / hot_event_end: measurement hook, HIP events (hipEvent_t, host handles)
 *     recorded by the dispatch of the kernel that reads every target row (the streaming
 *     logit-row kernel, or the small-vocabulary kernel on that path) when it starts and when it
 *     completes, so hipEventElapsedTime gives that kernel's own duration.  Either may be NULL.
 *   path: one of SPECDEC_PATH_*; any other value is SPECDEC_ERR_SHAPE.
 *   draw_event_begin / draw_event_end: the same hook around the kernels that run after the
 *     streaming kernel on the streaming path (accept scan, draw sums and pick): begin is recorded
 *     when the first of them starts, end when the last completes.  Not recorded on the
 *     small-vocabulary and one-launch paths (one kernel there).  Either may be NULL.
 *   spin_limit: SPECDEC_PATH_ONE_LAUNCH and SPECDEC_PATH_QUAD: polls a workgroup makes while it
 *     waits for a hand-off from another workgroup of the launch (0 = the default, 2^20 polls, about a second;
 *     negative = SPECDEC_ERR_SHAPE).  A wait that gives up reports its sequence as invalid
 *     (accept_len -1) instead of waiting longer, so the launch always completes; a small limit
 *     exercises that path in tests.
 * Passing opts == NULL to specdec_verify_ex is the same as specdec_verify (path AUTO). */
typedef struct {
  void* hot_event_begin;
  void* hot_event_end;
  int32_t path;
  int32_t spin_limit;
  void* draw_event_begin;
  void* draw_event_end;
} specdec_options;

specdec_status specdec_verify_ex(const void* target_logits, int32_t logits_dtype,
                                 const float* draft_probs, const uint8_t* draft_onehot,
                                 const int32_t* proposed, const int32_t* num_draft,
                                 const float* temperature, const float* uniforms,
                                 int32_t B, int32_t K, int32_t V,
                                 int32_t* accept_len, int32_t* out_tokens, float* out_probs,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 const specdec_options* opts);

/* Sample-and-match verify: the simpler exact scheme of "Decodificação especulativa
 * explicada" (gsantana.dev), section "A regra de amostragem por rejeição" (the paragraph after
 * the biased fallback).  Position i < k_b draws y_i ~ p_i by the inverse CDF above with
 * uniforms[b, i]; the draft x_i is kept while y_i == x_i; the first y_i != x_i is emitted and
 * ends the round (A = i); if all k_b are kept the bonus y_k ~ p_k is drawn with
 * uniforms[b, K] (A = k_b).  Every emitted token is a draw from p; a draft survives with
 * probability sum_x p(x) q(x), below the rejection rule's sum_x min(p(x), q(x)).  No draft
 * distribution is read.  Greedy rows, data errors, outputs and workspace are as for
 * specdec_verify (without the q conditions); a sequence's draft_onehot flag is irrelevant. */
specdec_status specdec_verify_match(const void* target_logits, int32_t logits_dtype,
                                    const int32_t* proposed, const int32_t* num_draft,
                                    const float* temperature, const float* uniforms,
                                    int32_t B, int32_t K, int32_t V,
                                    int32_t* accept_len, int32_t* out_tokens, float* out_probs,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * N-gram (prompt-lookup) drafter: the model-free proposer of
 *   - "Decodificação especulativa explicada" (gsantana.dev), section "A família de
 *     rascunhos", prompt lookup / n-gram drafting;
 *   - "ch15 · Speculative Decoding" (snowch.github.io), section "What proposes the tokens";
 *   - longest match first, after the longest-prefix match in "Speculative decoding: el
 *     secretario que adelanta lo que va a decir el jefe" (blog.lo0.es), section "Las cinco
 *     familias modernas".
 * For history h = tokens[b, 0..L) (L = lengths[b]): for n = min(n_max, L-1) down to n_min,
 * find the earliest p with h[p..p+n) == h[L-n..L) and p + n <= L - 1; the first n that has one
 * proposes h[p+n .. min(p+n+K, L)), so 1 <= num_draft[b] <= K.  No occurrence at any n:
 * num_draft[b] = 0.  L outside [0, capacity]: num_draft[b] = -1.  Unused proposed slots hold
 * -1.  The rows are one-hot drafts: verify them with draft_onehot[b] = 1.
 *
 * tokens      [B, capacity]  int32 histories; slots >= L may be loaded but are ignored.
 * lengths     [B]            int32 history lengths L.
 * n_min,n_max                1 <= n_min <= n_max <= SPECDEC_NGRAM_MAX_N.
 * K                          0 <= K <= SPECDEC_MAX_K proposals per sequence.
 * proposed    [B, K]   out   int32 (may be NULL when K == 0).
 * num_draft   [B]      out   int32 (the verify step's num_draft).
 * workspace                  device scratch of >= specdec_ngram_workspace_size(B, capacity)
 *                            bytes, 16-byte aligned; no initialisation needed.
 * One kernel launch, one workgroup per history, when capacity <= 8192 or the rows allow 16-byte
 * loads (tokens 16-byte aligned, capacity a multiple of 4); the workspace is then unused.
 * Otherwise two: per-tile keys in the workspace, then one wave per history takes their maximum
 * and copies the proposal.
 * Returns SPECDEC_ERR_SHAPE for out-of-range sizes or n_min / n_max, otherwise as for
 * specdec_verify. */
#define SPECDEC_NGRAM_MAX_N 32

size_t specdec_ngram_workspace_size(int32_t B, int32_t capacity);

specdec_status specdec_ngram_propose(const int32_t* tokens, const int32_t* lengths, int32_t B,
                                     int32_t capacity, int32_t n_min, int32_t n_max, int32_t K,
                                     int32_t* proposed, int32_t* num_draft, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Commit of a verified round: cache rollback and ragged compaction.  The step after verify in
 *   - "Decodificação especulativa explicada" (gsantana.dev), section "O ciclo de rascunho e
 *     verificação": the target's cache entries past the first rejection are dropped by
 *     truncating or moving a pointer back, and the drafter's cache is rolled back the same way;
 *   - "ch15 · Speculative Decoding" (snowch.github.io), section "The build";
 *   - "Speculative decoding: el secretario..." (blog.lo0.es), section "Pitfalls
 *     operacionales": each sequence accepts a different number of tokens per round.
 * For sequence b with A = accept_len[b] and L = seq_len[b] (tokens before the round), the
 * round emits n_b = A + 1 tokens out_tokens[b, 0..A]:
 *   tokens[b, L .. L+A] = out_tokens[b, 0..A];  seq_len[b] = L + A + 1;
 *   target_kv_len[b] = min(target_kv_len[b], L + A);  draft_kv_len[b] likewise
 *   (only the entries of the L prefix tokens and the A accepted drafts can be kept);
 *   packed_offsets[b] = n_0 + ... + n_{b-1}, packed_offsets[B] = the total, and
 *   packed_tokens[packed_offsets[b] + i] = out_tokens[b, i].
 * A sequence with A outside [0, K], L < 0, or L + A + 1 > capacity commits nothing: n_b = 0
 * and its lengths are left unchanged.
 *
 * accept_len      [B]        int32, from specdec_verify.
 * out_tokens      [B, K+1]   int32, from specdec_verify.
 * tokens          [B, capacity] int32 histories, appended in place; NULL = no history.
 * seq_len         [B]        int32 in/out.
 * target_kv_len   [B]        int32 in/out, or NULL.   draft_kv_len [B] likewise.
 * packed_tokens   [B*(K+1)]  int32 out, or NULL.      packed_offsets [B+1] int32 out, or NULL.
 * Needs no workspace.  SPECDEC_ERR_SHAPE: B < 0, K outside [0, SPECDEC_MAX_K], capacity < 1,
 * or B*(K+1) >= 2^31. */
specdec_status specdec_commit(const int32_t* accept_len, const int32_t* out_tokens, int32_t B,
                              int32_t K, int32_t* tokens, int32_t capacity, int32_t* seq_len,
                              int32_t* target_kv_len, int32_t* draft_kv_len,
                              int32_t* packed_tokens, int32_t* packed_offsets, void* stream);

/* ---------------------------------------------------------------------------------------
 * Acceptance telemetry and the per-route draft length.  The pages advise recording the
 * acceptance rate per route and choosing the draft length from it:
 *   - "Decodificação especulativa explicada" (gsantana.dev), sections "Quanto mais rápido: a
 *     matemática" (E[tokens per pass] = (1 - a^(k+1)) / (1 - a), speedup = E / (k c + 1)),
 *     "A tabela de speedup" (the best k per a and c) and "Checagem de realidade em produção"
 *     (record acceptance per route);
 *   - "Speculative decoding: el secretario..." (blog.lo0.es), sections "La matemática que
 *     importa: techo y speedup" and "Pitfalls operacionales" (tune the length dynamically).
 *
 * Counters: int64 [n_routes][SPECDEC_TELEMETRY_ROW], per route the fields
 *   0 rounds (valid rows)   1 drafted sum k_b   2 accepted sum A_b   3 emitted sum (A_b + 1)
 *   4 rounds with A_b = k_b   5 rounds with A_b < k_b (one rejected position each)
 *   6 invalid rows   7 reserved (0)   8 + a: rounds with A_b = a (a = 0..63).
 * A row is invalid when accept_len < 0, k_b is outside [0, K] or A_b > k_b; rows whose route id
 * is outside [0, n_routes) are not counted. */
#define SPECDEC_TELEMETRY_FIELDS 8
#define SPECDEC_TELEMETRY_ROW 72
#define SPECDEC_TELEMETRY_MAX_ROUTES 64

/* Adds one verified batch to the DEVICE counters (stream-ordered; the caller zeroes them once).
 * accept_len [B] int32 (from a verify call); num_draft [B] int32 or NULL (= K); route [B] int32
 * or NULL (= route 0); 1 <= n_routes <= SPECDEC_TELEMETRY_MAX_ROUTES.  Integer sums: the result
 * does not depend on the order.  Calls that overlap on the same counters race. */
specdec_status specdec_telemetry_update(const int32_t* accept_len, const int32_t* num_draft,
                                        const int32_t* route, int32_t B, int32_t K,
                                        int32_t n_routes, int64_t* counters, void* stream);

/* Host arithmetic on HOST copies of the counters.  specdec_alpha_estimate: accepted /
 * (accepted + rejected positions), the maximum-likelihood per-token rate (NaN without
 * observations).  specdec_expected_tokens / specdec_speedup: the formulas above (NaN outside
 * alpha in [0, 1], k >= 0, c >= 0).  specdec_choose_k: the k in [k_min, k_max] with the largest
 * speedup (the smaller k on ties), -1 for invalid arguments.  specdec_plan_k: k_table[r] for each
 * route (k_default for a route without observations). */
double specdec_alpha_estimate(const int64_t* route_counters);
double specdec_expected_tokens(double alpha, int32_t k);
double specdec_speedup(double alpha, int32_t k, double c);
int32_t specdec_choose_k(double alpha, double c, int32_t k_min, int32_t k_max);
specdec_status specdec_plan_k(const int64_t* counters, int32_t n_routes, double c, int32_t k_min,
                              int32_t k_max, int32_t k_default, int32_t* k_table);

/* Applies a plan on the DEVICE: num_draft[b] = min(num_draft[b], max(0, k_table[route[b]])) for
 * rows with num_draft[b] >= 0 and a route id in [0, n_routes) (route NULL = route 0).  The
 * proposals past the new count are simply not verified. */
specdec_status specdec_apply_k(int32_t* num_draft, const int32_t* route, const int32_t* k_table,
                               int32_t B, int32_t n_routes, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* specdec_status_string(int32_t status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t specdec_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECDEC_H_ */
