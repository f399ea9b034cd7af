/*
 * specsam.h — C ABI of the MI355X (gfx950) batched speculative-decoding step:
 * lossless verification of K drafted tokens against target logits, and
 * SAM-Decoding's per-sequence dynamic suffix automaton (extend and draft).
 *
 * Pages this interface follows (cited by title and section):
 *   [P1] "SAM投机推理：长序列强化学习训练加速利器" (CANN cann-recipes-train
 *        article): §1.1 "SAM 原理" (endpos, link, min_endpos, dynamic SAM
 *        updated after every verified token, the link-walk draft, acceptance
 *        test eps <= alpha(x)); §3.1.2 "拒绝采样加速" (recovered token at the
 *        rejected position, bonus token when all drafts pass).
 *   [P2] speculative-sampling guide "1. 投机采样到底在解决什么问题"
 *        (m.nxbn.cn): §2.2 "验证阶段的并行打分机制" (accept with
 *        min(1, p/q), resample from the positive part of p - q, K+1 target
 *        distributions from one forward, truncate at the first rejection).
 *   [P3] notes "投机采样" (gogongxt.com): "贪婪采样" (T = 0: accept iff the
 *        draft equals the target argmax), "SGLang 的实现" (coins per draft
 *        slot plus one final coin; one-hot drafts when no draft
 *        probabilities exist).
 *   [P4] SAM-Decoding summary (developer.volcengine.com): §3 "Suffix
 *        Automaton Construction" (Blumer's online construction, min_endpos),
 *        "Drafting with Suffix Automaton", "Update of Suffix Automaton".
 *
 * Conventions for every entry point:
 *   - Array arguments are DEVICE pointers to memory of the current HIP device,
 *     row-major and contiguous, owned by the caller. The library keeps no
 *     global state and never allocates, frees or synchronises.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     asynchronously on it; a state buffer or workspace must not be used on
 *     two streams at once.
 *   - Return codes are synchronous: SS_OK, or an SS_E* code for problems the
 *     host can see (bad sizes, null pointers, launch failure). Problems that
 *     depend on device data are reported per sequence in a sticky status word
 *     (bitwise OR of SS_ST_*) without any host synchronisation; a sequence
 *     flagged in a call is skipped by that call (its outputs are not written).
 */
#ifndef SPECSAM_H
#define SPECSAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes -------------------------------------------------------- */
#define SS_OK 0
#define SS_EINVAL (-1)     /* invalid argument (sizes, null pointer, dtype) */
#define SS_EWORKSPACE (-2) /* workspace too small */
#define SS_ELAUNCH (-3)    /* HIP launch error; see ss_last_error_string() */

/* ---- per-sequence status bits ------------------------------------------- */
#define SS_ST_SAM_CAPACITY (1 << 0) /* extend would exceed max_len tokens */
#define SS_ST_TOKEN_RANGE (1 << 1)  /* a token outside [0, V) */
#define SS_ST_DRAFT_LEN (1 << 2)    /* draft_len outside [0, K] */
#define SS_ST_NONFINITE (1 << 3)    /* row with NaN, +inf, or all -inf */
#define SS_ST_TEMPERATURE (1 << 4)  /* T NaN, negative, inf, or positive
                                       below the smallest normal float */
#define SS_ST_NO_UNIFORMS (1 << 5)  /* T > 0 but uniforms == NULL */
#define SS_ST_COUNT (1 << 6)        /* extend count outside [0, ld_tokens] */
#define SS_ST_TOP_P (1 << 7)        /* top_p NaN or outside (0, 1] */
#define SS_ST_TREE (1 << 8)         /* malformed draft tree (spec_verify_tree) */

#define SS_MAX_K 16            /* largest number of drafted tokens */
#define SS_MAX_LEN (1 << 24)   /* largest automaton capacity, tokens */
#define SS_MAX_TREE 64         /* largest draft tree, nodes (root included) */

#define SS_DTYPE_F32 0
#define SS_DTYPE_BF16 1

/* Library version (major*10000 + minor*100 + patch). */
int ss_version(void);

/* Text of the last SS_ELAUNCH / SS_EINVAL on the calling thread. */
const char* ss_last_error_string(void);

/* ========================================================================= *
 * Verification ([P2] §2.2, [P3] "贪婪采样" / "拒绝采样", [P1] §1.1, §3.1.2)
 * ========================================================================= */

/* Bytes of workspace spec_verify / spec_step need for (B, K, V); 0 if
 * unsupported. The workspace is scratch owned by the caller (256-byte
 * aligned): it needs no initialisation, its contents between calls do not
 * matter, and one buffer serves any call whose size fits. A workspace must
 * not serve two calls that may run concurrently. */
size_t ss_verify_workspace_bytes(int B, int K, int V);

/* The same with options: flags = 0, or SS_WS_TRUNCATION for calls that pass
 * top_k or top_p (truncation needs per-(row, chunk) histograms, band
 * segments and sums: about (K+1) * B * nchunks * (2 KiB + min(1024, V) *
 * 4 B), nchunks = ceil(V / 8192)). 0 for unsupported sizes or flags. */
#define SS_WS_TRUNCATION 1
size_t ss_verify_workspace_bytes_ex(int B, int K, int V, int flags);

/*
 * spec_verify — one batched verification step.
 *
 * For each sequence b with d = draft_len[b] drafts x_0..x_{d-1} and target
 * logits rows l_0..l_d (row j scores the token after the prompt plus drafts
 * x_0..x_{j-1}; rows j > d are never read):
 *   T = temperature[b] == 0 (greedy): accept x_j iff x_j == argmax l_j (lowest
 *     index on ties); the first mismatch emits argmax l_j and stops; if all d
 *     pass, argmax l_d is emitted.
 *   T > 0: p_j = softmax(l_j / T). Accept x_j iff u[b,j] <= p_j(x_j) / q_j(x_j)
 *     where q_j(x_j) is q[b,j,x_j] (q given) or 1 (q == NULL: one-hot drafts).
 *     At the first rejection j, emit a token drawn from max(0, p_j - q_j)
 *     normalised (q given; falls back to p_j if that is zero everywhere) or
 *     from p_j with x_j removed (one-hot), and stop. If all d pass, emit a
 *     bonus token drawn from p_d. Draws use the final coin u[b,K]: the
 *     smallest token i with (sum of weights of tokens <= i) > u * (total).
 *
 * Arguments:
 *   logits      [B, K+1, V], dtype SS_DTYPE_F32 (float) or SS_DTYPE_BF16
 *               (bfloat16, widened exactly to float). Must start on a
 *               16-byte boundary (SS_EINVAL otherwise); rows are read 16
 *               bytes at a time when V is a multiple of 4 (fp32) or 8
 *               (bf16), element by element otherwise.
 *   draft       [B, K] int32; entries j >= draft_len[b] are ignored.
 *   draft_len   [B] int32 in [0, K].
 *   q           [B, K, V] float draft probabilities, or NULL for one-hot;
 *               16-byte aligned like logits.
 *   temperature [B] float >= 0.
 *   uniforms    [B, K+1] float in [0, 1]: columns 0..K-1 are the acceptance
 *               coins, column K the final coin. May be NULL only if every
 *               temperature is 0. A final coin of 1 takes the distribution's
 *               last token of positive weight (the inverse CDF's limit).
 *   top_k       [B] int32 or NULL; top_p [B] float or NULL: truncation of the
 *               target distribution of a sequence at T > 0 before it is used
 *               anywhere above ([P3] "SGLang 的实现": the target probabilities
 *               are renormalised by top-k, then top-p, one value of each per
 *               request, applied to all K+1 positions). p_j is replaced by
 *               p'_j: top-k (1 <= k < V) keeps every token whose logit is at
 *               least the k-th largest logit of the row (ties kept); top-p
 *               (0 < top_p < 1), applied to what top-k kept, keeps whole
 *               groups of equal logits from the largest down until the kept
 *               share of what top-k kept reaches top_p; p'_j is p_j on the
 *               kept tokens, renormalised. k <= 0 or k >= V, and top_p = 1,
 *               do nothing; top_p NaN or outside (0, 1] sets SS_ST_TOP_P.
 *               Greedy sequences are not affected. Acceptance, residual,
 *               bonus and p_draft all use p'_j; logprobs stay those of the
 *               untruncated p_j. With either pointer non-NULL the workspace
 *               must come from ss_verify_workspace_bytes_ex(...,
 *               SS_WS_TRUNCATION).
 *   out_tokens  [B, K+1] int32: accepted drafts then the corrected / bonus
 *               token; -1 after num_emitted.
 *   num_emitted [B] int32 = accepted drafts + 1.
 *   p_draft     [B, K] float or NULL: p_j(x_j) for j < num_emitted and j < d
 *               at T > 0; -1 elsewhere.
 *   logprobs    [B, K+1] float or NULL: for j < num_emitted, the natural log
 *               of softmax(l_j / T)[out_tokens[b, j]] — the target's own
 *               log-probability of each emitted token (accepted, corrected or
 *               bonus), with T = 1 for greedy sequences ([P1] §2.1 compares
 *               these between decoding paths); NaN after num_emitted.
 *   status      [B] int32, OR-ed with SS_ST_* bits.
 *   workspace   ws_bytes >= ss_verify_workspace_bytes(B, K, V), 256-byte
 *               aligned.
 * Limits: 1 <= B, 1 <= K <= SS_MAX_K, 1 <= V <= 2^21. A temperature that is
 * positive but below the smallest normal float is reported as
 * SS_ST_TEMPERATURE.
 * Errors: SS_EINVAL for sizes/null pointers/dtype/misaligned logits or q,
 * SS_EWORKSPACE, SS_ELAUNCH.
 */
int spec_verify(const void* logits, int dtype, int B, int K, int V,
                const int32_t* draft, const int32_t* draft_len, const float* q,
                const float* temperature, const float* uniforms,
                const int32_t* top_k, const float* top_p, int32_t* out_tokens, int32_t* num_emitted, float* p_draft,
                float* logprobs, int32_t* status, void* workspace,
                size_t ws_bytes, void* stream);

/*
 * spec_step — one whole speculative step in one pass over the logits:
 * spec_verify with one-hot drafts (q = NULL), then, for each sequence, the
 * emitted tokens extend its automaton (sam_extend) and the next draft is
 * taken from it (sam_draft) — [P1] §1.1: the dynamic SAM is updated after each
 * verified token and drafts from its link walk.
 *   draft, draft_len    this step's drafts (from sam_draft or the previous
 *                       spec_step).
 *   sam_state, max_len  the automata (see below).
 *   next_draft [B, K], next_draft_len [B], next_match_len [B]: the drafts for
 *                       the next step; must not alias draft / draft_len.
 * Other arguments as spec_verify. A sequence flagged in this call is not
 * extended; its next draft comes from its unchanged automaton. Status bits of
 * the automaton itself go to the automaton's own status word (sam_status).
 */
int spec_step(const void* logits, int dtype, int B, int K, int V,
              const int32_t* draft, const int32_t* draft_len,
              const float* temperature, const float* uniforms,
              const int32_t* top_k, const float* top_p, void* sam_state,
              int max_len, int32_t* out_tokens, int32_t* num_emitted,
              float* p_draft, float* logprobs, int32_t* status,
              int32_t* next_draft,
              int32_t* next_draft_len, int32_t* next_match_len,
              void* workspace, size_t ws_bytes, void* stream);

/*
 * spec_step_noalloc — spec_step with no workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The workspace is a device array of
 * SS_SCRATCH_BYTES inside the library; each GPU the library runs on holds
 * its own copy until the process ends, its address taken on the first call
 * on that device. The call allocates and frees nothing. All calls on one GPU
 * share that array: calls that may overlap on a GPU (two streams, two host
 * threads) race and must not be issued; consecutive calls on one stream are
 * fine (the array needs no initialisation; whatever a previous call left in
 * it does not matter).
 * Arguments, outputs and status as spec_step. Errors as spec_step, and
 * SS_EWORKSPACE when the sizes need more than SS_SCRATCH_BYTES of workspace
 * (ss_verify_workspace_bytes_ex(B, K, V, flags) > SS_SCRATCH_BYTES, with
 * SS_WS_TRUNCATION when top_k or top_p is given): e.g. B = 256, K = 3,
 * V = 151936 needs about 0.65 MB; truncation needs far more.
 */
#define SS_SCRATCH_BYTES ((size_t)8 << 20)
int spec_step_noalloc(const void* logits, int dtype, int B, int K, int V,
                      const int32_t* draft, const int32_t* draft_len,
                      const float* temperature, const float* uniforms,
                      const int32_t* top_k, const float* top_p, void* sam_state,
                      int max_len, int32_t* out_tokens, int32_t* num_emitted,
                      float* p_draft, float* logprobs, int32_t* status,
                      int32_t* next_draft, int32_t* next_draft_len,
                      int32_t* next_match_len, void* stream);

/*
 * The two passes of spec_verify / spec_step as separate calls, for callers
 * that schedule them (and for timing the HBM pass alone):
 *   spec_stream  reads the logit rows j <= draft_len once and leaves per-row
 *                statistics in the workspace.
 *   spec_finish  judges the drafts, draws the recovered / bonus tokens (with
 *                the residual pass when q is given) and, when sam_state is
 *                non-NULL, updates the automata and writes the next drafts
 *                (then q must be NULL and the next-draft outputs non-NULL).
 * spec_finish must follow spec_stream on the same stream with the same
 * logits, sizes, drafts, temperatures, uniforms, top_k, top_p and workspace
 * (with truncation, spec_stream also leaves each truncated row's chunk
 * histograms and band segments, and spec_finish first runs the truncation
 * selection over them).
 */
int spec_stream(const void* logits, int dtype, int B, int K, int V,
                const int32_t* draft, const int32_t* draft_len,
                const float* temperature, const float* uniforms,
                const int32_t* top_k, const float* top_p, void* workspace,
                size_t ws_bytes, void* stream);

int spec_finish(const void* logits, int dtype, int B, int K, int V,
                const int32_t* draft, const int32_t* draft_len, const float* q,
                const float* temperature, const float* uniforms,
                const int32_t* top_k, const float* top_p, int32_t* out_tokens, int32_t* num_emitted, float* p_draft,
                float* logprobs, int32_t* status, void* sam_state, int max_len,
                int32_t* next_draft, int32_t* next_draft_len,
                int32_t* next_match_len, void* workspace, size_t ws_bytes,
                void* stream);

/*
 * spec_verify_tree — verification of one draft tree per sequence ([P3]
 * "SGLang 的实现": the target-only tree sampling, taken with both of its
 * acceptance thresholds at 1, its lossless case).
 *
 * Tree of sequence b: node 0 is the root (the last committed token); nodes
 * 1..n_nodes[b]-1 each carry a drafted token tokens[b,i] and a parent
 * parent[b,i] < i (parent[b,0] = -1). Logit row i of the sequence scores the
 * token after the path root..i. The children of a node are taken in
 * increasing node index and must carry distinct tokens.
 *   T = 0: from the root, move to the child whose token is the argmax of the
 *     current node's row (lowest index on ties); when there is none, emit the
 *     argmax and stop.
 *   T > 0: at depth t (t tokens accepted so far), with p = softmax(l_cur / T),
 *     the children c_1, c_2, ... add p(token) to a running sum in node order;
 *     the first child with u[b,t] <= its running sum is accepted. When none
 *     is, the final token is drawn with u[b,N-1] (inverse CDF in ascending
 *     token order, as spec_verify) from p with every child's token removed;
 *     at a leaf, from the leaf's row. Each emitted token is then distributed
 *     as the target's p.
 * Arguments:
 *   logits      [B, N, V] (dtype and alignment as spec_verify); rows >=
 *               n_nodes[b] unread.
 *   tokens, parent [B, N] int32; n_nodes [B] int32 in [1, N].
 *   temperature [B]; uniforms [B, N] float in [0, 1] (coins per depth, the
 *               last column the final coin), NULL only if every T is 0.
 *   out_tokens  [B, N] int32: accepted tokens then the final token, -1 after.
 *   out_nodes   [B, N] int32: the node each emitted token came from (the
 *               accepted child; for the final token the node whose row it was
 *               drawn from), -1 after.
 *   num_emitted [B] = accepted + 1. status [B] OR-ed with SS_ST_* (SS_ST_TREE
 *               for a malformed tree or n_nodes outside [1, N]).
 *   workspace   ss_tree_workspace_bytes(B, N, V), 256-byte aligned.
 * Limits: 1 <= B, 1 <= N <= SS_MAX_TREE, 1 <= V <= 2^21.
 */
size_t ss_tree_workspace_bytes(int B, int N, int V);
int spec_verify_tree(const void* logits, int dtype, int B, int N, int V,
                     const int32_t* tokens, const int32_t* parent,
                     const int32_t* n_nodes, const float* temperature,
                     const float* uniforms, int32_t* out_tokens, int32_t* out_nodes,
                     int32_t* num_emitted, int32_t* status, void* workspace,
                     size_t ws_bytes, void* stream);

/* ========================================================================= *
 * Dynamic suffix automaton ([P1] §1.1, [P4] §3)
 *
 * One automaton per sequence over that sequence's committed tokens. State 0 is
 * the root; every appended token creates one state ("cur") and at most one
 * clone, numbered in creation order (cur before clone). Each state has len
 * (longest string), link (suffix link, -1 for the root) and min_endpos (first
 * end position of its strings, 0-indexed; -1 for the root). Capacity per
 * sequence: max_len tokens, 2*max_len states, 3*max_len transitions.
 * ========================================================================= */

/* Bytes of one state buffer for B sequences of capacity max_len tokens. */
size_t sam_state_bytes(int B, int max_len);

/* Resets every sequence to the empty text (root only). V is the vocabulary
 * size used to range-check appended tokens. */
int sam_init(void* state, int B, int max_len, int V, void* stream);

/*
 * sam_extend — appends counts[b] tokens tokens[b*ld_tokens + 0 ..] to
 * sequence b, in order, by Blumer's online extension ([P4] §3 "Update of
 * Suffix Automaton": after verification the accepted tokens extend the
 * automaton). Serves both prefill (counts = prompt lengths) and the per-step
 * append (tokens = out_tokens, ld = K+1, counts = num_emitted).
 * A sequence whose status is non-zero is skipped. Capacity overflow, a token
 * outside [0, V) or a count outside [0, ld_tokens] sets the status bit and
 * stops before that token; tokens appended before it stay appended.
 */
int sam_extend(void* state, int B, int max_len, const int32_t* tokens,
               int ld_tokens, const int32_t* counts, void* stream);

/*
 * sam_draft — per sequence: from the state of the whole text follow suffix
 * links until a state with an outgoing transition ([P1] §1.1, the ABCBC
 * example); its len is the match length L and min_endpos p locates the first
 * earlier occurrence of the matched suffix. L == 0 gives draft_len 0;
 * otherwise draft_len = min(K, n-1-p) and draft[j] = text[p+1+j].
 *   draft [B, K] int32 (-1 padded), draft_len [B], match_len [B] int32.
 */
int sam_draft(const void* state, int B, int max_len, int K, int32_t* draft,
              int32_t* draft_len, int32_t* match_len, void* stream);

/*
 * sam_draft_tree — per sequence, a draft tree for spec_verify_tree from
 * several candidates: the state sam_draft's walk reaches, then up to M - 1 of
 * its suffix-link ancestors (shorter suffixes of the text whose occurrences
 * are a superset; the root ends the list), each giving the tokens after its
 * first occurrence (K at most, cut at the end of the text). The candidates
 * are merged into a trie in that order: node 0 is the root, a candidate walks
 * down the children carrying its tokens and adds a node where none matches,
 * so node order (which spec_verify_tree tries siblings in) follows the
 * candidates' order and candidate 0 is sam_draft's draft.
 *   K >= 1, M >= 0, 1 + M*K <= N <= SS_MAX_TREE.
 *   tokens, parent [B, N] int32: node i's token and parent (root: -1, -1;
 *   -1 past n_nodes); n_nodes [B]; match_len [B] (sam_draft's) or NULL.
 */
int sam_draft_tree(const void* state, int B, int max_len, int K, int M, int N,
                   int32_t* tokens, int32_t* parent, int32_t* n_nodes,
                   int32_t* match_len, void* stream);

/* sam_extend followed by sam_draft in one launch (per-step use). */
int sam_extend_draft(void* state, int B, int max_len, const int32_t* tokens,
                     int ld_tokens, const int32_t* counts, int K,
                     int32_t* draft, int32_t* draft_len, int32_t* match_len,
                     void* stream);

/* Measurement: sam_extend with work counters. Adds, over all sequences, to
 * stats[7] (uint64, device): tokens appended, hash lookups, 128-byte buckets
 * read by them, suffix-link steps that inserted a transition, clones,
 * transitions copied into clones, transitions redirected to clones. The
 * automaton ends up exactly as after sam_extend. */
int sam_extend_stats(void* state, int B, int max_len, const int32_t* tokens,
                     int ld_tokens, const int32_t* counts,
                     unsigned long long* stats, void* stream);

/*
 * sam_match — the static automaton of [P4] §3 ("Suffix Automaton
 * Construction": built offline over a corpus whose documents are joined with
 * an end-of-sequence token; "Drafting with Suffix Automaton"; "Update of
 * Suffix Automaton": the matching state is transferred with each accepted
 * token). static_state is a state buffer of ONE sequence (B = 1, capacity
 * static_max_len) holding the corpus, built with sam_init + sam_extend; it is
 * only read here.
 *   match [B, 2] int32 (state, length): the state of the longest suffix of
 *     sequence b's text that occurs in the corpus, and that suffix's length.
 *     Start from zeros (root, empty match); this call updates it in place.
 *     An entry that is not a state of the automaton, or whose length exceeds
 *     that state's longest string, is taken as the root.
 *   tokens [B, ld_tokens] int32, counts [B] (device; NULL: no tokens): the
 *     tokens appended to each sequence since the last call; a count outside
 *     [0, ld_tokens] reads no token and sets SS_ST_COUNT in status[b] (status
 *     [B] int32, or NULL). For each token t:
 *     if the state has a transition on t it is taken (length + 1); else
 *     suffix links are followed to the first state with one (length = that
 *     state's len + 1); if even the root has none, (root, 0).
 *   K > 0 also writes drafts: the static draft is the K tokens after the
 *     state's min_endpos in the corpus (cut at its end; none for an empty
 *     match). With dyn_draft/dyn_len/dyn_match given (all three, e.g. the
 *     next-draft outputs of spec_step), the dynamic draft is kept unless the
 *     static match is longer than dyn_match[b] + delta, as the page prefers
 *     the dynamic automaton's drafts. Without them the static drafts are
 *     written. draft [B, K] int32 (-1 padded), draft_len [B]; source [B]
 *     (or NULL) receives 1 where the static draft was taken.
 * K = 0 only advances the match states. delta >= 0.
 * CURRENTLY SWITCHED OFF: returns SS_EINVAL without launching anything (one
 * GPU run of its tests ended in a memory fault whose cause is not shown).
 */
int sam_match(const void* static_state, int static_max_len, int B, int32_t* match,
              const int32_t* tokens, int ld_tokens, const int32_t* counts, int K,
              int delta, const int32_t* dyn_draft, const int32_t* dyn_len,
              const int32_t* dyn_match, int32_t* draft, int32_t* draft_len,
              int32_t* source, int32_t* status, void* stream);

/* Copies the sticky per-sequence status words to status_out [B] int32. */
int sam_status(const void* state, int B, int max_len, int32_t* status_out,
               void* stream);

/*
 * sam_export — debugging and parity: copies sequence b's automaton into
 * caller device buffers.
 *   header_out [8] int32: n (tokens), last, num_states, num_edges, status,
 *              max_len, V, hash_slots.
 *   states_out [2*max_len, 4] int32 rows (len, link, min_endpos, first_edge);
 *              rows >= num_states are unspecified.
 *   edges_out  [hash_slots, 4] int32 rows (src, token, dst, next); src == -1
 *              marks an empty row. Each transition appears exactly once.
 *   text_out   [max_len] int32: the committed tokens.
 */
int sam_export(const void* state, int B, int max_len, int b,
               int32_t* header_out, int32_t* states_out, int32_t* edges_out,
               int32_t* text_out, void* stream);

/* Number of hash rows per sequence for capacity max_len (edges_out size). */
int sam_hash_slots(int max_len);

#ifdef __cplusplus
}
#endif

#endif /* SPECSAM_H */
