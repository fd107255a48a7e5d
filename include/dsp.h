/*
 * dsp.h -- C ABI of the MI355X (gfx950) library for confidence-scheduled
 * speculative decoding: Markov-head drafting (greedy chain and PCTree tree
 * expansion), the confidence scheduler, ragged packing and batched verify.
 *
 * Sources of the operations (web pages on DSpark and PCTree):
 *   [N]  DSpark study notes, pages.layerx.co.jp ("DSpark: Confidence-Scheduled
 *        Speculative Decoding with Semi-Autoregressive Generation"), sections 1-9.
 *   [P]  PCTree article, qiita.com ("Parent-Conditioned Drafting Tree").
 *   [S]  SGLang integration article, winzheng.jp ("DSpark in SGLang").
 *
 * Conventions shared by every call
 *   - All pointers are DEVICE pointers unless a parameter says "host".
 *     The library never allocates device memory: every call that needs
 *     scratch space takes (ws, ws_bytes) sized by its *_workspace_size query.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = default
 *     stream) and deterministic: identical inputs give identical bits.
 *   - Inputs are read only; outputs must not alias inputs or each other.
 *   - Return value: DSP_OK (0) or a negative DSP_ERR_* code. Argument checks
 *     run on the host before any HIP call, so an error return means nothing
 *     was launched. dsp_last_error() gives a message (thread local).
 *   - Data-dependent faults that only the device can see (a token id outside
 *     [0, V), a window outside [0, K], non-finite logits) are OR-ed into the
 *     device word `*status` as DSP_STATUS_* bits; the caller zeroes it before
 *     the call and reads it after synchronising. The affected request's
 *     outputs are set to -1.
 *   - Logit rows: element (row r, token v) lives at base + r*ld + v, with ld
 *     in elements, ld >= V. dtype is DSP_F32 or DSP_BF16 (bfloat16 bits).
 *   - Calls on the same stream may be issued back to back; concurrent calls
 *     must use distinct workspaces.
 */
#ifndef DSP_H
#define DSP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSP_OK                 0
#define DSP_ERR_NULL          -1  /* a required pointer is NULL */
#define DSP_ERR_SHAPE         -2  /* a size or stride is out of range */
#define DSP_ERR_DTYPE         -3  /* unknown dtype code */
#define DSP_ERR_ALIGN         -4  /* pointer alignment requirement not met */
#define DSP_ERR_WORKSPACE     -5  /* workspace NULL or smaller than the query */
#define DSP_ERR_UNSUPPORTED   -6  /* valid but unsupported combination */
#define DSP_ERR_HIP           -7  /* a HIP runtime call failed */

#define DSP_F32   0
#define DSP_BF16  1
/* bf16 base logits stored token-major (the chain's L only; see dsp_draft_markov_step) */
#define DSP_BF16_TOKEN_MAJOR  2

#define DSP_STATUS_TOKEN_RANGE   1  /* a token id outside [0, V) */
#define DSP_STATUS_WINDOW_RANGE  2  /* cu_seqlens / windows inconsistent with K or max_rows */
#define DSP_STATUS_NONFINITE     4  /* a logits row whose maximum is not finite */
#define DSP_STATUS_TIMEOUT       8  /* a persistent launch's grid barrier gave up waiting */

#define DSP_SCHED_EARLY_STOP  0
#define DSP_SCHED_ARGMAX      1
#define DSP_SCHED_TOP_M       2
#define DSP_SCHED_THRESHOLD   3

/* Library version, (major << 16) | minor. */
int32_t dsp_version(void);

/* Message describing the last error returned on this thread ("" if none). */
const char* dsp_last_error(void);

/* ------------------------------------------------------------------------ */
/* Counter-based uniforms.                                                   */
/*                                                                          */
/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As   */
/* Easy as 1, 2, 3", SC'11) keyed by (seed, 0). For n counters given as      */
/* ctr[4*j .. 4*j+3] (uint64, device), writes the four output words of each   */
/* block mapped to doubles in [0, 1) as (w >> 11) * 2^-53 into out[4*j ..].   */
/* This is the generator the verify call uses at counter (round, request id, */
/* position k, 0): word 0 is the accept uniform u_k, word 1 the sampling      */
/* uniform u'_k.                                                             */
/* ------------------------------------------------------------------------ */
int32_t dsp_philox_uniforms(const uint64_t* ctr, int64_t n, uint64_t seed, double* out,
                            void* stream);

/* ------------------------------------------------------------------------ */
/* Confidence head with sequential temperature scaling  ([N] 5.1; [S] STS)   */
/*                                                                          */
/* conf[i*K + k] = sigmoid((w . h_{i,k} + bias) / T_k): the probability that  */
/* draft k of request i survives verification given that drafts 1..k-1 did,  */
/* from a linear projection of the draft's hidden state; T_k (sts_temp[k],   */
/* device, nullable = all 1) is the position's calibration temperature. The  */
/* output is the scheduler's conf input.                                     */
/*   h: [R, K, H] hidden states, element (i, k, j) at h + i*ld_h_r +         */
/*      k*ld_h_k + j; h_dtype / w_dtype DSP_F32 or DSP_BF16; w: [H].         */
/*   Dot products in fp32 per 8 elements, summed in fp64; logit, temperature */
/*   and sigmoid in fp64, output fp32. A NaN result sets                     */
/*   DSP_STATUS_NONFINITE. No workspace.                                     */
/* ------------------------------------------------------------------------ */
int32_t dsp_confidence_head(const void* h, int32_t h_dtype, int64_t ld_h_r, int64_t ld_h_k, const void* w,
                            int32_t w_dtype, float bias, const float* sts_temp, int32_t R, int32_t K,
                            int32_t H, float* conf, int32_t* status, void* stream);

/* ------------------------------------------------------------------------ */
/* Survival products and window selection  ([N] 5.1-5.2, [S] "SPS cost table") */
/*                                                                          */
/* conf [R, K] float32 row-major: c_{i,k}, the probability that draft k of    */
/* request i survives given that drafts 1..k-1 did ([N] 5.1).                 */
/* Survival S_{i,k} = prod_{j<=k} c_{i,j} (fp64, left to right). Candidates   */
/* (i, k) are ranked by S descending (ties: i, then k ascending); with E_j the*/
/* sum of the first j survivals and cost[j] the step time when j draft tokens */
/* are verified, candidate j is taken iff E_j / cost[j] > E_{j-1} / cost[j-1] */
/* (throughput strictly rises), stopping at the first candidate that fails    */
/* (DSP_SCHED_EARLY_STOP, the non-anticipating rule of [N] 5.2), or the       */
/* smallest j maximising E_j / cost[j] (DSP_SCHED_ARGMAX, the SPS-argmax      */
/* budget of [S] / global search of [N] 9.2; cost must then be > 0).          */
/* DSP_SCHED_TOP_M takes the first max_tokens candidates of that order: a     */
/* verify capacity decided earlier (from confidences two steps old, [N] 9.2)  */
/* with the ranking from the current survivals. DSP_SCHED_THRESHOLD is the    */
/* conventional fixed threshold ([N] 5.2, 8.3): n_i = #{k : S_{i,k} >=        */
/* threshold} on the fp64 survival; threshold 0 verifies the full block.      */
/* Survivals are summed as exact integers on a 2^-Q grid,                     */
/* Q = min(40, 53 - ceil(log2(R*K))), so the windows are bit-reproducible.    */
/*   cost      [n_cost] fp64, n_cost >= R*K + 1 (device).                     */
/*   max_tokens  cap on N = sum_i n_i (< 0: none); the capacity in TOP_M mode.  */
/*   threshold   survival threshold of DSP_SCHED_THRESHOLD (ignored otherwise;  */
/*               NaN is rejected).                                             */
/* Outputs: windows [R] int32 (n_i in [0, K]); survival [R, K] fp64 (nullable);*/
/* stats [4] fp64 (nullable): N, E (in probability units), J = E / cost[N], Q. */
/* Limits: 1 <= K <= 128, 1 <= R, R*K <= 8192.                                 */
/* Workspace: dsp_schedule_windows_workspace_size(R, K) bytes (the ranked     */
/* keys), required in every mode.                                            */
/* ------------------------------------------------------------------------ */
size_t dsp_schedule_windows_workspace_size(int32_t R, int32_t K);
int32_t dsp_schedule_windows(const float* conf, int32_t R, int32_t K, const double* cost,
                             int32_t n_cost, int32_t mode, int32_t max_tokens, double threshold,
                             int32_t* windows, double* survival, double* stats,
                             void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Ragged pack  ([S] "Ragged verify")                                         */
/*                                                                          */
/* Request i contributes its anchor then its first windows[i] drafts, front  */
/* packed in request order: cu_seqlens[0] = 0,                               */
/* cu_seqlens[i+1] = cu_seqlens[i] + windows[i] + 1; tokens[cu_seqlens[i]+k] */
/* is the anchor (k = 0) or drafts[i*ld_drafts + k-1]; row_req / row_pos give */
/* (i, k) for every packed row. total_and_tier[0] = T = cu_seqlens[R];       */
/* total_and_tier[1] = the smallest tiers[t] >= T (tiers ascending, host      */
/* NULL / n_tiers = 0: T itself; -1 if none is large enough).                */
/* Buffers tokens/row_req/row_pos hold R*(K+1) entries; entries >= T are     */
/* left untouched. windows outside [0, K] set DSP_STATUS_WINDOW_RANGE.       */
/* Limits: 1 <= R <= 65536, 1 <= K <= 4096, n_tiers <= 64.                   */
/* ------------------------------------------------------------------------ */
int32_t dsp_pack_ragged(const int32_t* windows, const int32_t* anchors, const int32_t* drafts,
                        int64_t ld_drafts, int32_t R, int32_t K, const int32_t* tiers_host,
                        int32_t n_tiers, int32_t* cu_seqlens, int32_t* tokens, int32_t* row_req,
                        int32_t* row_pos, int32_t* total_and_tier, int32_t* status, void* stream);

/* ------------------------------------------------------------------------ */
/* Window selection and ragged pack in one call  ([N] 5.2; [S] "Ragged       */
/* verify")                                                                  */
/*                                                                          */
/* Exactly dsp_schedule_windows followed by dsp_pack_ragged on the windows    */
/* it wrote (same arguments, same outputs, bit for bit), with the pack run by */
/* the selection's own workgroup: one launch fewer between the scheduler and */
/* the verify. Limits and workspace: those of dsp_schedule_windows (which    */
/* are within the pack's).                                                   */
/* ------------------------------------------------------------------------ */
int32_t dsp_schedule_pack(const float* conf, int32_t R, int32_t K, const double* cost,
                          int32_t n_cost, int32_t mode, int32_t max_tokens, double threshold,
                          int32_t* windows, double* survival, double* stats,
                          const int32_t* anchors, const int32_t* drafts, int64_t ld_drafts,
                          const int32_t* tiers_host, int32_t n_tiers, int32_t* cu_seqlens,
                          int32_t* tokens, int32_t* row_req, int32_t* row_pos,
                          int32_t* total_and_tier, int32_t* status, void* ws, size_t ws_bytes,
                          void* stream);

/* ------------------------------------------------------------------------ */
/* Batched ragged verify  ([N] 1, 3 / Figure 1; [S] "three verify modes",     */
/* "Ragged verify"; [P] greedy tree verification)                            */
/*                                                                          */
/* Target logits are PACKED: request i owns rows cu_seqlens[i] ..            */
/* cu_seqlens[i+1]-1 of tgt; row cu_seqlens[i] + k predicts draft position   */
/* k+1. Its window is n_i = cu_seqlens[i+1] - cu_seqlens[i] - 1 (0..K).       */
/* Draft logits are dense: position k (1-based) of request i is row           */
/* drf + i*ld_d_r + (k-1)*ld_d_k. Draft tokens x_{i,k} at                    */
/* draft_tok[i*ld_x + k-1].                                                  */
/*                                                                          */
/* Chain mode (parent == NULL), temperature T > 0: for k = 1..n_i,            */
/* p_k = softmax(t_{k-1}/T), q_k = softmax(d_k/T); accept x_k iff             */
/* u_k < p_k(x_k)/q_k(x_k), left to right; at the first rejection the token  */
/* is drawn from norm(max(0, p_k - q_k)) with u'_k by inverse CDF over        */
/* ascending token id; if all n_i are accepted the bonus is drawn from        */
/* p_{n_i+1} with u'_{n_i+1}. u_k, u'_k: Philox4x64-10, key (seed, 0),        */
/* counter (round, req_id[i] or i, k, 0), words 0 and 1. round_dev (device,  */
/* nullable, in/out) replaces `round` with a device counter: each sampled call */
/* increments *round_dev once and uses the new value, so the replays of a     */
/* captured HIP graph draw fresh uniforms without any host update.           */
/* T == 0: greedy; x_k accepted iff it equals argmax t_{k-1} (lowest id on    */
/* ties), the stop token is that argmax; drf may be NULL.                     */
/* Tree mode (parent != NULL, T must be 0): draft_tok / parent are the        */
/* node tokens and parent indices [R, K] (-1 = root, parent[j] < j) of up to  */
/* K nodes; request i owns rows cu_seqlens[i] (root) and cu_seqlens[i]+1+j    */
/* (node j), n_nodes_i = cu_seqlens[i+1]-cu_seqlens[i]-1. From the root, move */
/* to the child whose token equals argmax of the current row; the bonus is    */
/* that argmax where no child matches.                                       */
/*                                                                          */
/* Outputs (device):                                                         */
/*   accepted_len [R] int32    accepted drafts (-1 if the request faulted)    */
/*   out_tokens [R, K+1] int32 accepted drafts then the corrected / bonus     */
/*                             token; -1 after it                            */
/*   stop_pos [R] int32        chain: position of the sampled token           */
/*                             (accepted_len + 1); tree: last accepted node   */
/*                             (-1 = root)                                   */
/*   p_x, q_x [R, K] float32   (nullable; chain, T > 0) p_k(x_k), q_k(x_k)    */
/*                             for every window position, 0 elsewhere        */
/* row_req, row_pos (nullable, together): the request and position of every  */
/* packed row, as written by dsp_pack_ragged (min(max_rows, R*(K+1)) entries */
/* each, read whether or not the row is below the packed total, so both must */
/* be that long); when given, draft rows are                                 */
/* located from them instead of by searching cu_seqlens (a row whose maps do */
/* not match cu_seqlens falls back to the search).                           */
/* cap (nullable, chain only): cap-accept commit windows [R] int32 ([S]       */
/* "three verify modes"): the decisions cover the whole packed window n_i,    */
/* but only the first c_i = min(max(cap_i, 0), n_i) positions are committed:  */
/* a rejection at k <= c_i stops there; otherwise the c_i drafts are kept and */
/* the bonus is drawn from p_{c_i+1} with the uniform of position c_i + 1 --  */
/* the result of verifying the window c_i alone (compact).                    */
/* ceiling (nullable, chain only): [R] int32, drafts accepted over the whole  */
/* packed window (the acceptance ceiling that trimming hides, [S]).           */
/* max_rows: host-known bound on cu_seqlens[R] (0 = R*(K+1)); tgt must hold    */
/* at least that many rows. Rows past min(cu_seqlens[R], max_rows) are never  */
/* read, and a request whose rows end past max_rows is a window fault.        */
/* Limits: 1 <= K <= 64, 1 <= V < 2^29 (rows under 2 GiB), ld >= V.         */
/* ------------------------------------------------------------------------ */
size_t dsp_verify_rejection_workspace_size(int32_t R, int32_t K, int32_t V, int32_t max_rows,
                                           int32_t t_dtype, int32_t d_dtype);
int32_t dsp_verify_rejection(const void* tgt, int32_t t_dtype, int64_t ld_t,
                             const int32_t* cu_seqlens,
                             const void* drf, int32_t d_dtype, int64_t ld_d_r, int64_t ld_d_k,
                             const int32_t* draft_tok, int64_t ld_x, const int32_t* parent,
                             int32_t R, int32_t K, int32_t V, int32_t max_rows,
                             float temperature, uint64_t seed, uint64_t round,
                             uint64_t* round_dev, const int64_t* req_id,
                             const int32_t* row_req, const int32_t* row_pos,
                             const int32_t* cap, int32_t* ceiling,
                             int32_t* accepted_len, int32_t* out_tokens, int32_t* stop_pos,
                             float* p_x, float* q_x, int32_t* status,
                             void* ws, size_t ws_bytes, void* stream);

/* The same verify for callers that cannot allocate device memory (code      */
/* under HIP graph capture, tight serving loops, harnesses that forbid       */
/* hipMalloc): no workspace argument and no allocation of any kind. The      */
/* scratch space is a fixed 8 MiB device array inside the library, one per  */
/* GPU it runs on, held until the process ends; a batch whose               */
/* dsp_verify_rejection_workspace_size exceeds 8 MiB is rejected with         */
/* DSP_ERR_WORKSPACE before anything is launched. The first call on a device */
/* looks the array's address up (hipGetSymbolAddress) with that device       */
/* current. Every call on one GPU shares that array: calls that overlap on  */
/* one GPU (different streams, concurrent threads) race and must not be     */
/* issued. Nothing needs clearing between calls (every entry a call reads,  */
/* that call wrote first). Arguments, outputs and errors as dsp_verify_rejection. */
int32_t dsp_verify_rejection_noalloc(const void* tgt, int32_t t_dtype, int64_t ld_t,
                                     const int32_t* cu_seqlens,
                                     const void* drf, int32_t d_dtype, int64_t ld_d_r, int64_t ld_d_k,
                                     const int32_t* draft_tok, int64_t ld_x, const int32_t* parent,
                                     int32_t R, int32_t K, int32_t V, int32_t max_rows,
                                     float temperature, uint64_t seed, uint64_t round,
                                     uint64_t* round_dev, const int64_t* req_id,
                                     const int32_t* row_req, const int32_t* row_pos,
                                     const int32_t* cap, int32_t* ceiling,
                                     int32_t* accepted_len, int32_t* out_tokens, int32_t* stop_pos,
                                     float* p_x, float* q_x, int32_t* status, void* stream);

/* ------------------------------------------------------------------------ */
/* Markov-head sequential stage, greedy chain  ([N] 4; [P] z_d = L_d +        */
/* Markov(y_{d-1}))                                                          */
/*                                                                          */
/* For d = 1..n_steps and every request i:                                   */
/*   z_d = L[i, d-1, :] + U[y_{d-1}, :] . W,   y_d = argmax_v z_d (fp32 z,    */
/*   lowest id on ties),  y_0 = prev_tok[i];                                  */
/*   logq[i, d-1] = z_d[y_d] - logsumexp(z_d)  (if logq != NULL).             */
/* L: bf16. l_dtype DSP_BF16: element (i, d, v) at L + i*ldL_r + d*ldL_d + v */
/*    (ldL_d >= V). l_dtype DSP_BF16_TOKEN_MAJOR: element (i, d, v) at       */
/*    L + i + d*ldL_d + v*ldL_r, i.e. ldL_r is the stride between tokens     */
/*    (ldL_r >= R, ldL_d >= (V-1)*ldL_r + R; a [B, V, R] buffer); it needs    */
/*    rank 256, R a multiple of 8, a 16-byte aligned L and both strides      */
/*    multiples of 8 (else DSP_ERR_UNSUPPORTED / _SHAPE / _ALIGN). Same       */
/*    results either way; the token-major tile of a step is one contiguous   */
/*    read per 32 tokens.                                                    */
/* U: bf16 [V, rank] row-major (row y = the first factor's row of token y).   */
/* Wt: bf16 [V, rank] row-major = the second factor W [rank, V] stored        */
/*     vocab-major (Wt[v*rank + j] = W[j][v]).                               */
/* y [R, n_steps] int32 with row stride ld_y; logq float32 same layout.       */
/* Limits: rank % 32 == 0, 32 <= rank <= 512, 1 <= n_steps, V >= 1.          */
/* ------------------------------------------------------------------------ */
size_t dsp_draft_markov_step_workspace_size(int32_t R, int32_t V, int32_t rank, int32_t n_steps,
                                            int32_t want_logq);
int32_t dsp_draft_markov_step(const void* L, int32_t l_dtype, int64_t ldL_r, int64_t ldL_d,
                              const void* U, const void* Wt, int32_t V, int32_t rank,
                              const int32_t* prev_tok, int32_t R, int32_t n_steps,
                              int32_t* y, int64_t ld_y, float* logq, int32_t* status,
                              void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Markov-head sequential stage, sampled chain  ([N] 1, 4; [S] "Ragged       */
/* verify": the draft side of the draft -> schedule -> pack -> verify cycle) */
/*                                                                          */
/* For d = 1..n_steps and every request i:                                   */
/*   z_d = L[i, d-1, :] + U[y_{d-1}, :] . W (fp32), y_0 = prev_tok[i];         */
/*   zh_d = bf16(z_d), round to nearest even, written to                     */
/*          z[i*ldz_r + (d-1)*ldz_d + v] (these rows are the draft logits    */
/*          that dsp_verify_rejection takes as drf, so q there is exactly the */
/*          law the token was drawn from);                                   */
/*   q_d = softmax(zh_d / T);  y_d = smallest v with                         */
/*          sum_{w<=v} q_d(w) > u_d (inverse CDF over ascending token ids;   */
/*          the last token with mass if rounding leaves none);              */
/*   logq[i, d-1] = log q_d(y_d) (if logq != NULL).                          */
/* u_d: Philox4x64-10, key (seed, 0), counter (round, req_id[i] or i, d, 1),  */
/* word 0 mapped to [0, 1) as (w >> 11) * 2^-53; stream 1 keeps the draft's   */
/* draws apart from the verify step's (stream 0). round_dev (device,         */
/* nullable) replaces `round` with *round_dev, read and not advanced (the    */
/* verify call advances it), so a captured cycle draws fresh uniforms.       */
/* L (either layout), U, Wt as dsp_draft_markov_step; z: bf16, 16-byte       */
/* aligned, ldz_d and                                                       */
/* ldz_r multiples of 8 elements, ldz_d >= V; y and logq [R, n_steps] with   */
/* row stride ld_y. temperature must be finite and > 0 (the greedy chain is  */
/* dsp_draft_markov_step). A row whose mass is not finite sets               */
/* DSP_STATUS_NONFINITE and writes y = -1.                                   */
/* ------------------------------------------------------------------------ */
size_t dsp_draft_markov_sample_workspace_size(int32_t R, int32_t V, int32_t rank, int32_t n_steps);
int32_t dsp_draft_markov_sample(const void* L, int32_t l_dtype, int64_t ldL_r, int64_t ldL_d,
                                const void* U, const void* Wt, int32_t V, int32_t rank,
                                const int32_t* prev_tok, int32_t R, int32_t n_steps, float temperature,
                                uint64_t seed, uint64_t round, const uint64_t* round_dev,
                                const int64_t* req_id, int32_t* y, int64_t ld_y, float* logq, void* z,
                                int64_t ldz_r, int64_t ldz_d, int32_t* status, void* ws, size_t ws_bytes,
                                void* stream);

/* ------------------------------------------------------------------------ */
/* RNN sequential head, greedy chain  ([N] 4, "RNN head": a memo that holds  */
/* the whole draft so far, updated once per position from the previous     */
/* memo, the previous token and the current backbone state; its correction  */
/* is added to the base logits as the Markov head's is)                     */
/*                                                                          */
/* s_0 = 0; for d = 1..n_steps, with y_0 = prev_tok[i]:                      */
/*   s_d = tanh(s_{d-1} A + E[y_{d-1}] + h_d G + bias)      (fp64, r entries) */
/*   z_d = L[i, d-1, :] + bf16(s_d) . W_o                   (MFMA, fp32 acc)  */
/*   y_d = argmax z_d (lowest id on ties of the fp32 values), logq as the    */
/*   Markov step. bf16(.) rounds to nearest, ties to even, from fp64.        */
/* h: bf16 backbone states, element (i, d, k) at h + i*ldh_r + d*ldh_k + k    */
/* (k < H). Gt: bf16 [r, H] (G transposed: memo entry j's weights over the  */
/* state contiguous); A: bf16 [r, r] row-major (s A); E: bf16 [V, r] token  */
/* table (16-byte aligned); bias: fp32 [r] or NULL; Wot: bf16 [V, r] (W_o   */
/* stored vocab-major, as Wt). L, y, logq, status as dsp_draft_markov_step. */
/* The state projection h G for every position is computed first, in fp64  */
/* (exact products, fp64 sums): it costs 2*R*n*H*r flops on the fp64 units. */
/* A previous token outside [0, V) sets DSP_STATUS_TOKEN_RANGE.             */
/* Limits: rank a multiple of 32 in [32, 512], H >= 1.                      */
/* ------------------------------------------------------------------------ */
size_t dsp_draft_rnn_step_workspace_size(int32_t R, int32_t V, int32_t rank, int32_t n_steps);
int32_t dsp_draft_rnn_step(const void* L, int32_t l_dtype, int64_t ldL_r, int64_t ldL_d,
                           const void* h, int32_t h_dtype, int64_t ldh_r, int64_t ldh_k, int32_t H,
                           const void* Gt, const void* A, const void* E, const float* bias,
                           const void* Wot, int32_t V, int32_t rank, const int32_t* prev_tok,
                           int32_t R, int32_t n_steps, int32_t* y, int64_t ld_y, float* logq,
                           int32_t* status, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* PCTree expansion  ([P] "the chain becomes a tree")                         */
/*                                                                          */
/* Per request, root = anchor with score 0. For depth d = 1..D and every      */
/* parent p of frontier F_{d-1}: z = L[i, d-1, :] + U[tok(p)] . W (one batched */
/* Markov call for all parents); children = top-k tokens by (z desc, id asc),*/
/* decided on fp32 z (ties within its rounding may go either way); child     */
/* score s = s(p) + z_v - logsumexp(z) (fp64). F_d = top-F                   */
/* children by (s desc, parent slot asc, child rank asc). The tree is the     */
/* top-N of all frontier nodes of all depths by (s desc, depth asc, slot asc),*/
/* parents re-indexed into that order (parent[j] < j, -1 = root).             */
/* Outputs [R, topN] (row stride topN): node_token, node_parent, node_depth   */
/* (int32), node_score (fp64); n_nodes [R] = nodes written (rest: -1 / 0).    */
/* anc_mask (nullable): [R, topN, W] uint64, W = ceil(topN / 64): bit (j % 64) */
/* of word j / 64 of node o is set iff node j is o or an ancestor of o (the   */
/* root is implicit) -- the tree-causal attention pattern of the target      */
/* forward that verifies the tree ([P]); rows past n_nodes are zero.         */
/* U, Wt layouts as dsp_draft_markov_step; L row-major only (l_dtype          */
/* DSP_BF16, ldL_d >= V; else DSP_ERR_UNSUPPORTED).                          */
/* The selection reads each base-logit row once more up front (R*(D-1) rows) */
/* to bound every parent row's 4th-largest z from below; entries under the   */
/* bound cannot be among the top 4, so the outputs do not depend on it.      */
/* A parent row with fewer than topk entries above -2^127 (masked -inf base  */
/* logits count as absent), or with a +inf or NaN base logit, sets            */
/* DSP_STATUS_NONFINITE; its children are then unspecified.                  */
/* Limits: 1 <= topk <= min(4, V), 1 <= frontier <= 64, topk*frontier <= 256,  */
/* 1 <= topN <= 1024, D*frontier <= 1024, rank as above.                      */
/* ------------------------------------------------------------------------ */
size_t dsp_tree_expand_workspace_size(int32_t R, int32_t D, int32_t V, int32_t rank,
                                      int32_t topk, int32_t frontier, int32_t topN);
int32_t dsp_tree_expand(const void* L, int32_t l_dtype, int64_t ldL_r, int64_t ldL_d,
                        const void* U, const void* Wt, int32_t V, int32_t rank,
                        const int32_t* anchor, int32_t R, int32_t D, int32_t topk,
                        int32_t frontier, int32_t topN,
                        int32_t* node_token, int32_t* node_parent, int32_t* node_depth,
                        double* node_score, int32_t* n_nodes, uint64_t* anc_mask, int32_t* status,
                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Calibration of the confidences against a verify  ([S] observability:     */
/* per-request confidences and calibration metrics such as ECE beside the   */
/* acceptance ceiling; [N] 5.1: c[i,k] is the probability that position k   */
/* survives given every earlier position was accepted)                      */
/*                                                                          */
/* conf [R, K] fp32 (row stride ld_conf >= K): the confidences the scheduler */
/* used; cu_seqlens [R+1]: the verify's packing (window n_i = cu[i+1] -     */
/* cu[i] - 1); decided [R]: drafts accepted over the decided window -- the  */
/* verify's accepted_len, or its ceiling under cap-accept (-1 = a faulted   */
/* request: nothing observed). Positions 1..m_i are accepted (outcome 1),   */
/* position m_i + 1 <= n_i is the first rejection (outcome 0), later ones   */
/* were never decided. With n_bins equal-width bins of [0, 1] (bin          */
/* floor(c * n_bins) in fp64, clamped to the range):                        */
/*   ECE = (1/n) sum_b | sum over bin b of (outcome - c) |  (fp64)          */
/* = sum_b (n_b/n) |mean outcome - mean c|, 0 when nothing was observed.    */
/* Outputs (device): ece [R] and n_obs [R] per request; batch [1 + 3*n_bins]*/
/* = batch ECE over every observed position, then per bin the count, the   */
/* sum of c and the sum of outcomes. Deterministic (fixed reduction order). */
/* Limits: R >= 1, 1 <= K <= 64, 1 <= n_bins <= 64. One workgroup.          */
/* ------------------------------------------------------------------------ */
int32_t dsp_verify_calibration(const float* conf, int64_t ld_conf, const int32_t* cu_seqlens,
                               const int32_t* decided, int32_t R, int32_t K, int32_t n_bins,
                               double* ece, int32_t* n_obs, double* batch, void* stream);

/* ------------------------------------------------------------------------ */
/* Read probe (measurement).                                                 */
/*                                                                          */
/* Streams `bytes` (a multiple of 16) from the 16-byte aligned device buffer */
/* p with plain 16-byte loads, eight in flight per thread (*sink, device, is */
/* written only for one data-dependent value, so the loads stay live): the  */
/* achievable read rate of the same buffers the streaming kernels read, a    */
/* second denominator beside the HBM peak.                                   */
/* ------------------------------------------------------------------------ */
int32_t dsp_stream_read(const void* p, size_t bytes, uint32_t* sink, void* stream);

/* ------------------------------------------------------------------------ */
/* Kernel timing (observability).                                            */
/*                                                                          */
/* dsp_prof_enable(mask): bit k set = time each launch of kernel k below     */
/* with a start/stop HIP event pair attached to the kernel's own dispatch on */
/* its launch stream (hipExtLaunchKernelGGL), so the interval is the kernel's */
/* execution, not host launch gaps (mask 0 = off, -1 = all).                 */
/* dsp_prof_query synchronises on the recorded events and returns the summed */
/* duration and launch count since the last reset. Not thread safe, and not  */
/* to be used while a stream is being captured into a graph.                 */
/* ------------------------------------------------------------------------ */
#define DSP_K_VERIFY_STATS     0  /* row statistics / arg-max streaming pass */
#define DSP_K_VERIFY_DECIDE    1  /* accept/reject decisions; greedy matching; tree walk */
#define DSP_K_VERIFY_RESIDUAL  2  /* sampled: per-chunk mass of the residual / bonus row */
#define DSP_K_VERIFY_SAMPLE    3  /* sampled: inverse-CDF draw of the correction token */
#define DSP_K_SCHEDULE         4  /* scheduler: prefix sums, throughput test, windows */
#define DSP_K_PACK             5
#define DSP_K_MARKOV_GEMM      6
#define DSP_K_MARKOV_MERGE     7  /* chain merge (and the persistent chain's key reset) */
#define DSP_K_TREE_GEMM        8
#define DSP_K_TREE_MERGE       9
#define DSP_K_TREE_FINAL      10
#define DSP_K_SCHEDULE_RANK   11  /* scheduler: ranking of the candidate keys */
#define DSP_K_CONFIDENCE      12  /* confidence head */
#define DSP_K_TREE_PROBE      13  /* PCTree: probe tokens of the base-logit rows */
#define DSP_K_CALIBRATION     14  /* calibration of the confidences against the verify */
#define DSP_K_RNN_MEMO        15  /* RNN head: memo update */
#define DSP_K_RNN_PROJ        16  /* RNN head: projection of the backbone states */
#define DSP_K_CHAIN_PERSIST   17  /* greedy chain: all steps in one persistent launch */
#define DSP_K_COUNT           18
int32_t dsp_prof_enable(int32_t mask);
int32_t dsp_prof_reset(void);
int32_t dsp_prof_query(int32_t kernel, double* total_ms, int64_t* launches);

/* ------------------------------------------------------------------------ */
/* Library options (process-wide; for tests and diagnostics).               */
/*                                                                          */
/* DSP_OPT_CHAIN_PERSISTENT: 1 lets dsp_draft_markov_step run all steps in  */
/*   one persistent launch where that path applies (see there); 0 (default) */
/*   keeps one launch per step, which measures faster on gfx950. Tokens are  */
/*   identical either way; log q agrees to fp32 rounding.                    */
/* DSP_OPT_SPIN_LIMIT: polls a persistent launch's grid barrier makes before */
/*   it gives up and sets DSP_STATUS_TIMEOUT (default 2^20, about a second); */
/*   0 makes every wait that is not already satisfied give up at once.       */
/* DSP_OPT_TREE_SPLIT: 1 (default) lets dsp_tree_expand run its depths whose */
/*   row blocks of 256 parents span at most 16 requests (rank <= 256,        */
/*   16-byte aligned L) on the GEMM with direct-to-LDS stages and a fixed    */
/*   issue order; 0 keeps the general GEMM for every depth. Both compute the */
/*   same sums in the same order: outputs are bit-identical.                 */
/* DSP_OPT_CHAIN_SCHED: 1 lets the greedy chain's and the RNN head's       */
/*   arg-max steps (no log q, rank <= 256, 16-byte aligned row-major L) run  */
/*   on the GEMM with direct-to-LDS stages and a fixed issue order; 0        */
/*   (default) keeps the general GEMM, which measures as fast or faster on   */
/*   gfx950. Outputs are bit-identical.                                      */
/* Returns DSP_ERR_SHAPE for an unknown option or a negative value. Not      */
/* thread safe; set before issuing work.                                     */
/* ------------------------------------------------------------------------ */
#define DSP_OPT_CHAIN_PERSISTENT  0
#define DSP_OPT_SPIN_LIMIT        1
#define DSP_OPT_TREE_SPLIT        2
#define DSP_OPT_CHAIN_SCHED       3
int32_t dsp_set_option(int32_t option, int64_t value);

#ifdef __cplusplus
}
#endif

#endif /* DSP_H */
