/*
 * lvtv -- speculative-sampling verify and E2E-TV loss on AMD MI355X (gfx950).
 *
 * C ABI. Plain pointers and sizes only. Every pointer argument except the
 * workspace-size queries is a DEVICE pointer on the current HIP device;
 * `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *
 * Ownership: the caller owns every buffer, the workspace included. The
 * library never allocates, frees or keeps device memory between calls and
 * never synchronises the stream. All work is enqueued on `stream` in order;
 * outputs are valid once the caller's later work on that stream (or an
 * event recorded after the call) has completed. One workspace serves one
 * call at a time: calls that share a workspace must be ordered on one
 * stream.
 *
 * Errors: a call returns LVTV_OK (0) or a negative code. A negative code
 * means nothing was enqueued and no output was written (host-checkable
 * errors: null pointers, bad sizes, unknown dtype, too small a workspace),
 * except LVTV_ERR_LAUNCH, returned when the HIP runtime rejects a launch.
 * Faults that live in device memory (per-request K, token ids,
 * temperatures, non-finite logits) cannot be checked on the host without a
 * sync; spec_verify reports them per request in `status` instead.
 *
 * Alignment: any element-aligned pointer is accepted. Rows that start on a
 * 16-byte boundary (a 16-byte-aligned base and V a multiple of 8) are read
 * with aligned 16-byte loads; other rows with unaligned ones, which gives
 * the same outputs and costs about 15 % (loss) to 30 % (verify) more time.
 *
 * Sources, cited by page title and section:
 *   "Reading Qwen Bebop and DeepSeek DSpark" (lilfry09.github.io), section
 *     "Formulas: what makes a guess worth it" (eqs. alpha(y), alpha_RS,
 *     d_TV, P(tau >= j), E[tau]) and section "Bebop's solution" (TV loss,
 *     end-to-end TV loss).
 *   "SpecOPD: Branch-Parallel On-Policy Distillation for Speculative
 *     Decoding" (paper.rainbus.top summary), prerequisite "Acceptance length
 *     and the E2E-TV objective" and method step (6).
 *   "Speculative Decoding and MTP" survey (papers-3lj.pages.dev), sections 2
 *     (draft/target loop), 3 (probabilistic correctness), 4 (greedy versus
 *     sampling), 21 (fuse acceptance and residual sampling on the GPU to
 *     avoid a CPU sync per cycle).
 */
#ifndef LVTV_H
#define LVTV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Logit storage types. */
#define LVTV_F32 0  /* IEEE binary32                                  */
#define LVTV_BF16 1 /* bfloat16 bit patterns in uint16 (top half of binary32) */

/* Return codes. */
#define LVTV_OK 0
#define LVTV_ERR_NULL (-1)      /* a required pointer is NULL            */
#define LVTV_ERR_SHAPE (-2)     /* a size is out of the supported range  */
#define LVTV_ERR_DTYPE (-3)     /* unknown dtype                         */
#define LVTV_ERR_WORKSPACE (-4) /* workspace NULL or smaller than queried */
#define LVTV_ERR_LAUNCH (-5)    /* the HIP runtime rejected a launch     */
#define LVTV_ERR_OBJECTIVE (-6) /* unknown loss objective                */
#define LVTV_ERR_TEMPERATURE (-7) /* loss temperature not finite and > 0 */
#define LVTV_ERR_OPTION (-8)    /* unknown debug option (lvtv_debug_draft_loss) */
#define LVTV_ERR_SCRATCH (-9)   /* sizes need more than spec_verify_noalloc's scratch */

/* Objectives of draft_loss_fwd_bwd, each summed over a branch's W positions
 * and averaged over the N branches. */
#define LVTV_OBJ_E2E_TV 0  /* -sum_j prod_{k<=j} alpha_k (e2e_tv_loss_fwd_bwd) */
#define LVTV_OBJ_STEP_TV 1 /* sum_j (1 - alpha_j), the per-step TV loss      */
#define LVTV_OBJ_CE 2      /* sum_j -sum_v p log q, cross-entropy            */
#define LVTV_OBJ_KL 3      /* sum_j sum_v p log(p / q), KL(p || q)           */

/* Supported ranges. */
#define LVTV_MAX_K 16         /* draft positions per request (Kmax)      */
#define LVTV_MAX_W 16         /* positions per branch (W)                */
#define LVTV_MAX_V (1 << 27)  /* vocabulary size                         */
#define LVTV_MAX_B 65535      /* requests per verify call (B)            */
#define LVTV_MAX_N 65535      /* branches per loss call (N)              */

/* Per-request status bits written by spec_verify. */
#define LVTV_STATUS_BAD_K 1           /* K_b outside [0, Kmax]                 */
#define LVTV_STATUS_BAD_TOKEN 2       /* a draft token (k < K_b) outside [0,V) */
#define LVTV_STATUS_BAD_TEMPERATURE 4 /* T_b negative, NaN or infinite         */
#define LVTV_STATUS_NONFINITE 8       /* a used row holds NaN or +inf, or is
                                         entirely -inf (after scaling)         */
#define LVTV_STATUS_BAD_TRUNCATION 16 /* top_p_b NaN or <= 0 (spec_verify_topkp) */

int lvtv_version(void);
const char* lvtv_strerror(int code);

/*
 * Zero-fill a workspace on `stream` (a plain fill kernel, so it may sit in a
 * captured graph). A utility only: no call depends on a workspace's
 * contents on entry. Returns LVTV_ERR_NULL / LVTV_ERR_WORKSPACE (misaligned)
 * before enqueueing anything.
 */
int lvtv_workspace_reset(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes spec_verify needs for these sizes (0 if the sizes are out
 * of range). Host function; no HIP call.
 */
size_t spec_verify_workspace_bytes(int32_t B, int32_t Kmax, int32_t V, int dtype);

/*
 * spec_verify -- one verify step for B requests.
 *
 * What it computes, per request b with K_b draft positions:
 *   * scaled logits s = fl32(x * fl32(1/T_b)), the same transform for target
 *     and draft (survey, section 4); p_k = softmax(s_target[b,k]) for
 *     k <= K_b, q_k = softmax(s_draft[b,k]) for k < K_b;
 *   * overlap alpha_k = sum_v min(p_k, q_k) = 1 - d_TV(p_k, q_k) for every
 *     k < K_b ("Formulas", eq. alpha_RS);
 *   * the accept scan: draft token y_k is accepted iff u_k < p_k(y_k)/q_k(y_k)
 *     (acceptance probability min(1, p/q), "Formulas", eq. alpha(y)), in
 *     order, up to the first rejection j (survey, section 2);
 *   * the correction token drawn from max(0, p_j - q_j)/Z_j if j < K_b
 *     (survey, section 3), or the bonus token drawn from p_{K_b} if every
 *     draft was accepted (survey, section 2); draws are inverse-CDF in
 *     ascending token id;
 *   * at T_b = 0 the greedy rule (survey, section 4): accept while y_k is
 *     the target argmax (lowest index among ties), emit the target argmax at
 *     the first mismatch or as the bonus; alpha_k = [argmax t == argmax d].
 * Randomness: Philox4x64-10 (Salmon et al., SC'11) with key (seed_b, 0) and
 * counter (b, k, 0, 0); u_k = (word0 >> 40) * 2^-24 for the accept test at
 * position k, u'_k = (word1 >> 40) * 2^-24 for a draw at position k. No
 * per-call state: a call is a pure function of its inputs.
 *
 * Arguments (device pointers; row-major, V contiguous):
 *   target_logits  [B, Kmax+1, V] of `dtype`; rows k > K_b are not read.
 *   draft_logits   [B, Kmax,   V] of `dtype`; rows k >= K_b are not read.
 *   dtype          LVTV_F32 or LVTV_BF16.
 *   draft_tokens   int32 [B, Kmax]; entries k >= K_b are not read.
 *   k_per_req      int32 [B], K_b in 0..Kmax (0 = one token sampled from p_0).
 *   temperature    float [B]; 0 = greedy, > 0 stochastic.
 *   seed           uint64 [B], Philox key word 0 for request b.
 *   B, Kmax, V     1 <= B <= LVTV_MAX_B, 0 <= Kmax <= LVTV_MAX_K,
 *                  1 <= V <= LVTV_MAX_V (else LVTV_ERR_SHAPE, and the workspace
 *                  query returns 0).
 *   accepted_len   int32 [B] out: j (number of accepted drafts), -1 if faulted.
 *   out_tokens     int32 [B, Kmax+1] out: y_0..y_{j-1}, the drawn token, then -1.
 *   alpha          float [B, Kmax] out: alpha_k for k < K_b, 0 otherwise.
 *   status         int32 [B] out: LVTV_STATUS_* bits, 0 if fine. A faulted
 *                  request gets accepted_len = -1, all tokens -1, alpha 0.
 *   workspace      device scratch of >= spec_verify_workspace_bytes(...)
 *                  bytes, 256-byte aligned. Its contents on entry do not
 *                  matter (every value a call reads from it, the call wrote
 *                  first). Calls sharing a workspace must be ordered on one
 *                  stream.
 *   stream         hipStream_t. Two kernels are enqueued: one workgroup per
 *                  used (request, position) row pair, then one per request.
 */
int spec_verify(const void* target_logits, const void* draft_logits, int dtype,
                const int32_t* draft_tokens, const int32_t* k_per_req,
                const float* temperature, const uint64_t* seed, int32_t B,
                int32_t Kmax, int32_t V, int32_t* accepted_len,
                int32_t* out_tokens, float* alpha, int32_t* status,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_noalloc -- spec_verify for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. It takes no workspace: the scratch lives in a static
 * device array of LVTV_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held until the process ends. The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine); the first call on a device looks
 * the array's address up once (hipGetSymbolAddress) with that device current.
 *
 * Arguments, results and errors as spec_verify, without workspace and
 * workspace_bytes; sizes whose spec_verify workspace would exceed the scratch
 * (spec_verify_workspace_bytes(B, Kmax, V, dtype) > LVTV_NOALLOC_SCRATCH_BYTES)
 * return LVTV_ERR_SCRATCH before enqueueing anything, and LVTV_ERR_LAUNCH is
 * also returned if the address lookup fails. Every call on one GPU shares
 * that GPU's array, which keeps the last call's contents (no call depends on
 * them): calls that overlap on one GPU (on different streams, or from several
 * threads without ordering) race and give undefined results; order them on
 * one stream.
 */
#define LVTV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int spec_verify_noalloc(const void* target_logits, const void* draft_logits, int dtype,
                        const int32_t* draft_tokens, const int32_t* k_per_req,
                        const float* temperature, const uint64_t* seed, int32_t B,
                        int32_t Kmax, int32_t V, int32_t* accepted_len,
                        int32_t* out_tokens, float* alpha, int32_t* status, void* stream);

/*
 * Workspace bytes spec_verify_packed needs (0 if out of range). Host only.
 */
size_t spec_verify_packed_workspace_bytes(int32_t B, int32_t total_rows, int32_t V,
                                          int dtype);

/*
 * spec_verify_packed -- spec_verify on a packed, variable-length layout:
 * each request's rows are stored back to back with no padding for a ragged
 * K ("Reading Qwen Bebop and DeepSeek DSpark", "DSpark's second piece":
 * every request gets its own verify length).
 *
 * Layout (device pointers; rows V contiguous):
 *   B              1 <= B <= LVTV_MAX_B; B <= total_rows <= B (LVTV_MAX_K + 1).
 *   row_offsets    int32 [B + 1]: request b owns the target rows
 *                  [row_offsets[b], row_offsets[b+1]), so
 *                  K_b = row_offsets[b+1] - row_offsets[b] - 1 (0..LVTV_MAX_K);
 *                  row_offsets[0] = 0 and row_offsets[B] = total_rows.
 *   target_logits  [total_rows, V] of `dtype`.
 *   draft_logits   [total_rows - B, V]: request b's draft rows start at
 *                  row_offsets[b] - b (K_b of them).
 *   draft_tokens   int32 [total_rows - B], packed like the draft rows.
 *   accepted_len   int32 [B] out.
 *   out_tokens     int32 [total_rows] out: request b's K_b + 1 slots at
 *                  row_offsets[b] (accepted drafts, the drawn token, then -1).
 *   alpha          float [total_rows - B] out, packed like the draft rows.
 *   temperature, seed, status, workspace, stream: as spec_verify (Philox
 *                  counters use the request index b and the position k, so a
 *                  request gives the same result in either layout).
 * Offsets that break the rules above fault every request
 * (LVTV_STATUS_BAD_K, accepted_len -1) and no out_tokens or alpha slot is
 * written. Three kernels are enqueued: one workgroup maps rows to requests
 * and checks the offsets, then the row and finalize kernels of spec_verify.
 */
int spec_verify_packed(const void* target_logits, const void* draft_logits, int dtype,
                       const int32_t* draft_tokens, const int32_t* row_offsets,
                       const float* temperature, const uint64_t* seed, int32_t B,
                       int32_t total_rows, int32_t V, int32_t* accepted_len,
                       int32_t* out_tokens, float* alpha, int32_t* status,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes spec_verify_topkp needs (0 if out of range). Host only.
 */
size_t spec_verify_topkp_workspace_bytes(int32_t B, int32_t Kmax, int32_t V, int dtype);

/*
 * spec_verify_topkp -- spec_verify with top-k / top-p truncation of p and q.
 *
 * The "Speculative Decoding and MTP" survey, section 4, has the verify step
 * compare p and q after the same temperature and top-p / top-k transforms.
 * The transforms (this library's reading; the pages do not spell them out),
 * applied to every used row on its own, the target rows for p and the draft
 * rows for q:
 *   order the tokens by scaled logit s = fl32(x * fl32(1/T)) descending, the
 *   lower token id first among equal s;
 *   top-k: keep the first top_k[b] tokens (top_k[b] <= 0 or >= V: all);
 *   top-p: of those, with weights e^(s - max s), keep the shortest prefix
 *   whose weight reaches top_p[b] times their total (top_p[b] >= 1: all);
 *   p (or q) is the softmax over the kept tokens, 0 elsewhere.
 * The verify step then runs unchanged on the truncated p and q. Greedy
 * requests (T = 0) are unaffected: the argmax is always kept.
 *
 * Arguments: as spec_verify, plus (device pointers)
 *   top_k          int32 [B].
 *   top_p          float [B]; NaN or <= 0 faults the request with
 *                  LVTV_STATUS_BAD_TRUNCATION (combined with any other bits).
 * The workspace must hold spec_verify_topkp_workspace_bytes(...) bytes.
 * Which prefix top-p keeps is a floating-point decision: the kernel forms
 * the weights in 64-bit fixed point to about 3e-7 of the kept total, so a
 * request whose cumulative weight lies that close to top_p times the total
 * may keep one token more or fewer than an exact computation would.
 * Three kernels are enqueued: one radix selection per used row (a few
 * passes over the row), then the row and finalize kernels of spec_verify.
 */
int spec_verify_topkp(const void* target_logits, const void* draft_logits, int dtype,
                      const int32_t* draft_tokens, const int32_t* k_per_req,
                      const float* temperature, const uint64_t* seed, const int32_t* top_k,
                      const float* top_p, int32_t B, int32_t Kmax, int32_t V,
                      int32_t* accepted_len, int32_t* out_tokens, float* alpha,
                      int32_t* status, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes e2e_tv_loss_fwd_bwd needs (0 if out of range). Host only.
 */
size_t e2e_tv_loss_workspace_bytes(int32_t N, int32_t W, int32_t V);

/*
 * e2e_tv_loss_fwd_bwd -- E2E-TV prefix-product loss and its gradient.
 *
 * What it computes (SpecOPD, method step (6); Bebop section, E[tau]):
 *   q_{n,k} = softmax(z[n,k,:]) of the draft logits (no temperature);
 *   alpha_{n,k} = sum_v min(q_{n,k}(v), p[n,k,v]) with p used as given;
 *   L_n = -sum_{j<W} prod_{k<=j} alpha_{n,k};   loss = (1/N) sum_n L_n;
 *   dlogits[n,k,u] = dloss/dz[n,k,u] with p held constant:
 *     (G_{n,k}/N) * q(u) * ([q(u) < p(u)] - S_{n,k}),
 *     G_{n,k} = -P_{k-1} R_k, P_j = prod_{i<=j} alpha_i, P_{-1} = 1,
 *     R_{W-1} = 1, R_k = 1 + alpha_{k+1} R_{k+1}, S = sum_{q<p} q;
 *   the subgradient of min at q = p is 0; dlogits is rounded to bfloat16,
 *   round-to-nearest-even, from its fp32 value.
 *
 * Arguments (device pointers; row-major, V contiguous):
 *   draft_logits   bfloat16 (uint16) [N, W, V].
 *   target_probs   float [N, W, V], constants.
 *   N, W, V        1 <= N <= LVTV_MAX_N, 1 <= W <= LVTV_MAX_W,
 *                  1 <= V <= LVTV_MAX_V.
 *   loss           float [1] out.
 *   alpha          float [N, W] out.
 *   dlogits        bfloat16 (uint16) [N, W, V] out.
 *   workspace      device scratch of >= e2e_tv_loss_workspace_bytes(...)
 *                  bytes, 256-byte aligned. Its contents on entry do not
 *                  matter: the call first clears the words its workgroups
 *                  exchange, so a workspace left by any earlier call (of
 *                  either op) or holding garbage is fine. Calls sharing a
 *                  workspace must be ordered on one stream.
 *   stream         hipStream_t. For V <= 155648 three kernels are enqueued
 *                  (the clear, one workgroup per half row, one finishing
 *                  workgroup); larger V take the multi-pass pipeline.
 * NaN or infinite inputs propagate into the outputs; there is no status.
 */
int e2e_tv_loss_fwd_bwd(const uint16_t* draft_logits, const float* target_probs,
                        int32_t N, int32_t W, int32_t V, float* loss,
                        float* alpha, uint16_t* dlogits, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Workspace bytes draft_loss_fwd_bwd needs (0 if out of range; the same as
 * e2e_tv_loss_workspace_bytes). Host only.
 */
size_t draft_loss_workspace_bytes(int32_t N, int32_t W, int32_t V);

/*
 * draft_loss_fwd_bwd -- the E2E-TV loss or one of the per-position
 * objectives the pages set against it, with the gradient with respect to
 * the draft logits ("Reading Qwen Bebop and DeepSeek DSpark", section
 * "Bebop's solution": CE = -sum_y p log q, KL(p || q) = sum_y p log(p / q),
 * L_TV = d_TV(p, q) = 1 - sum_y min(p, q); the "SpecOPD" summary's ablation,
 * Figure 8, compares the E2E-TV objective with CE).
 *
 *   objective      LVTV_OBJ_*: per branch n the loss is summed over the W
 *                  positions, loss = (1/N) sum_n L_n:
 *                    E2E_TV   L_n = -sum_j prod_{k<=j} alpha_{n,k} (exactly
 *                             e2e_tv_loss_fwd_bwd);
 *                    STEP_TV  L_n = sum_k (1 - alpha_{n,k});
 *                    CE       L_n = sum_k -sum_v p log q_{n,k}(v);
 *                    KL       L_n = sum_k sum_v p log(p / q_{n,k}(v)),
 *                             p log p = 0 where p = 0.
 *                  Gradients: STEP_TV as E2E_TV with dL_n/dalpha_k = -1;
 *                  CE and KL: dlogits[n,k,u] = (q(u) sum_v p(v) - p(u)) / N.
 *   alpha          float [N, W] out: alpha_{n,k} = sum_v min(q, p) for every
 *                  objective.
 *   Other arguments, layouts, workspace rules and errors as for
 *   e2e_tv_loss_fwd_bwd; an unknown objective returns LVTV_ERR_OBJECTIVE
 *   before enqueueing anything.
 * Every objective runs the single-read kernel when V <= 155648: z and p
 * are read once and dz written once (CE and KL read p a second time for a
 * row whose coefficient (sum p)/N rounds to another binary32 than 1/N, or
 * whose data is not 16-byte aligned). Larger V take the multi-pass pipeline
 * (z read three times, p twice).
 */
int draft_loss_fwd_bwd(const uint16_t* draft_logits, const float* target_probs,
                       int32_t N, int32_t W, int32_t V, int objective,
                       float* loss, float* alpha, uint16_t* dlogits,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes draft_loss_logits_fwd_bwd needs (0 if out of range; the
 * same as e2e_tv_loss_workspace_bytes). Host only.
 */
size_t draft_loss_logits_workspace_bytes(int32_t N, int32_t W, int32_t V);

/*
 * draft_loss_logits_fwd_bwd -- draft_loss_fwd_bwd with the target given as
 * bfloat16 logits and a temperature: the target softmax is computed inside
 * the kernels, so the target costs 2 bytes per token instead of 4 and no
 * probability tensor is ever written.
 *
 * What it computes: both rows take the verify step's temperature transform
 * ("Speculative Decoding and MTP" survey, section 4: p and q after the same
 * transform), s = fl32(x * fl32(1/T)); p_{n,k} = softmax(s_target[n,k]) and
 * q_{n,k} = softmax(s_draft[n,k]), so alpha_{n,k} = sum_v min(q, p) is the
 * overlap the verify step sees at temperature T ("Reading Qwen Bebop and
 * DeepSeek DSpark", section "Formulas", eq. alpha_RS). The objective and its
 * reduction are as draft_loss_fwd_bwd's. The gradient is taken with respect
 * to the raw draft logits through s = x * fl32(1/T): every dlogits value of
 * draft_loss_fwd_bwd is multiplied by fl32(1/T). p is a constant ("SpecOPD"
 * summary, method step (6)).
 *
 * Arguments (device pointers; row-major, V contiguous):
 *   draft_logits   bfloat16 (uint16) [N, W, V].
 *   target_logits  bfloat16 (uint16) [N, W, V], constants.
 *   temperature    host float, finite and > 0 with fl32(1/T) finite, else
 *                  LVTV_ERR_TEMPERATURE before enqueueing anything.
 *   objective, N, W, V, loss, alpha, dlogits, workspace, stream: as
 *                  draft_loss_fwd_bwd.
 * The TV objectives run the single-read kernel when V <= 155648; CE, KL and
 * larger V run the multi-pass pipeline.
 */
int draft_loss_logits_fwd_bwd(const uint16_t* draft_logits, const uint16_t* target_logits,
                              float temperature, int32_t N, int32_t W, int32_t V,
                              int objective, float* loss, float* alpha, uint16_t* dlogits,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Paths of lvtv_debug_draft_loss. */
#define LVTV_PATH_AUTO 0       /* what the product entry points take        */
#define LVTV_PATH_MULTI_PASS 2 /* force the multi-pass pipeline             */
#define LVTV_PATH_REREAD 3     /* CE / KL on the single-read kernel with
                                  every row's gradient rewritten from a
                                  second read of the target (the product
                                  calls do that only for rows whose
                                  coefficient (sum p)/N rounds to another
                                  binary32 than 1/N); same outputs        */

/*
 * lvtv_debug_draft_loss -- test and debugging hook, not a product path.
 *
 * Runs draft_loss_fwd_bwd (target_probs given, target_logits NULL) or
 * draft_loss_logits_fwd_bwd (target_logits given with `temperature`,
 * target_probs NULL) with settings the product calls fix:
 *   path         LVTV_PATH_AUTO, LVTV_PATH_MULTI_PASS or LVTV_PATH_REREAD
 *                (else LVTV_ERR_OPTION);
 *   spin_limit   polling rounds a half-row workgroup of the single-read
 *                kernel waits for the rest of its branch before leaving its
 *                row to the finishing launch, which recomputes it
 *                bit-identically (0: every row takes that repair path; the
 *                product calls use 65536);
 *   dlogits_f32  optional float [N, W, V] out: the gradient in fp32 before
 *                its rounding to bfloat16 (NULL: not written).
 * Everything else (arguments, workspace, errors) as the product calls;
 * exactly one of target_probs and target_logits must be non-NULL
 * (LVTV_ERR_NULL otherwise).
 */
int lvtv_debug_draft_loss(const uint16_t* draft_logits, const float* target_probs,
                          const uint16_t* target_logits, float temperature, int32_t N,
                          int32_t W, int32_t V, int objective, int path, int32_t spin_limit,
                          float* loss, float* alpha, uint16_t* dlogits, float* dlogits_f32,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * dspark_schedule -- confidence-scheduled verify lengths ("Reading Qwen
 * Bebop and DeepSeek DSpark", section "DSpark's second piece:
 * confidence-scheduled verify length").
 *
 * Request r has confidences c_{r,j}, j < L (the chance that draft token j
 * survives once every earlier one did; the pages' soft label is 1 - d_TV,
 * which is spec_verify's alpha). With prefix survivals
 * a_{r,j} = prod_{i<=j} c_{r,i}, verifying l_r tokens of each request feeds
 * B = sum_r (1 + l_r) tokens to the target model and yields
 * tau = sum_r (1 + sum_{j<l_r} a_{r,j}) tokens in expectation. The call picks
 * the l_r maximising Theta = tau * SPS(B).
 *
 * Arguments (device pointers):
 *   confidence   float [R, L]; clamped to [0, 1], NaN read as 0.
 *   sps          float [R (L + 1) + 1]: decode steps per second at batch
 *                size B (entry B; entries below R are not read).
 *   R, L         1 <= R, 1 <= L, R L <= LVTV_SCHED_MAX_ITEMS.
 *   verify_len   int32 [R] out: l_r in 0..L.
 *   best         double [2] out: Theta at the optimum and its B.
 *   stream       hipStream_t. One workgroup; no workspace.
 * Arithmetic: survivals in binary32, left to right; equal survivals are
 * taken in flat index order r L + j; tau and Theta in fp64; among equal
 * Theta the smallest B wins, and a NaN Theta never wins (all NaN: B = R).
 * Returns LVTV_ERR_SHAPE / LVTV_ERR_NULL before enqueueing anything.
 */
#define LVTV_SCHED_MAX_ITEMS 8192 /* R L of one dspark_schedule call */
int dspark_schedule(const float* confidence, const float* sps, int32_t R,
                    int32_t L, int32_t* verify_len, double* best, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LVTV_H */
