/*
 * av.h -- C ABI of the AdaFlash verify + on-policy-distillation pass on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed comes from the pages describing AdaFlash (arXiv
 * 2607.19223): the Pith review page "AdaFlash: Adaptive Speculative Decoding
 * via On-Policy Distilled Diffusion Drafters" (sections "What carries the
 * argument", Referee Report major comments 1-2 and minor comments 1, 2, 4,
 * "Axiom & Free-Parameter Ledger"), the Pith verdict record's skeptic
 * critique, and the ResearchPod summary's component list.
 *
 * Conventions shared by every entry point
 *  - All array arguments are DEVICE pointers owned by the caller; the library
 *    never allocates device memory, never frees, and keeps no pointer after a
 *    call returns.  Scalars are passed by value on the host.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    returns without synchronising.  Outputs are valid once the stream reaches
 *    the call.
 *  - Arguments the host can check are checked before anything is enqueued;
 *    a violation returns AV_EINVAL (or AV_EUNSUPPORTED for a shape or type
 *    outside the implemented range) and touches no memory.  A failed launch
 *    returns AV_EHIP.
 *  - Rows: a "row" is one (request, draft position) pair.  In the DENSE
 *    layout row r = b*k + i holds position i of request b (R = B*k rows).  In
 *    the RAGGED layout request b owns rows row_off[b] .. row_off[b+1]-1 and
 *    only those rows are stored (variable-length verification batching, no
 *    padding).
 *  - Logit rows are row-major [R, V]: element (r, j) at r*V + j, in float32
 *    (AV_F32) or bfloat16 (AV_BF16, upper half of a float32).  Logits must be
 *    finite; non-finite input is outside the contract (results unspecified).
 */
#ifndef AV_H
#define AV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AV_OK = 0,
  AV_EINVAL = -1,        /* bad argument detected on the host, nothing enqueued */
  AV_EUNSUPPORTED = -2,  /* valid but outside the implemented range */
  AV_EHIP = -3           /* the HIP runtime reported an error */
} av_status;

typedef enum { AV_F32 = 0, AV_BF16 = 1 } av_dtype;
typedef enum { AV_ROUND_CEIL = 0, AV_ROUND_FLOOR = 1 } av_round;

/* Bits a call can report through its optional device `status` word. */
#define AV_DEV_TIMEOUT 1      /* a cross-workgroup wait exceeded its bound; outputs invalid */
#define AV_DEV_BAD_OFFSETS 2  /* ragged offsets break 0 = off[0], 1 <= n_b <= k, off[B] = R;
                                 nothing was computed */

/* Largest draft block the pass accepts. */
#define AV_MAX_K 64

/*
 * av_length_head -- adaptive verification length.
 *
 * The pages' adaptive length head (Pith review page, Referee Report minor
 * comment 2, paper Sec. 3.2; ledger entry gamma; ResearchPod component 2)
 * maps a pooled drafter representation to one scalar, the predicted
 * acceptance rate, and turns it into the number of draft positions sent to
 * the target.  For each request b:
 *     z_b    = sum_h w[h] * h[b*H + h] + bias        (float64 accumulation)
 *     rate_b = 1 / (1 + exp(-z_b))
 *     bk_b   = clamp(ceil(gamma * rate_b * k), 1, k) (AV_ROUND_CEIL), or
 *              clamp(floor(gamma * rate_b * k), 1, k) (AV_ROUND_FLOOR).
 *
 *   h        [B, H] float32, row-major pooled drafter state (the pooling
 *            itself is the caller's; the pages do not specify it)
 *   w        [H] float32 head weights;  bias, gamma: host scalars
 *   rate_out [B] float32 rate_b, may be NULL;  bk_out [B] int32 b_k
 * Errors: NULL h/w/bk_out, B < 1, H < 1, k < 1, k > AV_MAX_K, bad round mode,
 * non-finite bias/gamma or gamma < 0 -> AV_EINVAL.
 */
int av_length_head(const float* h, const float* w, float bias, float gamma,
                   int B, int H, int k, int round_mode,
                   float* rate_out, int32_t* bk_out, void* stream);

/*
 * av_length_head_update -- one online update of the length head from the
 * outcome of a verification step (Pith review page, Referee Report major
 * comment 1, paper Sec. 3.2 "Online Update of the Length Head": an MSE loss
 * against the observed acceptance rate; "Axiom & Free-Parameter Ledger":
 * length head learning rate 2e-4, AdamW).  For each request b:
 *     rate_b  = sigmoid(w . h_b + bias)              (as av_length_head)
 *     label_b = acc_b / clamp(bk_b, 1, k)            (accepted fraction of
 *                                                     the verified block)
 *     loss    = (1/B) sum_b (rate_b - label_b)^2
 * then the gradients of loss with respect to w, bias and h, and one AdamW
 * step on w and bias with step number t = `step`:
 *     theta <- theta (1 - lr wd);  m <- beta1 m + (1 - beta1) g;
 *     v <- beta2 v + (1 - beta2) g^2;
 *     theta <- theta - lr / (1 - beta1^t) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 * Sums run in float64 in request order; parameters and moments stay float32.
 *
 *   h            [B, H] float32 pooled drafter state (the same input as
 *                av_length_head)
 *   acc, bk      [B] int32: accepted lengths (av_verify_opd_fwd's acc_len)
 *                and the verification lengths that step used
 *   w [H], bias [1], m_w [H], v_w [H], m_b [1], v_b [1]
 *                float32, updated in place (moments zero for a fresh head)
 *   step         number of this update, >= 1 (the caller counts updates)
 *   lr, beta1, beta2, eps, weight_decay
 *                AdamW constants (the pages print lr; the common defaults
 *                are 0.9, 0.999, 1e-8, 0.01)
 *   loss_out [1], rate_out [B], grad_h_out [B, H]: float32 outputs or NULL;
 *                grad_h_out uses w before the step
 *   workspace    >= av_head_update_workspace_bytes(B) bytes, 8-byte aligned,
 *                no initialisation needed
 * All pointers are device pointers; the call is asynchronous on `stream` (two
 * launches).  Errors (AV_EINVAL): NULL required pointer, B < 1, H < 1, k < 1
 * or > AV_MAX_K, step < 1, lr or weight_decay negative or non-finite, beta1 or
 * beta2 outside [0, 1), eps not positive and finite, workspace too small or
 * misaligned.
 */
size_t av_head_update_workspace_bytes(int B);
int av_length_head_update(const float* h, const int32_t* acc, const int32_t* bk, int B, int H, int k,
                          float* w, float* bias, float* m_w, float* v_w, float* m_b, float* v_b,
                          int step, double lr, double beta1, double beta2, double eps,
                          double weight_decay, float* loss_out, float* rate_out, float* grad_h_out,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * av_spec_verify -- sampling-based block verification (speculative sampling).
 *
 * The pages list the standard speculative-decoding acceptance formula as an
 * axiom (Pith review page, "Axiom & Free-Parameter Ledger", after Leviathan
 * et al. 2023) and cite Chen et al. 2023 on speculative sampling; this is
 * that published method at temperature 1.  For request b (rows as in
 * av_verify_opd_fwd; only verified positions i < b_k are tested), with
 * p = softmax(zp[r,:]) and q = softmax(zq[r,:]) at row r = row(b, i):
 *   position i is accepted iff u[r] * q(d) < p(d), d = draft[r] (a draft
 *     outside [0, V) is rejected), i.e. with probability min(1, p(d)/q(d));
 *   acc_len[b] = number of positions accepted before the first rejection;
 *   token[b]   = at the first rejected position, a draw from the residual
 *     max(0, p - q) / sum(max(0, p - q)) (p itself if that is zero
 *     everywhere), by the exponential race argmax_j r_j / E_j (ties to the
 *     lowest j), E_j = -ln(u_j), u_j = (w_j + 1/2) / 2^32 where w_j is word
 *     j % 4 of Philox4x32-10 (Salmon et al., SC 2011) with key (seed low 32
 *     bits, seed high 32 bits) and counter (j / 4, r, 0, 0); -1 when every
 *     verified position is accepted (the caller draws the bonus token from
 *     the target's next distribution).
 * Every emitted token (accepted draft or replacement) is then distributed
 * as a draw from the target.
 *
 * Arguments
 *   dtype, B, k, V, R, row_off, zp, zq, draft, bk: as av_verify_opd_fwd
 *   u            [R] float32 uniforms in [0, 1) for the acceptance tests
 *                (the caller's generator)
 *   seed         64-bit key of the replacement draw
 *   row_stats_in [R, stats_stride] float32 or NULL: lse_p (column 0) and
 *                lse_q (column 1) of every verified row, e.g. the row_stats
 *                of av_verify_opd_fwd on the same inputs (stride 4), whose
 *                first sweep already computed them; then no row is read
 *                whole for the acceptance tests (p(d) and q(d) are gathered)
 *                and only each request's first rejected row is read, for the
 *                replacement draw.  NULL: the call computes them.
 *   stats_stride >= 2 when row_stats_in is given
 *   acc_len, token  [B] int32 out
 *   row_stats    [R, 2] float32 out or NULL: (lse_p, lse_q) of verified rows
 *   status       [1] int32 out or NULL: 0, or AV_DEV_BAD_OFFSETS for a
 *                ragged request whose offsets are invalid (it gets acc 0,
 *                token -1)
 *   workspace    >= av_spec_workspace_bytes(B, R) bytes, 16-byte aligned, no
 *                initialisation needed
 * All pointers are device pointers; asynchronous on `stream` (three launches).
 * Errors: as av_verify_opd_fwd for the shared arguments; AV_EINVAL for NULL
 * u/acc_len/token/workspace, a workspace that is too small or misaligned, or
 * stats_stride < 2 with row_stats_in given.
 */
size_t av_spec_workspace_bytes(int B, int R);
int av_spec_verify(int dtype, int B, int k, int V, int R, const int32_t* row_off,
                   const void* zp, const void* zq, const int32_t* draft, const int32_t* bk,
                   const float* u, uint64_t seed, const float* row_stats_in, int stats_stride,
                   int32_t* acc_len, int32_t* token, float* row_stats, int32_t* status,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * av_workspace_bytes -- size of the scratch area av_verify_opd_fwd needs for
 * B requests and R stored rows (R = B*k dense).  Independent of V and dtype.
 * Returns 0 for invalid sizes.
 */
size_t av_workspace_bytes(int B, int k, int R);

/*
 * av_workspace_init -- zero a workspace once, before its first use, on
 * `stream`.  Every later call leaves it ready for the next one, so it is not
 * needed again while the buffer lives.  A workspace serves one call at a
 * time: two calls that may overlap (different streams) need two workspaces.
 */
int av_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * av_verify_opd_fwd -- fused block verification + OPD loss (+ gradient).
 *
 * For every stored row r (request b, position i), with zp/zq the target and
 * drafter logits of that position, p = softmax(zp), q = softmax(zq):
 *   tgt_argmax[r] = smallest j with zp[r,j] = max zp[r,:]   (greedy target
 *                   choice; Pith review page, Referee Report major comment 2)
 *   row r is VERIFIED iff i < b_k (dense: b_k = clamp(bk[b], 1, k); ragged:
 *                   every stored row is verified and b_k = n_b)
 *   acc_len[b]    = number of leading positions i < b_k with
 *                   draft[row(b,i)] == tgt_argmax[row(b,i)]  (greedy block
 *                   verification truncated at b_k; Pith verdict record,
 *                   skeptic critique; review page Sec. 2.1 Eq. (1) context).
 *                   A draft token outside [0, V) never matches.
 *   for verified rows, with ell_j = log q_j - log p_j, r_j = q_j * ell_j,
 *   c_j = [-tau <= r_j <= tau]:
 *     row_loss[r] = lambda * (-log q[a_r]) + (1 - lambda) * sum_j clip(r_j, -tau, tau)
 *                   (hard-label cross-entropy mixed with entry-wise clipped
 *                   reverse KL; review page "What carries the argument",
 *                   ResearchPod component 1, ledger entries alpha and delta)
 *     grad_zq[r,j] = grad_scale * ( lambda (q_j - [j = a_r])
 *                     + (1 - lambda) q_j (c_j (ell_j + 1) - S_r) ),
 *                   S_r = sum_j c_j q_j (ell_j + 1)        (d row_loss / d zq)
 *   unverified dense rows: row_loss 0, row_stats 0, grad_zq row 0.
 *   req_loss[b]  = sum of row_loss over b's verified rows (float64, fixed order)
 *   total_loss   = sum_b req_loss[b] (float64, fixed order)
 *   row_stats[r] = {lse_p, lse_q, S_r, clipped-KL sum} (float32), the state
 *                  av_verify_opd_bwd needs.
 *
 * Temperature (Pith review page, "Axiom & Free-Parameter Ledger": a
 * reverse-KL temperature of 1.0, not defined further).  With temperature
 * T != 1 the reverse-KL term uses p = softmax(zp / T) and q = softmax(zq / T)
 * in every formula above (ell, r, c, S, the clipped sum, lse_p and lse_q,
 * which become the log-sum-exps of zp / T and zq / T), while the
 * cross-entropy keeps q1 = softmax(zq):
 *     row_loss[r]  = lambda * (-log q1[a_r]) + (1 - lambda) * sum_j clip(r_j, -tau, tau)
 *     grad_zq[r,j] = grad_scale * ( lambda (q1_j - [j = a_r])
 *                     + (1 - lambda) q_j (c_j (ell_j + 1) - S_r) / T )
 * (no T^2 factor).  T = 1 is the pass above, bit for bit.
 *   lse_q1[r]    = log-sum-exp of zq[r,:] (temperature 1) of verified rows,
 *                  0 for unverified dense rows; the backward needs it when
 *                  T != 1.
 *
 * Arguments
 *   dtype        AV_F32 or AV_BF16 (element type of zp and zq)
 *   B, k, V      requests, draft block length (1..AV_MAX_K), vocabulary
 *   R            stored rows: B*k (dense) or row_off[B] (ragged)
 *   row_off      NULL -> dense layout;  else [B+1] int32 exclusive prefix sum
 *                of n_b (ragged).  Checked on the device (AV_DEV_BAD_OFFSETS)
 *   zp, zq       [R, V] target / drafter logits
 *   draft        [R] int32 draft tokens
 *   bk           [B] int32 verification lengths (dense; clamped to [1, k]);
 *                ignored (may be NULL) when ragged
 *   lambda       in [0, 1];  tau > 0 (may be +inf: no clipping);
 *   grad_scale   finite multiplier of the gradient (e.g. 1 / sum b_k)
 *   temperature  T > 0, finite (1: the plain pass)
 *   tgt_argmax   [R] int32 out;  acc_len [B] int32 out;  row_loss [R] float32 out
 *   req_loss     [B] float32 out or NULL;  total_loss [1] float32 out or NULL
 *   row_stats    [R, 4] float32 out or NULL
 *   lse_q1       [R] float32 out or NULL
 *   grad_zq      [R, V] out or NULL (NULL: forward only), of type grad_dtype
 *   grad_dtype   AV_F32 (the default: float32 entries) or AV_BF16 (each
 *                float32 entry rounded to nearest-even bfloat16, half the
 *                bytes written; the pages do not fix the gradient's
 *                precision, and bfloat16 rounding alone exceeds a 1e-3
 *                relative tolerance, so float32 is the reference form)
 *   status       [1] int32 out or NULL: 0, or AV_DEV_* bits found on device
 *   workspace    >= av_workspace_bytes(B, k, R) bytes, zeroed once by
 *                av_workspace_init before first use
 * Launch: one persistent 1024-thread workgroup per CU, rows taken from a
 * dispense counter in the workspace, longest first.  A ragged launch of long
 * rows (bfloat16 V >= 147456, float32 V >= 73728 with 16-byte rows) whose
 * rows end in a partial round runs the full rounds as whole rows and the
 * remaining rows as two halves each on two workgroups, which exchange their
 * statistics through the workspace (each wait bounded: AV_DEV_TIMEOUT); a
 * dense launch of such rows with at most half as many rows as CUs runs every
 * row in halves.  A dense launch with at most a quarter as many rows as CUs
 * (rows of bfloat16 V >= 106496, float32 V >= 53248 with 16-byte rows) runs
 * every row in quarters, each on its own workgroup of a team of four.
 * Errors (AV_EINVAL): NULL required pointer, B < 1, k < 1 or > AV_MAX_K,
 * V < 1, R inconsistent with the layout, lambda outside [0, 1] or NaN, tau
 * <= 0 or NaN, grad_scale non-finite, temperature not positive and finite,
 * workspace too small, row_stats or workspace not 16-byte aligned.
 * AV_EUNSUPPORTED: dtype or grad_dtype other than AV_F32/AV_BF16; ragged
 * with B > 4095 (the offsets are cached on chip); R*V >= 2^46.
 */
int av_verify_opd_fwd(int dtype, int B, int k, int V, int R,
                      const int32_t* row_off, const void* zp, const void* zq,
                      const int32_t* draft, const int32_t* bk,
                      float lambda, float tau, float grad_scale, float temperature,
                      int32_t* tgt_argmax, int32_t* acc_len, float* row_loss,
                      float* req_loss, float* total_loss, float* row_stats,
                      float* lse_q1, void* grad_zq, int grad_dtype, int32_t* status,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * av_verify_opd_fwd_noalloc -- av_verify_opd_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments, outputs and errors
 * without workspace / workspace_bytes.  The workspace is a library-owned
 * array of AV_NOALLOC_SCRATCH_BYTES bytes per GPU, resident until the process
 * ends; the call allocates nothing.  Limits and behaviour:
 *  - av_workspace_bytes(B, k, R) must not exceed AV_NOALLOC_SCRATCH_BYTES
 *    (4 MiB: B = 128 requests of 16 rows need 0.93 MiB; about 8800 rows in
 *    all), else AV_EUNSUPPORTED before anything is enqueued;
 *  - the array is looked up and zeroed synchronously on the first call on a
 *    device (or by av_init); make that first call, or av_init, outside graph
 *    capture;
 *  - every call on a GPU shares that GPU's array: calls that may overlap on
 *    one GPU (different streams without ordering) race; serialise them.
 */
#define AV_NOALLOC_SCRATCH_BYTES (4u << 20)
int av_verify_opd_fwd_noalloc(int dtype, int B, int k, int V, int R,
                              const int32_t* row_off, const void* zp, const void* zq,
                              const int32_t* draft, const int32_t* bk,
                              float lambda, float tau, float grad_scale, float temperature,
                              int32_t* tgt_argmax, int32_t* acc_len, float* row_loss,
                              float* req_loss, float* total_loss, float* row_stats,
                              float* lse_q1, void* grad_zq, int grad_dtype, int32_t* status,
                              void* stream);
/* Size of that array (AV_NOALLOC_SCRATCH_BYTES). */
size_t av_noalloc_max_bytes(void);
/* Per-device set-up of the current device (the no-allocation array, launch
 * facts); optional, for callers that must not pay it on a first call. */
int av_init(void);

/*
 * av_verify_opd_bwd -- gradient alone, from saved row statistics.
 *
 * Recomputes grad_zq exactly as av_verify_opd_fwd defines it, in one
 * streaming pass, from tgt_argmax and row_stats of an earlier forward call
 * with the same inputs and the same lambda/tau/grad_scale/temperature: every
 * entry uses the same float32 steps as the fused pass, so both write
 * identical bits.
 *   row_off, zp, zq, bk, dtype, B, k, V, R: as for av_verify_opd_fwd
 *   tgt_argmax [R] int32, row_stats [R, 4] float32: from the forward call
 *   lse_q1     [R] float32 from the forward call; required when
 *              temperature != 1, else ignored (may be NULL)
 *   grad_zq    [R, V] out of type grad_dtype (AV_F32 or AV_BF16, as for
 *              av_verify_opd_fwd; unverified dense rows are zeroed)
 *   vecs_per_thread  0 = automatic; otherwise the most 16-byte vectors one
 *              thread handles per work item (raised where needed so that a
 *              row has at most 64 items)
 * Errors as for av_verify_opd_fwd (AV_EINVAL also for a negative
 * vecs_per_thread, and for a NULL lse_q1 when temperature != 1).  AV_EUNSUPPORTED also for rows longer than 64 items:
 * V > 1048576 (bf16, V % 8 == 0, 16-byte aligned rows), V > 524288 (f32,
 * V % 4 == 0, aligned), V > 262144 otherwise.  Needs no workspace; row_off
 * only selects the ragged layout (every stored row verified).
 */
int av_verify_opd_bwd(int dtype, int B, int k, int V, int R,
                      const int32_t* row_off, const void* zp, const void* zq,
                      const int32_t* bk, const int32_t* tgt_argmax,
                      const float* row_stats, const float* lse_q1, float lambda,
                      float tau, float grad_scale, float temperature, void* grad_zq,
                      int grad_dtype, int vecs_per_thread, void* stream);

/*
 * av_lm_head_bwd -- backward of the drafter's LM head, the step after this
 * pass in training (Pith review page, "Axiom & Free-Parameter Ledger":
 * drafter updates with AdamW).  The head maps the hidden state of each
 * position to its logits, zq[r, v] = sum_h hid[r, h] W[v, h] (no bias); with
 * dz = d loss / d zq from av_verify_opd_fwd (grad_dtype AV_BF16):
 *     d_hid[r, h] = sum_v dz[r, v] W[v, h]
 *     d_w[v, h]   = sum_r dz[r, v] hid[r, h]
 * Two bfloat16 GEMMs with float32 accumulation on the matrix cores (the
 * library's own v_mfma_f32_32x32x16_bf16 kernels; the long sum over V of
 * d_hid may be split over workgroups, the partial sums then added in a fixed
 * order, so results are deterministic for a given device).
 *   dz     [R, V] bfloat16 row-major;  w [V, H] bfloat16;  hid [R, H] bfloat16
 *   d_hid  [R, H] float32 out, or NULL (then w may be NULL)
 *   d_w    [V, H] float32 out, or NULL (then hid may be NULL)
 *   workspace, workspace_bytes: device scratch for the split sum of d_hid,
 *          16-byte aligned, may be NULL / 0 (then d_hid is one sum per
 *          entry, which takes longer on small R H); av_lm_head_workspace_bytes
 *          (R, V, H) is the size the library uses on the current device, 0
 *          when it does not split.  Not read before it is written; nothing
 *          to initialise, and it may be reused across calls on one stream.
 * All pointers are device pointers; rows of 16-byte aligned operands with V
 * and H multiples of 8 take the 16-byte load path, any other shape an
 * element-wise one.  Asynchronous on `stream`.  Errors: AV_EINVAL for R, V or
 * H < 1, NULL dz, an output without its operand, or workspace_bytes > 0 with
 * a NULL workspace; AV_EUNSUPPORTED for R above 2^30 or V, H above 2^22; AV_EHIP for a
 * launch failure (text in av_lm_head_last_error(), per thread).
 */
size_t av_lm_head_workspace_bytes(int R, int V, int H);
int av_lm_head_bwd(int R, int V, int H, const void* dz, const void* w, const void* hid,
                   float* d_hid, float* d_w, void* workspace, size_t workspace_bytes,
                   void* stream);
const char* av_lm_head_last_error(void);

/* Human-readable text for an av_status value (static storage). */
const char* av_status_str(int status);

/* Text of the most recent AV_EHIP error on the calling thread. */
const char* av_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* AV_H */
