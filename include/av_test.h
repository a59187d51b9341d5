/*
 * av_test.h -- launch-form knobs of the fused pass, for tests and tuning.
 *
 * Not part of the library's contract: av_verify_opd_fwd (av.h) chooses the
 * launch form itself.  This entry point computes exactly what
 * av_verify_opd_fwd computes (same arguments, same outputs, same errors) but
 * lets the caller force the form, so that tests reach every code path of the
 * kernel at small widths.
 */
#ifndef AV_TEST_H
#define AV_TEST_H

#include "av.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * av_test_verify_opd_fwd -- av_verify_opd_fwd with two extra arguments:
 *   onchip_limit  0 = automatic.  Otherwise (regs | lds << 8): how many
 *                 16-byte vectors per thread of each row (or half row) the
 *                 pass keeps in registers and in LDS (each clamped to what
 *                 the build provides); the rest is read from HBM a second
 *                 time for the gradient.
 *   split_rows    0 = automatic (as av_verify_opd_fwd), 1 = whole rows,
 *                 2 = rows split into halves on workgroup pairs: workgroups
 *                 2p and 2p+1 take the two halves of the same rows in a fixed
 *                 order and hand each other their first-sweep statistics and
 *                 clip corrections through the workspace (16-byte vector
 *                 variants only, V >= 2 vectors; ignored otherwise).  Both
 *                 workgroups of a pair are resident for the whole launch, so
 *                 a half waits only for its partner (bounded: AV_DEV_TIMEOUT
 *                 if the device is shared so heavily that a partner never
 *                 runs).  3 = split tail, the form av_verify_opd_fwd picks
 *                 for a ragged launch whose last round of rows is partial:
 *                 here rows 0 .. R/2 - 1 whole and the rest as pairs of
 *                 halves, all claimed from the work dispenser (ragged layout
 *                 and 16-byte vector variants only; ignored otherwise).
 *                 4 = rows split into four parts on teams of four workgroups
 *                 (4t .. 4t+3), as 2 otherwise (16-byte vector variants, V
 *                 >= 4 vectors; ignored otherwise).
 * Errors: as av_verify_opd_fwd; AV_EINVAL also for a negative onchip_limit
 * or a split_rows outside 0..4.
 */
int av_test_verify_opd_fwd(int dtype, int B, int k, int V, int R,
                           const int32_t* row_off, const void* zp, const void* zq,
                           const int32_t* draft, const int32_t* bk,
                           float lambda, float tau, float grad_scale, float temperature,
                           int32_t* tgt_argmax, int32_t* acc_len, float* row_loss,
                           float* req_loss, float* total_loss, float* row_stats,
                           float* lse_q1, void* grad_zq, int grad_dtype, int32_t* status,
                           void* workspace, size_t workspace_bytes,
                           int onchip_limit, int split_rows, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AV_TEST_H */
