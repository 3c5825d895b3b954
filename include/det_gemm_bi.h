/*
 * det_gemm_bi.h -- C-ABI of the batch-invariant linear layer (det_gemm) of
 * the same library: forward y = x W^T and the backward dX = dY W and
 * dW = dY^T X, with a dW that is bitwise identical however the same logical
 * rows reach it.
 *
 * What is computed.  "[WS1 Closeout][Backward] Reusable gradient-invariance
 * harness and operator adapters", section "Required adapters", lists GEMM
 * dX/dW; "WS1 C4 (#270) closeout evidence" (status table and the note on
 * the reds) places the deterministic GEMM's dW in the same failure class as
 * RMSNorm's dweight, fixed by building parameter gradients from one FP32
 * contribution per logical row.  With x[rows][K], W[N][K], dY[rows][N]:
 *     y[r][n]  = sum_k x[r][k] W[n][k]                (bf16 out, FP32 accumulate)
 *     dX[r][k] = sum_n dY[r][n] W[n][k]               (bf16 out, FP32 accumulate)
 *     dW[n][k] = sum over logical rows l of dY[l][n] X[l][k]    (FP32)
 * dW is reduced in one canonical order (GDO-v1): logical rows in groups of
 * 16384; within a group, a chain of 32x32x16 bf16 matrix-core steps over
 * the rows in ascending 16-row steps from +0.0; across groups, a perfect
 * pairwise tree with +0.0 leaves up to the next power of two.  Rows past
 * the logical count are zero.  y and dX are row-local and run the same
 * chain over the contraction index for every row, whatever the call.
 *
 * Conventions are those of rmsnorm_bi.h: device pointers owned by the
 * caller, bf16 as raw 16-bit patterns, contiguous row-major tensors, 16-byte
 * alignment (4 bytes for dW), N and K multiples of 8, `stream` a
 * hipStream_t as void*, int status codes RMSNORM_* with the message in
 * rmsnorm_last_error(), no fallback path, rows == 0 a successful no-op.
 * Layouts are rmsnorm_layout objects (the same physical -> logical row maps
 * as the norm's; -1 = padding row, never read, output 0).
 */
#ifndef DET_GEMM_BI_H
#define DET_GEMM_BI_H

#include <stdint.h>

#include "rmsnorm_bi.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct det_gemm_dw_acc det_gemm_dw_acc;

/* y[rows][n] = x[rows][k] W^T.  layout may be NULL (no padding rows). */
int det_gemm_fwd(const rmsnorm_bf16* x, const rmsnorm_bf16* w, rmsnorm_bf16* y, int64_t rows,
                 int64_t n, int64_t k, const rmsnorm_layout* layout, void* stream);

/* dX[rows][k] = dY[rows][n] W.  Padding rows of the layout get dX = 0 and
 * their dY is not read. */
int det_gemm_bwd_dx(const rmsnorm_bf16* dy, const rmsnorm_bf16* w, rmsnorm_bf16* dx,
                    int64_t rows, int64_t n, int64_t k, const rmsnorm_layout* layout,
                    void* stream);

/* Canonical dW accumulator for n_logical rows (at most 64 * 16384) of a
 * layer with N = n outputs and K = k inputs.  Allocates the group results
 * (ceil(n_logical / 16384) x n x k FP32) and a logical-order staging copy
 * of x and dY (n_logical x (n + k) bf16).  Synchronous. */
int det_gemm_dw_acc_create(det_gemm_dw_acc** out, int64_t n_logical, int64_t n, int64_t k,
                           void* stream);

/* Adds one call's rows.  With layout == NULL the call must hold all
 * n_logical rows in logical order: the group results are computed at once
 * from x and dY.  Otherwise the call's real rows are copied to their
 * logical positions and the products run at finalize.  Every logical row
 * must be added exactly once (RMSNORM_ECOVERAGE otherwise); adding after a
 * finalize without a reset is RMSNORM_ESTATE.  The inputs may be reused
 * once the work enqueued here has run. */
int det_gemm_dw_contrib(const rmsnorm_bf16* x, const rmsnorm_bf16* dy, int64_t rows, int64_t n,
                        int64_t k, const rmsnorm_layout* layout, det_gemm_dw_acc* acc,
                        void* stream);

/* dW[n][k] (FP32) in the canonical order.  Checks that every logical row was
 * added (RMSNORM_ECOVERAGE).  May be called again: the same bits. */
int det_gemm_dw_finalize(det_gemm_dw_acc* acc, float* dw, void* stream);

/* Forget all added rows (no device work). */
int det_gemm_dw_acc_reset(det_gemm_dw_acc* acc, void* stream);

/* Waits for the device, then frees. */
int det_gemm_dw_acc_destroy(det_gemm_dw_acc* acc);

#ifdef __cplusplus
}
#endif

#endif /* DET_GEMM_BI_H */
