/*
 * det_embedding_bi.h -- C-ABI of the batch-invariant embedding of the same
 * library: the row gather y[r] = E[id(r)] and the table gradient
 * dE[v] = sum of dY over the logical rows whose token is v, bitwise
 * identical however the same logical rows reach it.
 *
 * What is computed.  "[WS1 Closeout][Backward] Reusable gradient-invariance
 * harness and operator adapters", Required adapters, lists Embedding /
 * LM-head; its Acceptance criteria ask for the embedding/LM-head weight
 * gradients by stable name.  The scatter-add of the embedding gradient is
 * reduced in one canonical order keyed by (token id, logical row), EDO-v1:
 * the occurrences of a token in ascending logical row index are cut into
 * blocks of 64; a block is folded from +0.0 in occurrence order in FP32; the
 * token's block partials meet in a perfect pairwise tree with +0.0 leaves
 * up to the next power of two; tokens that do not occur get +0.0.  (The
 * LM-head weight gradient of a vocabulary projection is det_gemm's dW with
 * N = vocabulary size.)
 *
 * Conventions are those of rmsnorm_bi.h (device pointers, raw bf16, 16-byte
 * aligned rows, dim % 8 == 0, hipStream_t as void*, RMSNORM_* status codes,
 * rmsnorm_last_error(), no fallback).  Token ids are int32.
 */
#ifndef DET_EMBEDDING_BI_H
#define DET_EMBEDDING_BI_H

#include <stdint.h>

#include "rmsnorm_bi.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct det_embedding_dw_acc det_embedding_dw_acc;

/* y[rows][dim] = table[ids[r]] (device ids, one per physical row).  Rows
 * that the layout marks as padding are not read and get 0; an id outside
 * [0, vocab) reads nothing and gives 0. */
int det_embedding_fwd(const int32_t* ids, const rmsnorm_bf16* table, rmsnorm_bf16* y,
                      int64_t rows, int64_t vocab, int64_t dim, const rmsnorm_layout* layout,
                      void* stream);

/* Accumulator of the table gradient for a batch of n_logical rows (at most
 * 2^21) whose token ids, in logical row order, are ids_host (a host array;
 * every id in [0, vocab)).  Builds the batch's canonical scatter plan on the
 * host and uploads it; allocates block partials and a logical-order staging
 * copy of dY.  Synchronous. */
int det_embedding_dw_acc_create(det_embedding_dw_acc** out, const int32_t* ids_host,
                                int64_t n_logical, int64_t vocab, int64_t dim, void* stream);

/* Replaces the batch's token ids (same n_logical) and resets the
 * accumulator.  Synchronous (waits for `stream`). */
int det_embedding_dw_acc_set_ids(det_embedding_dw_acc* acc, const int32_t* ids_host,
                                 void* stream);

/* Adds one call's dY rows.  With layout == NULL the call holds all
 * n_logical rows in logical order and the block folds run at once;
 * otherwise the call's real rows are copied to their logical positions and
 * the folds run at finalize.  Every logical row exactly once
 * (RMSNORM_ECOVERAGE), no contribution after finalize without a reset
 * (RMSNORM_ESTATE). */
int det_embedding_dw_contrib(const rmsnorm_bf16* dy, int64_t rows, int64_t dim,
                             const rmsnorm_layout* layout, det_embedding_dw_acc* acc,
                             void* stream);

/* dE[vocab][dim] (FP32, every row written).  May be called again: the same bits. */
int det_embedding_dw_finalize(det_embedding_dw_acc* acc, float* dE, void* stream);

/* The whole backward in one call, for a caller whose one call holds all
 * n_logical rows of dY in logical order (the B=N case): dE[vocab][dim] as
 * det_embedding_dw_contrib(layout NULL) + det_embedding_dw_finalize would
 * give it, bit for bit, with the same EDO-v1 order.  A token with one block
 * is folded straight into its dE row, so no block partial is written for it.
 * Needs an accumulator with no contribution (RMSNORM_ESTATE) and
 * rows == n_logical (RMSNORM_ECOVERAGE); leaves it finalized without
 * partials, so det_embedding_dw_finalize then returns RMSNORM_ESTATE until
 * det_embedding_dw_acc_reset.  dE must not alias dy. */
int det_embedding_bwd(const rmsnorm_bf16* dy, int64_t rows, int64_t dim, det_embedding_dw_acc* acc,
                      float* dE, void* stream);

int det_embedding_dw_acc_reset(det_embedding_dw_acc* acc, void* stream);
int det_embedding_dw_acc_destroy(det_embedding_dw_acc* acc);

#ifdef __cplusplus
}
#endif

#endif /* DET_EMBEDDING_BI_H */
