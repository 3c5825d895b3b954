/*
 * embedding_oracle.c -- plain, slow CPU oracle for the embedding table
 * gradient (the "Embedding / LM-head" adapter), and an FP32 emulation of
 * the canonical scatter order EDO-v1.
 *
 * TEST INFRASTRUCTURE ONLY, like the other oracle sources: no code is
 * shared with the HIP library; inputs are the same bf16 bit patterns and
 * integer token ids.
 *
 * Sources.  "[WS1 Closeout][Backward] Reusable gradient-invariance harness
 * and operator adapters", Required adapters, lists Embedding / LM-head, and
 * its Acceptance criteria ask for stable names and verdicts of the
 * embedding/LM-head weight gradients; "WS1 C4 (#270) closeout evidence"
 * (status table) lists embedding / lm_head among the candidates.  The pages
 * print no formula; the reading used is the standard lookup
 *     y[r][j] = E[id(r)][j]
 * whose VJP is the scatter-add
 *     dE[v][j] = sum over logical rows l with id(l) = v of dY[l][j].
 * Summed here in ascending logical row index (FP64), so no layout can
 * enter; tokens that do not occur get 0.  Padding rows (map value -1) are
 * not read and get y = 0.
 *
 * EDO-v1 (the order the GPU reduces in, emulated in FP32 below): for each
 * token v, its occurrences in ascending logical row index are cut into
 * blocks of 64 consecutive occurrences; a block is folded from +0.0 in
 * occurrence order (one FP32 rounding per added row); the token's block
 * partials are combined by a perfect pairwise tree with +0.0 leaves up to
 * the next power of two.
 *
 * Pins (tests/test_oracle_pins.py): a pure-Python loop on tiny inputs
 * (bitwise: exact sums), the count closed form (dY = 1 gives the token
 * histogram), linearity in dY, padding and layout invariance, refused ids;
 * EDO-v1 emulation: exact when every partial is representable, a
 * hand-derived golden case that distinguishes the block/tree order from a
 * left fold, and the FP32 error bound against FP64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EMB_OK 0
#define EMB_EINVAL (-1)
#define EMB_ELAYOUT (-3)
#define EDO_BLOCK 64

static float emb_widen(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static int emb_inverse(const int32_t* row_logical, int64_t rows, int64_t n_logical, int64_t* inv) {
    for (int64_t l = 0; l < n_logical; ++l) inv[l] = -1;
    for (int64_t p = 0; p < rows; ++p) {
        const int64_t l = row_logical ? row_logical[p] : p;
        if (l == -1) continue;
        if (l < 0 || l >= n_logical || inv[l] != -1) return EMB_ELAYOUT;
        inv[l] = p;
    }
    return EMB_OK;
}

/* y[r] = table[ids[r]] for the call's physical rows; padding rows 0. */
int oracle_embedding_fwd(const int32_t* ids, const uint16_t* table, int64_t rows, int64_t vocab,
                         int64_t dim, const int32_t* row_logical, double* y) {
    for (int64_t r = 0; r < rows; ++r) {
        const int pad = row_logical && row_logical[r] < 0;
        if (!pad && (ids[r] < 0 || ids[r] >= vocab)) return EMB_EINVAL;
        for (int64_t j = 0; j < dim; ++j)
            y[r * dim + j] = pad ? 0.0 : (double)emb_widen(table[(int64_t)ids[r] * dim + j]);
    }
    return EMB_OK;
}

/* dE[vocab][ncols] (FP64) and the matching sum of |terms| over the rows the
 * call holds, in ascending logical index; only the columns in cols[] (all
 * columns if cols is NULL, ncols = dim). */
int oracle_embedding_bwd(const int32_t* ids, const uint16_t* dy, int64_t rows, int64_t vocab,
                         int64_t dim, const int32_t* row_logical, int64_t n_logical,
                         const int64_t* cols, int64_t ncols, double* dE, double* dE_abs) {
    int64_t* inv = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_logical > 0 ? n_logical : 1));
    if (!inv) return EMB_EINVAL;
    if (emb_inverse(row_logical, rows, n_logical, inv) != EMB_OK) {
        free(inv);
        return EMB_ELAYOUT;
    }
    for (int64_t e = 0; e < vocab * ncols; ++e) {
        dE[e] = 0.0;
        dE_abs[e] = 0.0;
    }
    for (int64_t l = 0; l < n_logical; ++l) {
        const int64_t p = inv[l];
        if (p < 0) continue;
        const int64_t v = ids[p];
        if (v < 0 || v >= vocab) {
            free(inv);
            return EMB_EINVAL;
        }
        for (int64_t c = 0; c < ncols; ++c) {
            const int64_t j = cols ? cols[c] : c;
            const double g = (double)emb_widen(dy[p * dim + j]);
            dE[v * ncols + c] += g;
            dE_abs[v * ncols + c] += fabs(g);
        }
    }
    free(inv);
    return EMB_OK;
}

/* perfect pairwise tree over q[0..n), +0.0 past n, n padded to a power of two */
static float edo_tree(const float* q, int64_t n, int64_t lo, int64_t width) {
    if (width == 1) return lo < n ? q[lo] : 0.0f;
    const int64_t h = width / 2;
    const float a = edo_tree(q, n, lo, h);
    const float b = edo_tree(q, n, lo + h, h);
    return a + b;
}

/* FP32 emulation of EDO-v1 on logical-order inputs (ids[n_logical],
 * dy[n_logical][dim]): out[vocab][dim]. */
int oracle_edo_v1_f32(const int32_t* ids, const uint16_t* dy, int64_t n_logical, int64_t vocab,
                      int64_t dim, float* out) {
    for (int64_t e = 0; e < vocab * dim; ++e) out[e] = 0.0f;
    int64_t* cnt = (int64_t*)calloc((size_t)vocab + 1, sizeof(int64_t));
    int64_t* occ = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_logical > 0 ? n_logical : 1));
    int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(vocab + 1));
    if (!cnt || !occ || !pos) {
        free(cnt); free(occ); free(pos);
        return EMB_EINVAL;
    }
    for (int64_t l = 0; l < n_logical; ++l) {
        if (ids[l] < 0 || ids[l] >= vocab) {
            free(cnt); free(occ); free(pos);
            return EMB_EINVAL;
        }
        cnt[ids[l] + 1]++;
    }
    for (int64_t v = 0; v < vocab; ++v) cnt[v + 1] += cnt[v];     /* start of each token's list */
    for (int64_t v = 0; v <= vocab; ++v) pos[v] = cnt[v];
    for (int64_t l = 0; l < n_logical; ++l) occ[pos[ids[l]]++] = l; /* ascending l within a token */
    for (int64_t v = 0; v < vocab; ++v) {
        const int64_t a = cnt[v], n = cnt[v + 1] - cnt[v];
        if (n == 0) continue;
        const int64_t nb = (n + EDO_BLOCK - 1) / EDO_BLOCK;
        int64_t width = 1;
        while (width < nb) width *= 2;
        float* q = (float*)malloc(sizeof(float) * (size_t)nb);
        for (int64_t j = 0; j < dim; ++j) {
            for (int64_t b = 0; b < nb; ++b) {
                float acc = 0.0f;
                for (int64_t i = b * EDO_BLOCK; i < n && i < (b + 1) * EDO_BLOCK; ++i)
                    acc = acc + emb_widen(dy[occ[a + i] * dim + j]);
                q[b] = acc;
            }
            out[v * dim + j] = edo_tree(q, nb, 0, width);
        }
        free(q);
    }
    free(cnt); free(occ); free(pos);
    return EMB_OK;
}
