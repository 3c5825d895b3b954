/*
 * linear_oracle.c -- plain, slow FP64 CPU oracle for the backward of a
 * linear layer (the "GEMM dX/dW" adapter).
 *
 * TEST INFRASTRUCTURE ONLY, like rmsnorm_oracle.c: it shares no source,
 * header, table or helper with the HIP library and receives the same bf16
 * bit patterns, widened exactly.
 *
 * Sources.  "[WS1 Closeout][Backward] Reusable gradient-invariance harness
 * and operator adapters", section "Required adapters", lists GEMM dX/dW
 * among the required gradients; "WS1 C4 (#270) closeout evidence" (status
 * table and the note on the reds) puts the deterministic GEMM's dW in the
 * same failure class as RMSNorm's dweight; its fix builds parameter
 * gradients from one FP32 contribution per logical row.  The pages print no
 * formula; the reading used is the standard linear layer
 *     y[r][n]  = sum_k x[r][k] * W[n][k]          (y = x W^T)
 * with x[rows][K], W[N][K], y[rows][N], and its VJP
 *     dX[r][k] = sum_n dY[r][n] * W[n][k]         (dX = dY W)
 *     dW[n][k] = sum over logical rows l of dY[l][n] * X[l][k]   (dW = dY^T X).
 * dX is row-local; dW is summed here in ascending logical row index (the
 * physical layout cannot enter).  Padding rows (map value -1) are never read
 * and get y = dX = 0.
 *
 * Pins (tests/test_oracle_pins.py): a pure-Python triple loop on tiny
 * inputs (bitwise: every partial sum is exact there), a single row
 * (dW = outer product, exact), the identity weight (dX = dY, exact), the
 * trace identity <dY, X W^T> = <dW, W> = <dX, X>, central differences of
 * that bilinear form, padding neutrality and layout invariance.
 *
 * Build: compiled together with rmsnorm_oracle.c (gcc -O2 -std=c11
 * -ffp-contract=off, no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LIN_OK 0
#define LIN_EINVAL (-1)
#define LIN_ELAYOUT (-3)

static double lin_widen(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* physical row of every logical row (-1 if the call lacks it); validates the map */
static int lin_inverse(const int32_t* row_logical, int64_t rows, int64_t n_logical, int64_t* inv) {
    for (int64_t l = 0; l < n_logical; ++l) inv[l] = -1;
    for (int64_t p = 0; p < rows; ++p) {
        const int64_t l = row_logical ? row_logical[p] : p;
        if (l == -1) continue;
        if (l < 0 || l >= n_logical || inv[l] != -1) return LIN_ELAYOUT;
        inv[l] = p;
    }
    return LIN_OK;
}

/* y = x W^T on the physical rows; padding rows get 0. */
int oracle_linear_fwd(const uint16_t* x, const uint16_t* w, int64_t rows, int64_t n, int64_t k,
                      const int32_t* row_logical, double* y) {
    if (rows < 0 || n <= 0 || k <= 0) return LIN_EINVAL;
    for (int64_t r = 0; r < rows; ++r) {
        const int pad = row_logical && row_logical[r] < 0;
        for (int64_t o = 0; o < n; ++o) {
            double s = 0.0;
            if (!pad)
                for (int64_t i = 0; i < k; ++i) s += lin_widen(x[r * k + i]) * lin_widen(w[o * k + i]);
            y[r * n + o] = s;
        }
    }
    return LIN_OK;
}

/* dX for the call's physical rows, and dW / |dW| over the rows the call holds
 * in ascending logical index. */
int oracle_linear_bwd(const uint16_t* x, const uint16_t* w, const uint16_t* dy, int64_t rows,
                      int64_t n, int64_t k, const int32_t* row_logical, int64_t n_logical,
                      double* dx, double* dw, double* dw_abs) {
    if (rows < 0 || n <= 0 || k <= 0 || n_logical < 0) return LIN_EINVAL;
    int64_t* inv = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_logical > 0 ? n_logical : 1));
    if (!inv) return LIN_EINVAL;
    if (lin_inverse(row_logical, rows, n_logical, inv) != LIN_OK) {
        free(inv);
        return LIN_ELAYOUT;
    }
    for (int64_t r = 0; r < rows; ++r) {
        const int pad = row_logical && row_logical[r] < 0;
        for (int64_t i = 0; i < k; ++i) {
            double s = 0.0;
            if (!pad)
                for (int64_t o = 0; o < n; ++o) s += lin_widen(dy[r * n + o]) * lin_widen(w[o * k + i]);
            dx[r * k + i] = s;
        }
    }
    for (int64_t e = 0; e < n * k; ++e) {
        dw[e] = 0.0;
        dw_abs[e] = 0.0;
    }
    for (int64_t l = 0; l < n_logical; ++l) {
        const int64_t p = inv[l];
        if (p < 0) continue;
        for (int64_t o = 0; o < n; ++o) {
            const double g = lin_widen(dy[p * n + o]);
            for (int64_t i = 0; i < k; ++i) {
                const double c = g * lin_widen(x[p * k + i]);
                dw[o * k + i] += c;
                dw_abs[o * k + i] += fabs(c);
            }
        }
    }
    free(inv);
    return LIN_OK;
}

/* Single outputs of an identity-layout call, one at a time (for sizes whose
 * full products are too slow here): kind 0 = dX[a][b], kind 1 = dW[a][b]
 * (summed over all rows in ascending order), kind 2 = |dW|[a][b], kind 3 =
 * y[a][b] (row a of x against row b of W, the forward y = x W^T). */
int oracle_linear_sample(const uint16_t* x, const uint16_t* w, const uint16_t* dy, int64_t rows,
                         int64_t n, int64_t k, int64_t count, const int32_t* kind,
                         const int64_t* ia, const int64_t* ib, double* out) {
    for (int64_t s = 0; s < count; ++s) {
        double acc = 0.0;
        if (kind[s] == 0) {
            const int64_t r = ia[s], i = ib[s];
            if (r < 0 || r >= rows || i < 0 || i >= k) return LIN_EINVAL;
            for (int64_t o = 0; o < n; ++o) acc += lin_widen(dy[r * n + o]) * lin_widen(w[o * k + i]);
        } else if (kind[s] == 1 || kind[s] == 2) {
            const int64_t o = ia[s], i = ib[s];
            if (o < 0 || o >= n || i < 0 || i >= k) return LIN_EINVAL;
            for (int64_t r = 0; r < rows; ++r) {
                const double c = lin_widen(dy[r * n + o]) * lin_widen(x[r * k + i]);
                acc += kind[s] == 1 ? c : fabs(c);
            }
        } else if (kind[s] == 3) {
            const int64_t r = ia[s], o = ib[s];
            if (r < 0 || r >= rows || o < 0 || o >= n) return LIN_EINVAL;
            for (int64_t i = 0; i < k; ++i) acc += lin_widen(x[r * k + i]) * lin_widen(w[o * k + i]);
        } else {
            return LIN_EINVAL;
        }
        out[s] = acc;
    }
    return LIN_OK;
}
