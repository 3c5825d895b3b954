/*
 * rmsnorm_oracle.c -- plain, slow FP64 CPU oracle for RMSNorm forward and
 * backward (dx, dweight), plus an FP32 emulation of the canonical dweight
 * order CDO-v2.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no source,
 * header, table or helper with the HIP library; it receives the same bf16
 * bit patterns and widens them exactly.
 *
 * Sources.  The operation is the RMSNorm whose "dx/dweight" gradients are a
 * required adapter in "[WS1 Closeout][Backward] Reusable gradient-invariance
 * harness and operator adapters" (section "Required adapters").  The pages
 * never print the formula; the reading used here is the standard one:
 *     rstd = 1 / sqrt(mean_j x_j^2 + eps),   y_j = x_j * rstd * w_j,
 * with eps inside the square root and a plain (not 1+w) weight.  Its VJP:
 *     dot  = sum_j dy_j w_j x_j
 *     dx_j = rstd * (dy_j w_j - x_j * rstd^2 * dot / H)
 *     dweight_j = sum over rows of dy_j * x_j * rstd.
 * "WS1 C4 (#270) closeout evidence", section "Historical finding -- RMSNorm
 * dweight is not chunk/batch decomposable", is the reason dweight is defined
 * over *logical* rows: this oracle always sums rows in ascending logical
 * index, so its output cannot depend on the physical layout.  Rows marked
 * -1 (padding) are never read and produce zeros ("Acceptance map": inactive
 * tokens contribute 0).
 *
 * Pins (tests/test_oracle_pins.py): explicit Jacobian, central finite
 * differences of the FP64 forward, the radial identity sum_j x_j dx_j =
 * eps*rstd^3*dot, the dx/dweight cross identity, H=1 and zero-row closed
 * forms, scale invariance and the norm identity of the forward, padding
 * neutrality and layout invariance.  The CDO-v2 emulation is pinned by
 * exactly representable sums and a hand-derived golden case
 * (tests/golden/cdo_v2_order.json).  Nothing here is "parity unpinned".
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared (no fast-math:
 * every float operation below must round exactly once as written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ELAYOUT (-3)

/* bf16 is the upper half of an IEEE binary32: widening is exact. */
static float bf16_bits_to_float(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

void oracle_widen_bf16(const uint16_t* in, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (double)bf16_bits_to_float(in[i]);
}

/* bf16 bit pattern nearest to a finite double: round to FP32 (nearest even),
 * then keep the upper half, rounding to nearest even on the dropped half.
 * This is how a bf16 activation is stored between two ops of a chain. */
void oracle_round_bf16(const double* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) {
        const float f = (float)in[i];
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        const uint32_t lsb = (u >> 16) & 1u;
        out[i] = (uint16_t)((u + 0x7FFFu + lsb) >> 16);
    }
}

/* Inverse of a physical->logical row map.  Every value must be -1 (padding)
 * or a logical index in [0, n_logical), each logical index at most once.
 * inv[l] = physical row holding logical row l, or -1 if this call does not
 * hold it. */
static int invert_layout(const int32_t* row_logical, int64_t rows, int64_t n_logical,
                         int64_t* inv) {
    for (int64_t l = 0; l < n_logical; ++l) inv[l] = -1;
    for (int64_t p = 0; p < rows; ++p) {
        int64_t l = row_logical ? (int64_t)row_logical[p] : p;
        if (l == -1) continue;
        if (l < 0 || l >= n_logical) return ORACLE_ELAYOUT;
        if (inv[l] != -1) return ORACLE_ELAYOUT;
        inv[l] = p;
    }
    return ORACLE_OK;
}

static int is_pad(const int32_t* row_logical, int64_t p) {
    return row_logical != NULL && row_logical[p] < 0;
}

/* rstd of one row, straight from the definition. */
static double row_rstd(const double* xr, int64_t H, double eps) {
    double ss = 0.0;
    for (int64_t j = 0; j < H; ++j) ss += xr[j] * xr[j];
    return 1.0 / sqrt(ss / (double)H + eps);
}

/* Forward.  y[p][j] = x[p][j] * rstd[p] * w[j]; padding rows give y = 0 and
 * rstd = 0. */
int oracle_rmsnorm_fwd(const double* x, const double* w, int64_t rows, int64_t H, double eps,
                       const int32_t* row_logical, double* y, double* rstd) {
    if (rows < 0 || H <= 0 || eps < 0.0) return ORACLE_EINVAL;
    for (int64_t p = 0; p < rows; ++p) {
        const double* xr = x + p * H;
        double* yr = y + p * H;
        if (is_pad(row_logical, p)) {
            for (int64_t j = 0; j < H; ++j) yr[j] = 0.0;
            rstd[p] = 0.0;
            continue;
        }
        double r = row_rstd(xr, H, eps);
        for (int64_t j = 0; j < H; ++j) yr[j] = xr[j] * r * w[j];
        rstd[p] = r;
    }
    return ORACLE_OK;
}

/* Backward.  dx per physical row (zeros for padding); dweight and the
 * absolute-sum scale dweight_abs[j] = sum |dy_j x_j rstd| summed over the
 * logical rows this call holds, in ascending logical index.  row_logical may
 * be NULL (identity: logical row = physical row, n_logical = rows). */
int oracle_rmsnorm_bwd(const double* x, const double* w, const double* dy, int64_t rows,
                       int64_t H, double eps, const int32_t* row_logical, int64_t n_logical,
                       double* dx, double* dweight, double* dweight_abs) {
    if (rows < 0 || H <= 0 || eps < 0.0 || n_logical < 0) return ORACLE_EINVAL;
    if (row_logical == NULL) n_logical = rows;
    int64_t* inv = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_logical > 0 ? n_logical : 1));
    if (!inv) return ORACLE_EINVAL;
    int rc = invert_layout(row_logical, rows, n_logical, inv);
    if (rc != ORACLE_OK) {
        free(inv);
        return rc;
    }

    for (int64_t p = 0; p < rows; ++p) {
        const double* xr = x + p * H;
        const double* dyr = dy + p * H;
        double* dxr = dx + p * H;
        if (is_pad(row_logical, p)) {
            for (int64_t j = 0; j < H; ++j) dxr[j] = 0.0;
            continue;
        }
        double r = row_rstd(xr, H, eps);
        double dot = 0.0;
        for (int64_t j = 0; j < H; ++j) dot += dyr[j] * w[j] * xr[j];
        for (int64_t j = 0; j < H; ++j) dxr[j] = r * (dyr[j] * w[j] - xr[j] * r * r * dot / (double)H);
    }

    for (int64_t j = 0; j < H; ++j) {
        dweight[j] = 0.0;
        if (dweight_abs) dweight_abs[j] = 0.0;
    }
    for (int64_t l = 0; l < n_logical; ++l) {
        int64_t p = inv[l];
        if (p < 0) continue;
        const double* xr = x + p * H;
        const double* dyr = dy + p * H;
        double r = row_rstd(xr, H, eps);
        for (int64_t j = 0; j < H; ++j) {
            double t = dyr[j] * xr[j] * r;
            dweight[j] += t;
            if (dweight_abs) dweight_abs[j] += fabs(t);
        }
    }
    free(inv);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * CDO-v2: the canonical FP32 order in which dweight is reduced.  The pages
 * fix only that parameter gradients are built from one FP32 contribution per
 * logical row and reduced in an order that never changes ("WS1 C4 (#270)
 * closeout evidence", opening note and Acceptance map); the order below is
 * this project's reading of that, written out plainly:
 *   c[l][j] = fl32(fl32(dy * x) * rstd)    one value per logical row; dy*x
 *       of two bf16 values is exact in FP32, so c is dy*x*rstd rounded once
 *   block b holds logical rows 64b .. 64b+63; slot s = l - 64b
 *   stream w (0..3) folds slots w, w+4, w+8, ..., w+60 in ascending order,
 *       starting from +0.0; a slot the accumulation does not hold adds +0.0
 *   P[b] = (q0+q1)+(q2+q3)
 *   dweight = perfect pairwise tree over P[0 .. 2^ceil(log2 nb)),
 *       leaves past nb being +0.0.
 * This emulation exists so the GPU result can be compared bit for bit.
 * ---------------------------------------------------------------------- */

#define CDO_BLOCK 64
#define CDO_STREAMS 4

/* Pairwise tree over leaves[lo .. lo+n), n a power of two, leaves at or past
 * nb counting as +0.0. */
static float cdo_tree(const float* leaves, int64_t nb, int64_t lo, int64_t n) {
    if (n == 1) return lo < nb ? leaves[lo] : 0.0f;
    float a = cdo_tree(leaves, nb, lo, n / 2);
    float b = cdo_tree(leaves, nb, lo + n / 2, n / 2);
    return a + b;
}

int oracle_cdo_v2_dweight_f32(const uint16_t* x, const uint16_t* dy, const float* rstd,
                              int64_t rows, int64_t H, const int32_t* row_logical,
                              int64_t n_logical, float* dweight) {
    if (rows < 0 || H <= 0 || n_logical < 0) return ORACLE_EINVAL;
    if (row_logical == NULL) n_logical = rows;
    int64_t* inv = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_logical > 0 ? n_logical : 1));
    if (!inv) return ORACLE_EINVAL;
    int rc = invert_layout(row_logical, rows, n_logical, inv);
    if (rc != ORACLE_OK) {
        free(inv);
        return rc;
    }
    int64_t nb = (n_logical + CDO_BLOCK - 1) / CDO_BLOCK;
    int64_t npad = 1;
    while (npad < nb) npad *= 2;
    float* P = (float*)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
    if (!P) {
        free(inv);
        return ORACLE_EINVAL;
    }
    for (int64_t j = 0; j < H; ++j) {
        for (int64_t b = 0; b < nb; ++b) {
            float q[CDO_STREAMS];
            for (int w = 0; w < CDO_STREAMS; ++w) {
                float acc = 0.0f;
                for (int s = w; s < CDO_BLOCK; s += CDO_STREAMS) {
                    int64_t l = b * CDO_BLOCK + s;
                    if (l >= n_logical || inv[l] < 0) continue;
                    int64_t p = inv[l];
                    float xv = bf16_bits_to_float(x[p * H + j]);
                    float dyv = bf16_bits_to_float(dy[p * H + j]);
                    float prod = dyv * xv; /* exact: two 8-bit significands */
                    float c = prod * rstd[p];
                    acc = acc + c;
                }
                q[w] = acc;
            }
            P[b] = (q[0] + q[1]) + (q[2] + q[3]);
        }
        dweight[j] = nb > 0 ? cdo_tree(P, nb, 0, npad) : 0.0f;
    }
    free(P);
    free(inv);
    return ORACLE_OK;
}
