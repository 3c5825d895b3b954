"""Pins of the FP64 oracle against facts other than itself.

Each test checks the oracle against mathematics it does not restate: brute
force (central finite differences of the forward), closed forms of special
cases (constant rows, H = 1, zero rows), invariants (scale invariance,
Euler/homogeneity identities, orthogonality of dx to x when eps = 0), exact
bit patterns, and the hand-derived CDO-v2 golden case.  A plausible mistake
(a dropped term, a wrong sign or index, eps outside the square root, a sum
instead of a mean, the wrong fold order) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _loss(orc, x, w, u, eps, rl=None):
    y, _ = orc.rmsnorm_fwd(x, w, eps, rl)
    return float(np.sum(u * y))


# ------------------------------------------------------------------ widening
def pin_widen_bf16_exact_bit_patterns(orc):
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x4380, 0x3780],
                    dtype=np.uint16)
    got = orc.widen_bf16(bits)
    want = [1.0, -1.0, 3.140625, 0.0, -0.0, math.inf, -math.inf, 2.0 ** -133, 256.0, 2.0 ** -16]
    assert list(got) == want
    assert math.copysign(1.0, got[4]) == -1.0


# ------------------------------------------------------------------- forward
def pin_forward_constant_row_closed_form(orc):
    # x = c * 1  =>  rstd = (c^2 + eps)^-1/2 ; c = 3, eps = 7 gives exactly 1/4.
    H = 6
    x = np.full((1, H), 3.0)
    w = _rng(1).uniform(0.5, 1.5, H)
    y, rstd = orc.rmsnorm_fwd(x, w, 7.0)
    assert rstd[0] == 0.25
    np.testing.assert_array_equal(y[0], 0.75 * w)


def pin_forward_zero_row_and_eps_inside_sqrt(orc):
    x = np.zeros((1, 4))
    w = np.ones(4)
    y, rstd = orc.rmsnorm_fwd(x, w, 0.25)
    assert rstd[0] == 2.0            # eps^-1/2, not 1/eps
    assert np.all(y == 0.0)


def pin_forward_two_element_worked_example(orc):
    # x = (3, 4), eps = 0: mean square 12.5, rstd = 1/sqrt(12.5) = sqrt(2)/5.
    y, rstd = orc.rmsnorm_fwd(np.array([[3.0, 4.0]]), np.array([1.0, 0.5]), 0.0)
    assert rstd[0] == pytest.approx(math.sqrt(2.0) / 5.0, rel=1e-15)
    assert y[0, 0] == pytest.approx(3.0 * math.sqrt(2.0) / 5.0, rel=1e-15)
    assert y[0, 1] == pytest.approx(0.5 * 4.0 * math.sqrt(2.0) / 5.0, rel=1e-15)


def pin_forward_norm_identity_and_scale_invariance(orc):
    # eps = 0: sum_j (y_j / w_j)^2 = H exactly in exact arithmetic, and y is
    # invariant to scaling x.
    rng = _rng(2)
    H = 37
    x = rng.normal(size=(5, H))
    w = rng.uniform(0.5, 1.5, H)
    y, _ = orc.rmsnorm_fwd(x, w, 0.0)
    np.testing.assert_allclose(np.sum((y / w) ** 2, axis=1), H, rtol=1e-13)
    y2, _ = orc.rmsnorm_fwd(x * 1024.0, w, 0.0)
    np.testing.assert_allclose(y2, y, rtol=1e-14, atol=0)
    # eps > 0 shrinks the norm below H and the shrink vanishes for large x.
    y3, _ = orc.rmsnorm_fwd(x * 1e-3, w, 1e-6)
    assert np.all(np.sum((y3 / w) ** 2, axis=1) < H)


# ------------------------------------------------------------------ backward
def _fd_grads(orc, x, w, u, eps, h_rel=1e-6):
    gx = np.zeros_like(x)
    for i in range(x.shape[0]):
        for j in range(x.shape[1]):
            h = h_rel * max(1.0, abs(x[i, j]))
            xp = x.copy(); xp[i, j] += h
            xm = x.copy(); xm[i, j] -= h
            gx[i, j] = (_loss(orc, xp, w, u, eps) - _loss(orc, xm, w, u, eps)) / (2 * h)
    gw = np.zeros_like(w)
    for j in range(w.shape[0]):
        h = h_rel * max(1.0, abs(w[j]))
        wp = w.copy(); wp[j] += h
        wm = w.copy(); wm[j] -= h
        gw[j] = (_loss(orc, x, wp, u, eps) - _loss(orc, x, wm, u, eps)) / (2 * h)
    return gx, gw


def pin_backward_matches_central_finite_differences_h8_t59(orc, eps):
    """Brute force on the hidden=8, 59-row shape of the page's matrix."""
    from invariant_rmsnorm_backward_amd import inputs
    wl = inputs.workload_h8()
    x = orc.widen_bf16(inputs.bf16_bits(inputs.gen_x(wl)))
    w = orc.widen_bf16(inputs.bf16_bits(inputs.gen_w(wl)))
    u = orc.widen_bf16(inputs.bf16_bits(inputs.gen_dy(wl)))
    dx, dw, _ = orc.rmsnorm_bwd(x, w, u, eps)
    gx, gw = _fd_grads(orc, x, w, u, eps)
    sx = np.max(np.abs(dx))
    sw = np.max(np.abs(dw))
    assert np.all(np.abs(gx - dx) <= 1e-7 * (np.abs(dx) + sx))
    assert np.all(np.abs(gw - dw) <= 1e-7 * (np.abs(dw) + sw))


def pin_backward_explicit_jacobian(orc):
    """dx = J^T dy, with the Jacobian J_ij = d y_i / d x_j built column by
    column by central differences of the forward.  J is not symmetric (row i
    carries w_i), so using J instead of J^T fails."""
    rng = _rng(3)
    H = 16
    x = rng.normal(size=(1, H))
    w = rng.uniform(0.5, 1.5, H)
    dy = rng.normal(size=(1, H))
    eps = 1e-3
    J = np.zeros((H, H))
    for j in range(H):
        h = 1e-6
        xp = x.copy(); xp[0, j] += h
        xm = x.copy(); xm[0, j] -= h
        J[:, j] = (orc.rmsnorm_fwd(xp, w, eps)[0][0] - orc.rmsnorm_fwd(xm, w, eps)[0][0]) / (2 * h)
    dx, dw, _ = orc.rmsnorm_bwd(x, w, dy, eps)
    np.testing.assert_allclose(dx[0], J.T @ dy[0], rtol=1e-7, atol=1e-9)


def pin_backward_orthogonality_and_radial_identity(orc):
    rng = _rng(4)
    H = 64
    x = rng.normal(size=(7, H))
    w = rng.uniform(0.5, 1.5, H)
    dy = rng.normal(size=(7, H))
    # eps = 0: y is scale invariant in x, so (Euler) sum_j x_j dx_j = 0.
    dx, _, _ = orc.rmsnorm_bwd(x, w, dy, 0.0)
    dots = np.sum(x * dx, axis=1)
    assert np.all(np.abs(dots) <= 1e-12 * np.sum(np.abs(x * dx), axis=1))
    # eps > 0: d/dt L(t x) at t = 1 equals sum_j x_j dx_j; check by a 1-D
    # central difference along the ray, row by row.
    eps = 0.3
    dx, _, _ = orc.rmsnorm_bwd(x, w, dy, eps)
    for i in range(7):
        xi = x[i:i + 1]
        ui = dy[i:i + 1]
        h = 1e-6
        fd = (_loss(orc, xi * (1 + h), w, ui, eps) - _loss(orc, xi * (1 - h), w, ui, eps)) / (2 * h)
        assert fd == pytest.approx(np.sum(xi * dx[i]), rel=1e-7, abs=1e-10)


def pin_dweight_euler_identity(orc):
    # y is linear in w, so sum_j w_j dL/dw_j = L = sum y * dy.
    rng = _rng(5)
    H = 24
    x = rng.normal(size=(11, H))
    w = rng.uniform(0.5, 1.5, H)
    dy = rng.normal(size=(11, H))
    eps = 1e-6
    _, dw, dwa = orc.rmsnorm_bwd(x, w, dy, eps)
    L = _loss(orc, x, w, dy, eps)
    assert float(np.dot(w, dw)) == pytest.approx(L, rel=1e-12)
    assert np.all(dwa >= np.abs(dw))


def pin_h1_closed_form(orc):
    # H = 1: y = w x / sqrt(x^2 + eps); dy/dx = w eps / (x^2 + eps)^(3/2).
    x = np.array([[0.7], [-2.0], [0.0]])
    w = np.array([1.3])
    dy = np.array([[0.5], [-1.5], [2.0]])
    eps = 0.09
    dx, dw, _ = orc.rmsnorm_bwd(x, w, dy, eps)
    for i in range(3):
        xv = x[i, 0]
        assert dx[i, 0] == pytest.approx(dy[i, 0] * 1.3 * eps / (xv * xv + eps) ** 1.5, rel=1e-14)
    want_dw = sum(dy[i, 0] * x[i, 0] / math.sqrt(x[i, 0] ** 2 + eps) for i in range(3))
    assert dw[0] == pytest.approx(want_dw, rel=1e-14)


def pin_zero_row_backward(orc):
    H = 8
    x = np.zeros((1, H))
    w = _rng(6).uniform(0.5, 1.5, H)
    dy = _rng(7).normal(size=(1, H))
    dx, dw, _ = orc.rmsnorm_bwd(x, w, dy, 0.25)
    np.testing.assert_array_equal(dx[0], 2.0 * dy[0] * w)      # rstd = 2
    assert np.all(dw == 0.0)


# ------------------------------------------------------ padding and layouts
def pin_padding_rows_are_never_read_and_contribute_nothing(orc):
    rng = _rng(8)
    H = 16
    x = rng.normal(size=(9, H))
    w = rng.uniform(0.5, 1.5, H)
    dy = rng.normal(size=(9, H))
    eps = 1e-6
    # physical: 2 pads, 9 real rows in order, 3 pads; pads hold NaN / Inf.
    rl = np.array([-1, -1] + list(range(9)) + [-1, -1, -1], dtype=np.int32)
    xp = np.full((14, H), np.nan); xp[2:11] = x; xp[11] = np.inf
    dyp = np.full((14, H), np.inf); dyp[2:11] = dy
    y0, r0 = orc.rmsnorm_fwd(x, w, eps)
    y1, r1 = orc.rmsnorm_fwd(xp, w, eps, rl)
    np.testing.assert_array_equal(y1[2:11], y0)
    assert np.all(y1[rl < 0] == 0) and np.all(r1[rl < 0] == 0)
    np.testing.assert_array_equal(r1[2:11], r0)
    dx0, dw0, _ = orc.rmsnorm_bwd(x, w, dy, eps)
    dx1, dw1, _ = orc.rmsnorm_bwd(xp, w, dyp, eps, rl, 9)
    np.testing.assert_array_equal(dx1[2:11], dx0)
    assert np.all(dx1[rl < 0] == 0)
    np.testing.assert_array_equal(dw1, dw0)


def pin_inactive_rows_contribute_exactly_zero(orc):
    rng = _rng(9)
    H = 16
    x = rng.normal(size=(12, H))
    w = rng.uniform(0.5, 1.5, H)
    dy = rng.normal(size=(12, H))
    inactive = np.array([1, 4, 5, 10])
    dy[inactive] = 0.0
    dy[inactive[:2]] = -0.0
    _, dw_all, _ = orc.rmsnorm_bwd(x, w, dy, 1e-6)
    keep = np.setdiff1d(np.arange(12), inactive)
    rl = np.full(12, -1, dtype=np.int32)
    rl[keep] = np.arange(len(keep))
    _, dw_act, _ = orc.rmsnorm_bwd(x, w, dy, 1e-6, rl, len(keep))
    np.testing.assert_array_equal(dw_all, dw_act)


def pin_oracle_is_layout_invariant(orc):
    rng = _rng(10)
    H, T = 24, 40
    x = rng.normal(size=(T, H))
    w = rng.uniform(0.5, 1.5, H)
    dy = rng.normal(size=(T, H))
    dx0, dw0, _ = orc.rmsnorm_bwd(x, w, dy, 1e-6)
    perm = rng.permutation(T)
    rl = perm.astype(np.int32)            # physical row p holds logical row perm[p]
    dx1, dw1, _ = orc.rmsnorm_bwd(x[perm], w, dy[perm], 1e-6, rl, T)
    np.testing.assert_array_equal(dw1, dw0)
    restored = np.empty_like(dx1)
    restored[perm] = dx1
    np.testing.assert_array_equal(restored, dx0)


def pin_invalid_layouts_are_refused(orc):
    x = np.ones((3, 8)); w = np.ones(8); dy = np.ones((3, 8))
    with pytest.raises(oracle.OracleError):
        orc.rmsnorm_bwd(x, w, dy, 1e-6, np.array([0, 0, 1], np.int32), 3)   # duplicate
    with pytest.raises(oracle.OracleError):
        orc.rmsnorm_bwd(x, w, dy, 1e-6, np.array([0, 1, 3], np.int32), 3)   # out of range


# ------------------------------------------------------------ CDO-v2 (FP32)
def _golden_cases():
    with open(os.path.join(GOLDEN, "cdo_v2_order.json")) as f:
        g = json.load(f)
    out = []
    for c in g["cases"]:
        T, H = c["n_logical"], c["hidden"]
        x = np.full((T, H), int(c["x_bits_default"], 16), dtype=np.uint16)
        for e in c["x_overrides"]:
            x[e["row"], e["col"]] = int(e["bits"], 16)
        dy = np.zeros((T, H), dtype=np.uint16)
        for e in c["dy_nonzero"]:
            dy[e["row"], e["col"]] = int(e["bits"], 16)
        rbits = np.full(T, int(c["rstd_bits_default"], 16), dtype=np.uint32)
        for e in c["rstd_overrides"]:
            rbits[e["row"]] = int(e["bits"], 16)
        out.append((c, x, dy, rbits.view(np.float32)))
    return out


def _expected(c):
    if "expected_cdo_v2" in c:
        return c["expected_cdo_v2"]
    want = [0.0] * c["hidden"]
    for col, v in c["expected_cdo_v2_sparse"].items():
        want[int(col)] = v
    return want


def pin_cdo_v2_golden_cases(orc):
    for c, x, dy, rstd in _golden_cases():
        got = orc.cdo_v2_dweight_f32(x, dy, rstd)
        assert [float(v) for v in got] == _expected(c), c["name"]
    # the order case really distinguishes the order: a logical left fold differs
    c, x, dy, rstd = _golden_cases()[0]
    left = np.zeros(c["hidden"], dtype=np.float32)
    for row in orc.widen_bf16(dy).astype(np.float32):
        left = (left + row).astype(np.float32)
    assert [float(v) for v in left] == c["expected_logical_left_fold"]


def pin_cdo_v2_golden_cases_are_layout_invariant(orc):
    for c, x, dy, rstd in _golden_cases():
        T = c["n_logical"]
        perm = _rng(11).permutation(T)
        got = orc.cdo_v2_dweight_f32(x[perm], dy[perm], rstd[perm], perm.astype(np.int32), T)
        assert [float(v) for v in got] == _expected(c), c["name"]


def pin_cdo_v2_exact_when_every_partial_is_representable(orc):
    # small integers: every partial sum is exact in FP32, so the canonical
    # order must reproduce the exact (FP64) dweight bit for bit.
    rng = _rng(12)
    T, H = 777, 40
    xv = rng.integers(-4, 5, size=(T, H)).astype(np.float32)
    dyv = rng.integers(-4, 5, size=(T, H)).astype(np.float32)
    to_bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    x, dy = to_bits(xv), to_bits(dyv)
    rstd = np.ones(T, dtype=np.float32)
    got = orc.cdo_v2_dweight_f32(x, dy, rstd)
    exact = np.sum(xv.astype(np.float64) * dyv.astype(np.float64), axis=0)
    np.testing.assert_array_equal(got.astype(np.float64), exact)


def pin_cdo_v2_within_fp32_error_bound_of_fp64(orc):
    from invariant_rmsnorm_backward_amd import inputs
    wl = inputs.scaled(inputs.workload_h8(), "h64_t1000", hidden=64, lengths=[300, 200, 500])
    xb = inputs.bf16_bits(inputs.gen_x(wl))
    wb = inputs.bf16_bits(inputs.gen_w(wl))
    dyb = inputs.bf16_bits(inputs.gen_dy(wl))
    _, rstd64 = orc.rmsnorm_fwd_bf16(xb, wb, wl.eps)
    rstd32 = rstd64.astype(np.float32)
    got = orc.cdo_v2_dweight_f32(xb, dyb, rstd32).astype(np.float64)
    # exact-in-FP64 reference with the same FP32 rstd
    x = orc.widen_bf16(xb); dy = orc.widen_bf16(dyb)
    terms = dy * x * rstd32.astype(np.float64)[:, None]
    ref = terms.sum(axis=0)
    scale = np.abs(terms).sum(axis=0)
    T = wl.n_logical
    depth = 2 + 8 + 3 + int(math.ceil(math.log2(max(1, (T + 63) // 64))))
    assert np.all(np.abs(got - ref) <= depth * 2.0 ** -24 * scale * 1.01)


# -------------------------------------------------------- linear layer (GEMM)
def _bits(vals) -> np.ndarray:
    """bf16 bit patterns of float values that bf16 represents exactly."""
    f = np.asarray(vals, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _val(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rand_bf16(rng, shape, scale=1.0):
    """Random bf16 patterns of N(0, scale^2) values (rounded by truncation)."""
    f = (rng.normal(size=shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def pin_linear_brute_force_tiny(orc):
    """Triple loops in Python floats over values k/8 in [-2, 2]: every partial
    sum is exact, so the oracle must agree bit for bit."""
    rng = _rng(20)
    R, N, K = 5, 3, 4
    x = _bits(rng.integers(-16, 17, size=(R, K)) / 8.0)
    w = _bits(rng.integers(-16, 17, size=(N, K)) / 8.0)
    dy = _bits(rng.integers(-16, 17, size=(R, N)) / 8.0)
    X, W, DY = _val(x), _val(w), _val(dy)
    y = [[sum(X[r][k] * W[n][k] for k in range(K)) for n in range(N)] for r in range(R)]
    dx = [[sum(DY[r][n] * W[n][k] for n in range(N)) for k in range(K)] for r in range(R)]
    dw = [[sum(DY[r][n] * X[r][k] for r in range(R)) for k in range(K)] for n in range(N)]
    np.testing.assert_array_equal(orc.linear_fwd_bf16(x, w), np.array(y))
    gdx, gdw, gabs = orc.linear_bwd_bf16(x, w, dy)
    np.testing.assert_array_equal(gdx, np.array(dx))
    np.testing.assert_array_equal(gdw, np.array(dw))
    absum = [[sum(abs(DY[r][n] * X[r][k]) for r in range(R)) for k in range(K)] for n in range(N)]
    np.testing.assert_array_equal(gabs, np.array(absum))


def pin_linear_single_row_is_an_outer_product(orc):
    rng = _rng(21)
    x = _rand_bf16(rng, (1, 7))
    w = _rand_bf16(rng, (5, 7))
    dy = _rand_bf16(rng, (1, 5))
    _, dw, _ = orc.linear_bwd_bf16(x, w, dy)
    np.testing.assert_array_equal(dw, np.outer(_val(dy)[0], _val(x)[0]))   # products of bf16 are exact


def pin_linear_identity_weight(orc):
    rng = _rng(22)
    K = 6
    x = _rand_bf16(rng, (9, K))
    dy = _rand_bf16(rng, (9, K))
    w = _bits(np.eye(K))
    np.testing.assert_array_equal(orc.linear_fwd_bf16(x, w), _val(x))
    dx, _, _ = orc.linear_bwd_bf16(x, w, dy)
    np.testing.assert_array_equal(dx, _val(dy))


def pin_linear_trace_identity(orc):
    """<dY, X W^T> = <dW, W> = <dX, X>: the forward, dW and dX agree."""
    rng = _rng(23)
    R, N, K = 37, 11, 13
    x, w, dy = _rand_bf16(rng, (R, K)), _rand_bf16(rng, (N, K)), _rand_bf16(rng, (R, N))
    y = orc.linear_fwd_bf16(x, w)
    dx, dw, _ = orc.linear_bwd_bf16(x, w, dy)
    a = float(np.sum(_val(dy) * y))
    b = float(np.sum(dw * _val(w)))
    c = float(np.sum(dx * _val(x)))
    scale = float(np.sum(np.abs(_val(dy)) @ np.abs(_val(w)) * np.abs(_val(x)).sum(0) / R)) + 1.0
    assert abs(a - b) <= 1e-12 * scale and abs(a - c) <= 1e-12 * scale


def pin_linear_finite_differences(orc):
    """L = <dY, X W^T> is bilinear, so moving one entry of W (or X) to its
    neighbouring bf16 value, a change d, changes L by exactly d * dW (or
    d * dX) up to FP64 rounding."""
    rng = _rng(24)
    R, N, K = 9, 4, 6
    x, w, dy = _rand_bf16(rng, (R, K)), _rand_bf16(rng, (N, K)), _rand_bf16(rng, (R, N))
    dx, dw, _ = orc.linear_bwd_bf16(x, w, dy)

    def L(xb, wb):
        return float(np.sum(_val(dy) * orc.linear_fwd_bf16(xb, wb)))

    base = L(x, w)
    for n in range(N):
        for k in range(K):
            w2 = w.copy()
            w2[n, k] = w[n, k] + 1          # the neighbouring bf16 value
            d = _val(w2[n, k]) - _val(w[n, k])
            if d == 0:
                continue
            assert abs((L(x, w2) - base) / d - dw[n, k]) <= 1e-9 * (1 + abs(dw[n, k])), (n, k)
    for r in range(R):
        for k in range(K):
            x2 = x.copy()
            x2[r, k] = x[r, k] + 1
            d = _val(x2[r, k]) - _val(x[r, k])
            if d == 0:
                continue
            assert abs((L(x2, w) - base) / d - dx[r, k]) <= 1e-9 * (1 + abs(dx[r, k])), (r, k)


def pin_linear_padding_and_layout_invariance(orc):
    rng = _rng(25)
    T, N, K = 23, 5, 8
    x, w, dy = _rand_bf16(rng, (T, K)), _rand_bf16(rng, (N, K)), _rand_bf16(rng, (T, N))
    dx0, dw0, _ = orc.linear_bwd_bf16(x, w, dy)
    perm = rng.permutation(T)
    # padding rows full of NaN patterns, interleaved with the permuted rows
    rl = np.concatenate([perm[:10], [-1, -1], perm[10:], [-1]]).astype(np.int32)
    xp = np.full((len(rl), K), 0x7FC1, np.uint16)
    dyp = np.full((len(rl), N), 0x7FC1, np.uint16)
    real = rl >= 0
    xp[real] = x[rl[real]]
    dyp[real] = dy[rl[real]]
    dx1, dw1, _ = orc.linear_bwd_bf16(xp, w, dyp, rl, T)
    np.testing.assert_array_equal(dw1, dw0)
    assert np.all(dx1[~real] == 0)
    np.testing.assert_array_equal(dx1[real], dx0[rl[real]])
    y1 = orc.linear_fwd_bf16(xp, w, rl)
    assert np.all(y1[~real] == 0)
    with pytest.raises(oracle.OracleError):
        orc.linear_bwd_bf16(x[:3], w, dy[:3], np.array([0, 0, 1], np.int32), 3)


def pin_linear_samples_match_the_full_products(orc):
    rng = _rng(26)
    R, N, K = 31, 7, 9
    x, w, dy = _rand_bf16(rng, (R, K)), _rand_bf16(rng, (N, K)), _rand_bf16(rng, (R, N))
    dx, dw, dwa = orc.linear_bwd_bf16(x, w, dy)
    y = orc.linear_fwd_bf16(x, w)
    kind = np.array([0, 0, 1, 1, 2, 3, 3], np.int32)
    ia = np.array([3, 30, 0, 6, 4, 0, 30], np.int64)
    ib = np.array([8, 0, 5, 8, 2, 6, 0], np.int64)
    got = orc.linear_sample_bf16(x, w, dy, kind, ia, ib)
    np.testing.assert_array_equal(got, [dx[3, 8], dx[30, 0], dw[0, 5], dw[6, 8], dwa[4, 2],
                                        y[0, 6], y[30, 0]])
    with pytest.raises(oracle.OracleError):
        orc.linear_sample_bf16(x, w, dy, np.array([3], np.int32), np.array([R], np.int64),
                               np.array([0], np.int64))


def pin_round_bf16(orc):
    """Exactly representable values keep their bits; halfway cases go to the
    even neighbour; everything else to the nearest bf16 value."""
    exact = np.array([0.0, 1.0, -2.5, 1.5 * 2.0 ** 127, 2.0 ** -126, -0.0078125])
    np.testing.assert_array_equal(_val(orc.round_bf16(exact)), exact)
    one_ulp = 2.0 ** -7                        # bf16 spacing in [1, 2)
    ties = np.array([1.0 + one_ulp / 2, 1.0 + 3 * one_ulp / 2, -(1.0 + one_ulp / 2)])
    np.testing.assert_array_equal(_val(orc.round_bf16(ties)), [1.0, 1.0 + 2 * one_ulp, -1.0])
    rng = _rng(27)
    v = rng.normal(size=4000) * 10.0 ** rng.integers(-20, 20, size=4000)
    got = _val(orc.round_bf16(v))
    lo = (np.frexp(np.abs(v))[1] - 1).astype(np.float64)
    spacing = 2.0 ** (lo - 7)
    assert np.all(np.abs(got - v) <= spacing / 2 * (1 + 2.0 ** -20))


# ------------------------------------------------------- embedding (EDO-v1)
def pin_embedding_brute_force_tiny(orc):
    rng = _rng(30)
    T, V, D = 11, 5, 3
    ids = rng.integers(0, V, size=T).astype(np.int32)
    table = _bits(rng.integers(-16, 17, size=(V, D)) / 8.0)
    dy = _bits(rng.integers(-16, 17, size=(T, D)) / 8.0)
    Y = [[float(_val(table[ids[r], j])) for j in range(D)] for r in range(T)]
    np.testing.assert_array_equal(orc.embedding_fwd_bf16(ids, table), np.array(Y))
    dE = [[sum(float(_val(dy[l, j])) for l in range(T) if ids[l] == v) for j in range(D)]
          for v in range(V)]
    got, _ = orc.embedding_bwd_bf16(ids, dy, V)
    np.testing.assert_array_equal(got, np.array(dE))
    got_cols, _ = orc.embedding_bwd_bf16(ids, dy, V, cols=np.array([2, 0]))
    np.testing.assert_array_equal(got_cols, np.array(dE)[:, [2, 0]])


def pin_embedding_counts_closed_form(orc):
    """dY = 1 everywhere: dE[v][j] is the number of occurrences of v."""
    rng = _rng(31)
    T, V, D = 300, 17, 4
    ids = rng.integers(0, V, size=T).astype(np.int32)
    ones = _bits(np.ones((T, D)))
    dE, _ = orc.embedding_bwd_bf16(ids, ones, V)
    hist = np.bincount(ids, minlength=V).astype(np.float64)
    np.testing.assert_array_equal(dE, np.repeat(hist[:, None], D, axis=1))
    np.testing.assert_array_equal(orc.edo_v1_f32(ids, ones, V), dE.astype(np.float32))


def pin_embedding_padding_layout_and_refusals(orc):
    rng = _rng(32)
    T, V, D = 40, 9, 8
    ids = rng.integers(0, V, size=T).astype(np.int32)
    dy = _rand_bf16(rng, (T, D))
    dE0, _ = orc.embedding_bwd_bf16(ids, dy, V)
    perm = rng.permutation(T)
    rl = np.concatenate([perm[:7], [-1], perm[7:], [-1, -1]]).astype(np.int32)
    real = rl >= 0
    ids_p = np.full(len(rl), 10 ** 6, np.int32)          # padding ids are never read
    ids_p[real] = ids[rl[real]]
    dy_p = np.full((len(rl), D), 0x7FC1, np.uint16)
    dy_p[real] = dy[rl[real]]
    dE1, _ = orc.embedding_bwd_bf16(ids_p, dy_p, V, rl, T)
    np.testing.assert_array_equal(dE1, dE0)
    table = _rand_bf16(rng, (V, D))
    y = orc.embedding_fwd_bf16(ids_p, table, rl)
    assert np.all(y[~real] == 0)
    np.testing.assert_array_equal(y[real], _val(table[ids[rl[real]]]))
    with pytest.raises(oracle.OracleError):
        orc.embedding_bwd_bf16(np.array([0, V], np.int32), dy[:2], V)
    with pytest.raises(oracle.OracleError):
        orc.edo_v1_f32(np.array([0, -1], np.int32), dy[:2], V)


def pin_edo_v1_exact_when_every_partial_is_representable(orc):
    rng = _rng(33)
    T, V, D = 500, 7, 5                       # tokens with several 64-occurrence blocks
    ids = rng.integers(0, V, size=T).astype(np.int32)
    dy = _bits(rng.integers(-16, 17, size=(T, D)) / 8.0)
    dE, _ = orc.embedding_bwd_bf16(ids, dy, V)
    np.testing.assert_array_equal(orc.edo_v1_f32(ids, dy, V), dE.astype(np.float32))


def pin_edo_v1_hand_derived_order(orc):
    """Token 0 occurs 130 times: 2^24 first, then 129 ones.  FP32 spacing at
    2^24 is 2, so a 1 added to 2^24 is lost (ties to even).  EDO-v1: block 0
    (occurrences 0..63) = 2^24, block 1 = 64, block 2 = 2; tree over 4 leaves
    (2^24 + 64) + (2 + 0) = 16777282.  A left fold over all occurrences would
    give 2^24 = 16777216, blocks of 32 would give 16777314.  Token 1 occurs
    once (value 0.5) and token 2 never.  Token 3 occurs 193 times: 2^24,
    then zeros except occurrences 128 and 192 (value 1): blocks 2^24, 0, 1,
    1, and the tree (2^24 + 0) + (1 + 1) = 16777218, where a left fold over
    the blocks would lose both ones (16777216)."""
    n0, n3 = 130, 193
    ids = np.concatenate([np.zeros(n0, np.int32), np.full(n3, 3, np.int32)])
    ids = np.insert(ids, 57, 1)                   # token 1 sits between token 0's rows
    vals0 = np.ones(n0)
    vals0[0] = 2.0 ** 24
    vals3 = np.zeros(n3)
    vals3[0] = 2.0 ** 24
    vals3[128] = 1.0
    vals3[192] = 1.0
    vals = np.insert(np.concatenate([vals0, vals3]), 57, 0.5)
    dy = _bits(vals[:, None])
    got = orc.edo_v1_f32(ids, dy, 4)
    assert got[0, 0] == np.float32(16777282.0)
    assert got[1, 0] == np.float32(0.5) and got[2, 0] == 0.0
    assert got[3, 0] == np.float32(16777218.0)


def pin_edo_v1_within_fp32_error_bound(orc):
    rng = _rng(34)
    T, V, D = 3000, 11, 6
    ids = np.minimum(rng.zipf(1.3, size=T) - 1, V - 1).astype(np.int32)
    dy = _rand_bf16(rng, (T, D))
    ref, dabs = orc.embedding_bwd_bf16(ids, dy, V)
    got = orc.edo_v1_f32(ids, dy, V).astype(np.float64)
    nmax = np.bincount(ids, minlength=V).max()
    depth = 64 + int(math.ceil(math.log2(max(1, (nmax + 63) // 64)))) + 1
    assert np.all(np.abs(got - ref) <= depth * 2.0 ** -24 * dabs * 1.01)


EMBEDDING_PINS = [pin_embedding_brute_force_tiny, pin_embedding_counts_closed_form,
                  pin_embedding_padding_layout_and_refusals,
                  pin_edo_v1_exact_when_every_partial_is_representable, pin_edo_v1_hand_derived_order,
                  pin_edo_v1_within_fp32_error_bound]


@pytest.mark.parametrize("pin", EMBEDDING_PINS, ids=lambda f: f.__name__)
def test_embedding_oracle_pins(pin):
    pin(oracle)


LINEAR_PINS = [pin_round_bf16, pin_linear_brute_force_tiny, pin_linear_single_row_is_an_outer_product,
               pin_linear_identity_weight, pin_linear_trace_identity, pin_linear_finite_differences,
               pin_linear_padding_and_layout_invariance, pin_linear_samples_match_the_full_products]


@pytest.mark.parametrize("pin", LINEAR_PINS, ids=lambda f: f.__name__)
def test_linear_oracle_pins(pin):
    pin(oracle)


# ------------------------------------------------------------- the tests
PINS = [pin_widen_bf16_exact_bit_patterns, pin_forward_constant_row_closed_form, pin_forward_zero_row_and_eps_inside_sqrt, pin_forward_two_element_worked_example, pin_forward_norm_identity_and_scale_invariance, pin_backward_matches_central_finite_differences_h8_t59, pin_backward_explicit_jacobian, pin_backward_orthogonality_and_radial_identity, pin_dweight_euler_identity, pin_h1_closed_form, pin_zero_row_backward, pin_padding_rows_are_never_read_and_contribute_nothing, pin_inactive_rows_contribute_exactly_zero, pin_oracle_is_layout_invariant, pin_invalid_layouts_are_refused, pin_cdo_v2_golden_cases, pin_cdo_v2_golden_cases_are_layout_invariant, pin_cdo_v2_exact_when_every_partial_is_representable, pin_cdo_v2_within_fp32_error_bound_of_fp64]


def test_widen_bf16_exact_bit_patterns():
    pin_widen_bf16_exact_bit_patterns(oracle)


def test_forward_constant_row_closed_form():
    pin_forward_constant_row_closed_form(oracle)


def test_forward_zero_row_and_eps_inside_sqrt():
    pin_forward_zero_row_and_eps_inside_sqrt(oracle)


def test_forward_two_element_worked_example():
    pin_forward_two_element_worked_example(oracle)


def test_forward_norm_identity_and_scale_invariance():
    pin_forward_norm_identity_and_scale_invariance(oracle)


@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_backward_matches_central_finite_differences_h8_t59(eps):
    pin_backward_matches_central_finite_differences_h8_t59(oracle, eps)


def test_backward_explicit_jacobian():
    pin_backward_explicit_jacobian(oracle)


def test_backward_orthogonality_and_radial_identity():
    pin_backward_orthogonality_and_radial_identity(oracle)


def test_dweight_euler_identity():
    pin_dweight_euler_identity(oracle)


def test_h1_closed_form():
    pin_h1_closed_form(oracle)


def test_zero_row_backward():
    pin_zero_row_backward(oracle)


def test_padding_rows_are_never_read_and_contribute_nothing():
    pin_padding_rows_are_never_read_and_contribute_nothing(oracle)


def test_inactive_rows_contribute_exactly_zero():
    pin_inactive_rows_contribute_exactly_zero(oracle)


def test_oracle_is_layout_invariant():
    pin_oracle_is_layout_invariant(oracle)


def test_invalid_layouts_are_refused():
    pin_invalid_layouts_are_refused(oracle)


def test_cdo_v2_golden_cases():
    pin_cdo_v2_golden_cases(oracle)


def test_cdo_v2_golden_cases_are_layout_invariant():
    pin_cdo_v2_golden_cases_are_layout_invariant(oracle)


def test_cdo_v2_exact_when_every_partial_is_representable():
    pin_cdo_v2_exact_when_every_partial_is_representable(oracle)


def test_cdo_v2_within_fp32_error_bound_of_fp64():
    pin_cdo_v2_within_fp32_error_bound_of_fp64(oracle)
