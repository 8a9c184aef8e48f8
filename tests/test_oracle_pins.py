"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties an oracle function to something other than itself: the
explicit d^p Kronecker expansion, the exact polynomial kernel, hand-worked
values, an SVD bound, brute-force loops, or an invariance. CPU only.
"""
import json
import os

import numpy as np
import pytest

from oracle import llops_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_theta(rng, p, t, d, m):
    return rng.standard_normal((p, t, d, m)) / np.sqrt(d)


def _selection_theta(d, p):
    """Theta for the exact kernel: m = d^p columns, column (a_1..a_p) of
    Theta_j is e_{a_j}, so phi(x)_{a} = prod_j x_{a_j}."""
    m = d ** p
    th = np.zeros((p, 1, d, m))
    for col in range(m):
        idx = np.unravel_index(col, (d,) * p)
        for j in range(p):
            th[j, 0, idx[j], col] = 1.0
    return th


# --------------------------------------------------------------------------
# P-1: factorised map == explicit psi_p(X) W_hat (column-wise Kronecker)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("d,p,t,m", [(2, 2, 1, 3), (2, 2, 2, 3), (3, 1, 2, 5), (3, 2, 3, 5),
                                     (4, 3, 2, 3), (2, 3, 3, 5), (8, 2, 2, 5), (3, 4, 2, 3)])
def test_featmap_equals_kronecker_sketch(d, p, t, m):
    rng = np.random.default_rng(100 + d * 10 + p)
    X = rng.standard_normal((7, d))
    th = _rand_theta(rng, p, t, d, m)
    fast = O.featmap(X, th)
    slow = O.psi(X, p) @ O.w_hat(th)
    np.testing.assert_allclose(fast, slow, rtol=1e-12, atol=1e-12 * np.abs(slow).max())


def test_featmap_golden_toy():
    g = _golden("toy_featmap_p2_d2_m3.json")
    X = np.array(g["X"], float)
    th = np.array(g["theta_p_t_d_m"], float)
    np.testing.assert_array_equal(O.featmap(X, th[:, :1]), g["phi_t1"])
    np.testing.assert_array_equal(O.featmap(X, th[:, :1], square=True), g["phi_t1_squared"])
    np.testing.assert_array_equal(O.featmap(X, th), g["phi_t2"])
    np.testing.assert_array_equal(O.featmap(X, th, square=True), g["phi_t2_squared"])
    # the explicit sketch agrees on the hand-worked values too
    np.testing.assert_allclose(O.psi(X, 2) @ O.w_hat(th), g["phi_t2"], atol=1e-12)


def test_psi_kron_layout():
    # psi_2(1,2) = (1,2,2,4) in (a,b) -> a*d+b order
    np.testing.assert_array_equal(O.psi(np.array([[1.0, 2.0]]), 2), [[1, 2, 2, 4]])
    # <psi_p(x), psi_p(y)> = (x^T y)^p
    rng = np.random.default_rng(1)
    x, y = rng.standard_normal((2, 1, 3))
    for p in (1, 2, 3):
        np.testing.assert_allclose(O.psi(x, p) @ O.psi(y, p).T, (x @ y.T) ** p, rtol=1e-12)


# --------------------------------------------------------------------------
# P-2: exact polynomial kernel reached with selection Theta
# --------------------------------------------------------------------------
@pytest.mark.parametrize("d,p", [(2, 2), (3, 2), (4, 2), (2, 3), (3, 3)])
def test_exact_kernel(d, p):
    rng = np.random.default_rng(7 * d + p)
    Q = rng.standard_normal((5, d))
    K = rng.standard_normal((6, d))
    th = _selection_theta(d, p)
    got = O.featmap(Q, th) @ O.featmap(K, th).T
    np.testing.assert_allclose(got, (Q @ K.T) ** p, rtol=1e-11, atol=1e-12)


def test_exact_kernel_squared_closed_form():
    rng = np.random.default_rng(3)
    d = 3
    Q = rng.standard_normal((4, d))
    K = rng.standard_normal((5, d))
    th = _selection_theta(d, 2)
    got = O.featmap(Q, th, square=True) @ O.featmap(K, th, square=True).T
    np.testing.assert_allclose(got, ((Q * Q) @ (K * K).T) ** 2, rtol=1e-11)


# --------------------------------------------------------------------------
# P-3: special cases named on the pages (Flatten, BASED); P-9: p = 1
# --------------------------------------------------------------------------
def test_shared_theta_is_elementwise_power():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((6, 4))
    T1 = rng.standard_normal((4, 5))
    for p in (2, 3, 4):
        th = np.stack([T1[None]] * p)  # [p, 1, d, m], all Theta_j equal
        np.testing.assert_allclose(O.featmap(X, th), (X @ T1) ** p, rtol=1e-12)


def test_based_special_case():
    """BASED: phi(x) = vec((Wx)(Wx)^T) with W in R^{m' x d}: Theta_1 column
    (a,b) = W_a, Theta_2 column (a,b) = W_b."""
    rng = np.random.default_rng(5)
    d, mp = 4, 3
    W = rng.standard_normal((mp, d))
    X = rng.standard_normal((5, d))
    th = np.zeros((2, 1, d, mp * mp))
    for a in range(mp):
        for b in range(mp):
            th[0, 0, :, a * mp + b] = W[a]
            th[1, 0, :, a * mp + b] = W[b]
    want = np.array([np.outer(W @ x, W @ x).ravel() for x in X])
    np.testing.assert_allclose(O.featmap(X, th), want, rtol=1e-12)


def test_degree_one_is_plain_linear_map():
    rng = np.random.default_rng(6)
    X = rng.standard_normal((5, 4))
    th = _rand_theta(rng, 1, 3, 4, 6)
    np.testing.assert_allclose(O.featmap(X, th), X @ th[0].sum(axis=0), rtol=1e-12)


# --------------------------------------------------------------------------
# P-4: Eckart-Young floor and Theorem 3.1's tightness
# --------------------------------------------------------------------------
def test_eckart_young_floor_bounds_any_sketch():
    rng = np.random.default_rng(8)
    d, p, m, n = 3, 2, 4, 12
    Q = rng.standard_normal((n, d))
    K = rng.standard_normal((n, d))
    floor = O.eckart_young_floor(Q, K, p, m)
    A = O.poly_kernel(Q, K, p)
    assert floor > 0
    for trial in range(20):
        tq = _rand_theta(rng, p, 2, d, m)
        tk = _rand_theta(rng, p, 2, d, m)
        err = np.sum((O.featmap(Q, tq) @ O.featmap(K, tk).T - A) ** 2)
        assert err >= floor * (1 - 1e-12)
    # m at least the rank of A (<= dim of psi_2 span = 6) -> floor vanishes
    assert O.eckart_young_floor(Q, K, p, 6) < 1e-18 * np.sum(A ** 2)
    # m = 0 -> the floor is all of ||A||_F^2
    np.testing.assert_allclose(O.eckart_young_floor(Q, K, p, 0), np.sum(A ** 2), rtol=1e-12)


def test_theorem_3_1_linear_sketch_reaches_floor():
    rng = np.random.default_rng(9)
    d, p, m, n = 3, 2, 3, 10
    Q = rng.standard_normal((n, d))
    K = rng.standard_normal((n, d))
    W1, W2 = O.optimal_linear_sketch(Q, K, p, m)
    A = O.poly_kernel(Q, K, p)
    err = np.sum(((O.psi(Q, p) @ W1) @ (O.psi(K, p) @ W2).T - A) ** 2)
    np.testing.assert_allclose(err, O.eckart_young_floor(Q, K, p, m), rtol=1e-8)


# --------------------------------------------------------------------------
# P-5..P-8: attention forms
# --------------------------------------------------------------------------
def _brute_attention(Q, K, V, tq, tk, square, normalize, delta, causal):
    """Per-row loops with the kernel taken from the explicit sketch
    <psi_p(q) W_q, psi_p(k) W_k> (no featmap, no matrix associativity)."""
    p = tq.shape[0]
    fq = O.psi(Q, p) @ O.w_hat(tq)
    fk = O.psi(K, p) @ O.w_hat(tk)
    if square:
        fq, fk = fq * fq, fk * fk
    n, dv = V.shape
    out = np.zeros((n, dv))
    for i in range(n):
        num = np.zeros(dv)
        den = 0.0
        for j in range(n):
            if causal and j > i:
                continue
            w = float(sum(fq[i, a] * fk[j, a] for a in range(fq.shape[1])))
            num += w * V[j]
            den += w
        out[i] = num / (den + delta) if normalize else num
    return out


@pytest.mark.parametrize("square,normalize", [(False, False), (True, True), (False, True)])
def test_noncausal_vs_bruteforce(square, normalize):
    rng = np.random.default_rng(10)
    n, d, dv, p, t, m = 9, 3, 2, 2, 2, 4
    Q, K = rng.standard_normal((2, n, d))
    V = rng.standard_normal((n, dv))
    tq, tk = _rand_theta(rng, p, t, d, m), _rand_theta(rng, p, t, d, m)
    got = O.linattn(Q, K, V, tq, tk, square=square, normalize=normalize, delta=0.3)
    want = _brute_attention(Q, K, V, tq, tk, square, normalize, 0.3, causal=False)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("square,normalize", [(False, False), (True, True)])
@pytest.mark.parametrize("chunk", [1, 4, 7, 16])
def test_causal_chunked_vs_bruteforce(square, normalize, chunk):
    rng = np.random.default_rng(11)
    n, d, dv, p, t, m = 13, 3, 2, 3, 2, 4
    Q, K = rng.standard_normal((2, n, d))
    V = rng.standard_normal((n, dv))
    tq, tk = _rand_theta(rng, p, t, d, m), _rand_theta(rng, p, t, d, m)
    got, S, z = O.causal_chunked(Q, K, V, tq, tk, square=square, normalize=normalize,
                                 delta=0.2, chunk=chunk)
    want = _brute_attention(Q, K, V, tq, tk, square, normalize, 0.2, causal=True)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
    quad = O.causal_quadratic(Q, K, V, tq, tk, square=square, normalize=normalize, delta=0.2)
    np.testing.assert_allclose(got, quad, rtol=1e-10, atol=1e-12)
    S_ref, z_ref = O.state_from_prefix(K, V, tk, square=square)
    np.testing.assert_allclose(S, S_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(z, z_ref, rtol=1e-11, atol=1e-12)


def test_attention_golden_exact_kernel():
    g = _golden("exact_kernel_attention_d2.json")
    q, k, v = (np.array(g[x], float) for x in ("q", "k", "v"))
    th = _selection_theta(2, 2)
    dl = g["delta"]
    out, _, _ = O.causal_chunked(q, k, v, th, th, normalize=True, delta=dl, chunk=2)
    np.testing.assert_allclose(out, g["causal_normalized"], rtol=1e-14)
    out, _, _ = O.causal_chunked(q, k, v, th, th, chunk=2)
    np.testing.assert_allclose(out, g["causal_raw"], rtol=1e-14)
    np.testing.assert_allclose(O.linattn(q, k, v, th, th, normalize=True, delta=dl),
                               g["noncausal_normalized"], rtol=1e-14)
    out, _, _ = O.causal_chunked(q, k, v, th, th, square=True, normalize=True, delta=dl,
                                 chunk=3)
    np.testing.assert_allclose(out, g["causal_squared_normalized"], rtol=1e-14)
    # decode from an empty state walks the same rows
    outs, _, _ = O.decode(np.zeros((4, 2)), np.zeros(4), q, k, v, th, th,
                          normalize=True, delta=dl)
    np.testing.assert_allclose(outs, g["causal_normalized"], rtol=1e-14)


def test_state_continuation_and_decode_match_prefill():
    rng = np.random.default_rng(12)
    n, d, dv, p, t, m = 20, 4, 3, 2, 2, 5
    Q, K = rng.standard_normal((2, n, d))
    V = rng.standard_normal((n, dv))
    tq, tk = _rand_theta(rng, p, t, d, m), _rand_theta(rng, p, t, d, m)
    kw = dict(square=True, normalize=True, delta=1e-3)
    full, S, z = O.causal_chunked(Q, K, V, tq, tk, chunk=4, **kw)
    a, S1, z1 = O.causal_chunked(Q[:11], K[:11], V[:11], tq, tk, chunk=3, **kw)
    b, S2, z2 = O.causal_chunked(Q[11:], K[11:], V[11:], tq, tk, chunk=5, S0=S1, z0=z1, **kw)
    np.testing.assert_allclose(np.vstack([a, b]), full, rtol=1e-11)
    np.testing.assert_allclose(S2, S, rtol=1e-11)
    np.testing.assert_allclose(z2, z, rtol=1e-11)
    outs, Sd, zd = O.decode(S1, z1, Q[11:], K[11:], V[11:], tq, tk, **kw)
    np.testing.assert_allclose(outs, full[11:], rtol=1e-11)
    np.testing.assert_allclose(Sd, S, rtol=1e-11)


def test_normaliser_with_unit_values():
    """V = 1: out_i = den0_i / (den0_i + delta) where den0 is the weight sum."""
    rng = np.random.default_rng(13)
    n, d, p, t, m = 10, 3, 2, 2, 4
    Q, K = rng.standard_normal((2, n, d))
    tq, tk = _rand_theta(rng, p, t, d, m), _rand_theta(rng, p, t, d, m)
    ones = np.ones((n, 1))
    raw, _, _ = O.causal_chunked(Q, K, ones, tq, tk, square=True, chunk=4)
    out, _, _ = O.causal_chunked(Q, K, ones, tq, tk, square=True, normalize=True,
                                 delta=0.05, chunk=4)
    np.testing.assert_allclose(out, raw / (raw + 0.05), rtol=1e-12)


def test_normalised_output_is_convex_combination():
    rng = np.random.default_rng(14)
    n, d, dv, p, t, m = 15, 3, 4, 2, 3, 6
    Q, K = rng.standard_normal((2, n, d))
    V = rng.standard_normal((n, dv))
    tq, tk = _rand_theta(rng, p, t, d, m), _rand_theta(rng, p, t, d, m)
    out, _, _ = O.causal_chunked(Q, K, V, tq, tk, square=True, normalize=True, delta=0.0,
                                 chunk=4)
    for i in range(n):
        lo, hi = V[: i + 1].min(axis=0), V[: i + 1].max(axis=0)
        assert np.all(out[i] >= lo - 1e-12) and np.all(out[i] <= hi + 1e-12)
    np.testing.assert_allclose(out[0], V[0], rtol=1e-12)


# --------------------------------------------------------------------------
# P-10: ordering conventions do not matter
# --------------------------------------------------------------------------
def test_symmetries():
    rng = np.random.default_rng(15)
    n, d, dv, p, t, m = 8, 3, 2, 3, 3, 5
    Q, K = rng.standard_normal((2, n, d))
    V = rng.standard_normal((n, dv))
    tq, tk = _rand_theta(rng, p, t, d, m), _rand_theta(rng, p, t, d, m)
    base = O.featmap(Q, tq, square=True)
    np.testing.assert_allclose(O.featmap(Q, tq[:, ::-1], square=True), base, rtol=1e-12)
    np.testing.assert_allclose(O.featmap(Q, tq[[2, 0, 1]], square=True), base, rtol=1e-12)
    perm = rng.permutation(m)
    out, _, _ = O.causal_chunked(Q, K, V, tq, tk, square=True, normalize=True, chunk=3)
    outp, _, _ = O.causal_chunked(Q, K, V, tq[..., perm], tk[..., perm], square=True,
                                  normalize=True, chunk=3)
    np.testing.assert_allclose(outp, out, rtol=1e-12)


def test_batched_wrappers_use_per_head_theta():
    rng = np.random.default_rng(16)
    B, H, n, d, dv, p, t, m = 2, 3, 6, 3, 2, 2, 2, 4
    Q, K = rng.standard_normal((2, B, H, n, d))
    V = rng.standard_normal((B, H, n, dv))
    tq = rng.standard_normal((H, p, t, d, m))
    tk = rng.standard_normal((H, p, t, d, m))
    out, S, z = O.causal_bh(Q, K, V, tq, tk, chunk=4, normalize=True, delta=0.1)
    for b in range(B):
        for h in range(H):
            want = O.causal_quadratic(Q[b, h], K[b, h], V[b, h], tq[h], tk[h],
                                      normalize=True, delta=0.1)
            np.testing.assert_allclose(out[b, h], want, rtol=1e-11)
    shared = O.featmap_bh(Q, tq[1])
    np.testing.assert_allclose(shared[1, 2], O.featmap(Q[1, 2], tq[1]), rtol=1e-14)


# ---------------------------------------------------------------------------
# feature-map backward (gradients of L = sum(dphi * phi))
# ---------------------------------------------------------------------------
def _loss(X, theta, G, square):
    return float(np.sum(G * O.featmap(X, theta, square)))


@pytest.mark.parametrize("p,t,square", [(2, 2, False), (2, 2, True), (3, 1, True), (1, 3, False)])
def test_featmap_bwd_matches_central_differences(p, t, square):
    """Every entry of dX and dTheta against a central difference of the loss
    in float64 (step 1e-6 on O(1) values: truncation error ~1e-12)."""
    rng = np.random.default_rng(31)
    n, d, m = 5, 3, 4
    X = rng.standard_normal((n, d))
    theta = rng.standard_normal((p, t, d, m)) * 0.7
    G = rng.standard_normal((n, m))
    dX, dth = O.featmap_bwd(X, theta, G, square)
    eps = 1e-6
    for idx in np.ndindex(X.shape):
        Xp, Xm = X.copy(), X.copy()
        Xp[idx] += eps
        Xm[idx] -= eps
        fd = (_loss(Xp, theta, G, square) - _loss(Xm, theta, G, square)) / (2 * eps)
        assert abs(dX[idx] - fd) <= 1e-6 * max(1.0, abs(fd))
    for idx in np.ndindex(theta.shape):
        tp, tm = theta.copy(), theta.copy()
        tp[idx] += eps
        tm[idx] -= eps
        fd = (_loss(X, tp, G, square) - _loss(X, tm, G, square)) / (2 * eps)
        assert abs(dth[idx] - fd) <= 1e-6 * max(1.0, abs(fd))


def test_featmap_bwd_degree_one_is_linear_map_gradient():
    """p = t = 1 makes phi = X Theta: the textbook gradients dX = dphi Theta^T
    and dTheta = X^T dphi; squared, phi = (X Theta)^2 doubles dphi by X Theta."""
    rng = np.random.default_rng(32)
    X = rng.standard_normal((7, 4))
    W = rng.standard_normal((4, 6))
    G = rng.standard_normal((7, 6))
    dX, dth = O.featmap_bwd(X, W[None, None], G)
    assert np.allclose(dX, G @ W.T, rtol=1e-13, atol=1e-13)
    assert np.allclose(dth[0, 0], X.T @ G, rtol=1e-13, atol=1e-13)
    dX2, dth2 = O.featmap_bwd(X, W[None, None], G, square=True)
    G2 = 2.0 * (X @ W) * G
    assert np.allclose(dX2, G2 @ W.T, rtol=1e-12, atol=1e-12)
    assert np.allclose(dth2[0, 0], X.T @ G2, rtol=1e-12, atol=1e-12)


def test_featmap_bwd_shared_theta_sums_heads():
    """With one Theta for every head its gradient is the sum of the per-head
    gradients (the same array appears in every head's map)."""
    rng = np.random.default_rng(33)
    X = rng.standard_normal((2, 3, 4, 3))
    th = rng.standard_normal((2, 2, 3, 4))
    G = rng.standard_normal((2, 3, 4, 4))
    _, dth_shared = O.featmap_bwd_bh(X, th, G)
    _, dth_heads = O.featmap_bwd_bh(X, np.repeat(th[None], 3, axis=0), G)
    assert np.allclose(dth_shared, dth_heads.sum(axis=0), rtol=1e-13, atol=1e-13)


def _causal_loss(Q, K, V, tq, tk, G, square, normalize, delta):
    return float(np.sum(G * O.causal_quadratic(Q, K, V, tq, tk, square=square,
                                               normalize=normalize, delta=delta)))


@pytest.mark.parametrize("square,normalize", [(False, False), (True, False), (False, True),
                                              (True, True)])
def test_causal_bwd_matches_central_differences(square, normalize):
    """Every entry of dQ, dK, dV, dTheta_q and dTheta_k against a central
    difference of L = sum(G * out) through the materialised causal form, in
    float64 (normalised runs use squared or positive features so the
    denominator stays away from zero)."""
    rng = np.random.default_rng(41)
    n, d, dv, m, p, t = 6, 3, 2, 4, 2, 2
    Q = rng.standard_normal((n, d)) * 0.8
    K = rng.standard_normal((n, d)) * 0.8
    V = rng.standard_normal((n, dv))
    tq = rng.standard_normal((p, t, d, m)) * 0.6
    tk = rng.standard_normal((p, t, d, m)) * 0.6
    if normalize and not square:  # keep phi > 0: Theta and inputs of one sign
        Q, K, tq, tk = np.abs(Q), np.abs(K), np.abs(tq), np.abs(tk)
    G = rng.standard_normal((n, dv))
    delta = 0.3 if normalize else 0.0
    args = [Q, K, V, tq, tk]
    grads = O.causal_bwd(*args, G, square=square, normalize=normalize, delta=delta)
    eps = 1e-6
    for which in range(5):
        for idx in np.ndindex(args[which].shape):
            ap = [a.copy() for a in args]
            am = [a.copy() for a in args]
            ap[which][idx] += eps
            am[which][idx] -= eps
            fd = (_causal_loss(*ap, G, square, normalize, delta)
                  - _causal_loss(*am, G, square, normalize, delta)) / (2 * eps)
            got = grads[which][idx]
            assert abs(got - fd) <= 2e-6 * max(1.0, abs(fd)), (which, idx, got, fd)


def test_causal_attn_bwd_first_token_and_last_value():
    """Closed forms at the ends of the sequence: the first query sees only
    the first key, so dPq[0] = (G[0].V[0]) Pk[0] without a normaliser; the
    last value is reached only by the last query, so dV[-1] = (Pq[-1].Pk[-1]) G[-1]."""
    rng = np.random.default_rng(42)
    n, m, dv = 7, 5, 3
    Pq, Pk = rng.standard_normal((n, m)), rng.standard_normal((n, m))
    V, G = rng.standard_normal((n, dv)), rng.standard_normal((n, dv))
    dPq, dPk, dV = O.causal_attn_bwd(Pq, Pk, V, G)
    assert np.allclose(dPq[0], (G[0] @ V[0]) * Pk[0], rtol=1e-13, atol=1e-13)
    assert np.allclose(dV[-1], (Pq[-1] @ Pk[-1]) * G[-1], rtol=1e-13, atol=1e-13)
    assert np.allclose(dPk[-1], (G[-1] @ V[-1]) * Pq[-1], rtol=1e-13, atol=1e-13)


def test_causal_bwd_shared_theta_sums_heads():
    """causal_bwd_bh with a shared Theta returns the head sum of the per-head
    gradients of the same Theta copied to every head."""
    rng = np.random.default_rng(43)
    B, H, n, d, dv, m = 1, 3, 5, 3, 2, 4
    Q, K = rng.standard_normal((B, H, n, d)), rng.standard_normal((B, H, n, d))
    V, G = rng.standard_normal((B, H, n, dv)), rng.standard_normal((B, H, n, dv))
    tq, tk = rng.standard_normal((2, 1, d, m)), rng.standard_normal((2, 1, d, m))
    shared = O.causal_bwd_bh(Q, K, V, tq, tk, G, square=True)
    per = O.causal_bwd_bh(Q, K, V, np.stack([tq] * H), np.stack([tk] * H), G, square=True)
    for a, b in zip(shared[:3], per[:3]):
        assert np.allclose(a, b, rtol=1e-13, atol=1e-13)
    assert np.allclose(shared[3], per[3].sum(0), rtol=1e-12, atol=1e-12)
    assert np.allclose(shared[4], per[4].sum(0), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("normalize,chunk", [(False, 4), (True, 4), (True, 7), (False, 64)])
def test_causal_attn_bwd_chunked_equals_materialised(normalize, chunk):
    """The chunked backward (prefix and suffix states) equals the materialised
    chain rule (itself pinned by central differences above), ragged chunks
    included."""
    rng = np.random.default_rng(44)
    n, m, dv = 23, 6, 5
    Pq = np.abs(rng.standard_normal((n, m)))
    Pk = np.abs(rng.standard_normal((n, m)))
    V, G = rng.standard_normal((n, dv)), rng.standard_normal((n, dv))
    want = O.causal_attn_bwd(Pq, Pk, V, G, normalize=normalize, delta=0.5)
    got = O.causal_attn_bwd_chunked(Pq, Pk, V, G, normalize=normalize, delta=0.5, chunk=chunk)
    for a, b in zip(got, want):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def _lin_loss(Q, K, V, tq, tk, G, square, normalize, delta):
    return float(np.sum(G * O.linattn(Q, K, V, tq, tk, square=square, normalize=normalize,
                                      delta=delta)))


@pytest.mark.parametrize("square,normalize", [(False, False), (True, True)])
def test_linattn_bwd_matches_central_differences(square, normalize):
    """Non-causal: every entry of dQ, dK, dV, dTheta_q, dTheta_k against a
    central difference of L = sum(G * linattn(...))."""
    rng = np.random.default_rng(45)
    n, d, dv, m, p, t = 6, 3, 2, 4, 2, 2
    args = [rng.standard_normal((n, d)) * 0.8, rng.standard_normal((n, d)) * 0.8,
            rng.standard_normal((n, dv)), rng.standard_normal((p, t, d, m)) * 0.6,
            rng.standard_normal((p, t, d, m)) * 0.6]
    G = rng.standard_normal((n, dv))
    delta = 0.3 if normalize else 0.0
    grads = O.linattn_bwd(*args, G, square=square, normalize=normalize, delta=delta)
    eps = 1e-6
    for which in range(5):
        for idx in np.ndindex(args[which].shape):
            ap = [a.copy() for a in args]
            am = [a.copy() for a in args]
            ap[which][idx] += eps
            am[which][idx] -= eps
            fd = (_lin_loss(*ap, G, square, normalize, delta)
                  - _lin_loss(*am, G, square, normalize, delta)) / (2 * eps)
            assert abs(grads[which][idx] - fd) <= 2e-6 * max(1.0, abs(fd)), (which, idx)


def test_attn_bwd_causal_flag_matches_causal_attn_bwd():
    rng = np.random.default_rng(46)
    Pq, Pk = np.abs(rng.standard_normal((9, 4))), np.abs(rng.standard_normal((9, 4)))
    V, G = rng.standard_normal((9, 3)), rng.standard_normal((9, 3))
    for a, b in zip(O.attn_bwd(Pq, Pk, V, G, True, 0.2, causal=True),
                    O.causal_attn_bwd(Pq, Pk, V, G, True, 0.2)):
        assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("normalize", [False, True])
def test_attn_bwd_factored_equals_materialised(normalize):
    """The factored non-causal backward (states S = Pk^T V, z = Pk^T 1) equals
    the materialised chain rule, which the central-difference test above pins."""
    rng = np.random.default_rng(45)
    n, m, dv = 19, 6, 5
    Pq = np.abs(rng.standard_normal((n, m)))
    Pk = np.abs(rng.standard_normal((n, m)))
    V, G = rng.standard_normal((n, dv)), rng.standard_normal((n, dv))
    want = O.attn_bwd(Pq, Pk, V, G, normalize=normalize, delta=0.5, causal=False)
    got = O.attn_bwd_factored(Pq, Pk, V, G, normalize=normalize, delta=0.5)
    for a, b in zip(got, want):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


# ---- gated (decayed) causal attention --------------------------------------

def _gated_inputs(rng, n=9, d=3, dv=2, m=4, t=2):
    Q, K = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    V = rng.standard_normal((n, dv))
    tq, tk = rng.standard_normal((2, t, d, m)), rng.standard_normal((2, t, d, m))
    g = -np.abs(rng.standard_normal(n))
    return Q, K, V, tq, tk, g


@pytest.mark.parametrize("normalize", [False, True])
def test_gated_zero_gate_is_causal(normalize):
    """log_gate = 0 (no decay) reduces both gated forms to causal_quadratic."""
    rng = np.random.default_rng(60)
    Q, K, V, tq, tk, g = _gated_inputs(rng)
    z = np.zeros_like(g)
    want = O.causal_quadratic(Q, K, V, tq, tk, square=True, normalize=normalize, delta=0.25)
    a = O.gated_causal_quadratic(Q, K, V, tq, tk, z, square=True, normalize=normalize, delta=0.25)
    b, _, _ = O.gated_recurrent(Q, K, V, tq, tk, z, square=True, normalize=normalize, delta=0.25)
    assert np.allclose(a, want, rtol=1e-12, atol=1e-12)
    assert np.allclose(b, want, rtol=1e-12, atol=1e-12)


def test_gated_geometric_series():
    """Scalar features (d = m = p = t = 1, Theta = 1), k = v = 1 and a constant
    decay gamma: out_i = q_i (1 - gamma^(i+1)) / (1 - gamma), the geometric
    sum over keys 0..i with weight gamma^(i-j)."""
    n, gamma = 12, 0.8
    q = np.linspace(0.5, 2.0, n)[:, None]
    ones = np.ones((n, 1))
    th = np.ones((1, 1, 1, 1))
    g = np.full(n, np.log(gamma))
    want = q[:, 0] * (1 - gamma ** (np.arange(n) + 1)) / (1 - gamma)
    a = O.gated_causal_quadratic(q, ones, ones, th, th, g)
    b, S, z = O.gated_recurrent(q, ones, ones, th, th, g)
    assert np.allclose(a[:, 0], want, rtol=1e-13)
    assert np.allclose(b[:, 0], want, rtol=1e-13)
    assert np.isclose(S[0, 0], (1 - gamma ** n) / (1 - gamma), rtol=1e-13)


def test_gated_full_forgetting():
    """A gate of exp(-800) = 0 forgets everything before the current token:
    normalised with delta = 0 and a positive (squared) map, out_i = v_i."""
    rng = np.random.default_rng(61)
    Q, K, V, tq, tk, _ = _gated_inputs(rng)
    g = np.full(Q.shape[0], -800.0)
    a = O.gated_causal_quadratic(Q, K, V, tq, tk, g, square=True, normalize=True)
    b, _, _ = O.gated_recurrent(Q, K, V, tq, tk, g, square=True, normalize=True)
    assert np.allclose(a, V, rtol=1e-12, atol=1e-12)
    assert np.allclose(b, V, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("normalize", [False, True])
def test_gated_recurrent_equals_materialised_and_continues(normalize):
    """The recurrence equals the decay-masked matrix form, and splitting the
    sequence with the first half's (S, z) as the second half's initial state
    reproduces the whole."""
    rng = np.random.default_rng(62)
    Q, K, V, tq, tk, g = _gated_inputs(rng, n=15)
    kw = dict(square=True, normalize=normalize, delta=0.5)
    whole, S, z = O.gated_recurrent(Q, K, V, tq, tk, g, **kw)
    assert np.allclose(O.gated_causal_quadratic(Q, K, V, tq, tk, g, **kw), whole,
                       rtol=1e-12, atol=1e-12)
    k = 6
    _, S1, z1 = O.gated_recurrent(Q[:k], K[:k], V[:k], tq, tk, g[:k], **kw)
    second = O.gated_causal_quadratic(Q[k:], K[k:], V[k:], tq, tk, g[k:], S0=S1, z0=z1, **kw)
    assert np.allclose(second, whole[k:], rtol=1e-12, atol=1e-12)
    _, S2, z2 = O.gated_recurrent(Q[k:], K[k:], V[k:], tq, tk, g[k:], S0=S1, z0=z1, **kw)
    assert np.allclose(S2, S, rtol=1e-12, atol=1e-12) and np.allclose(z2, z, rtol=1e-12)


# ---- gated attention backward ------------------------------------------------

def _gated_loss(Q, K, V, tq, tk, g, G, **kw):
    return float((G * O.gated_causal_quadratic(Q, K, V, tq, tk, g, **kw)).sum())


@pytest.mark.parametrize("square,normalize", [(False, False), (True, False), (True, True)])
def test_gated_bwd_central_differences(square, normalize):
    """Every entry of Q, K, V, Theta_q, Theta_k and the log gates against
    (L(x + h) - L(x - h)) / 2h of L = sum(G * gated_causal_quadratic)."""
    rng = np.random.default_rng(70 + 2 * square + normalize)
    n, d, dv, m, p, t = 7, 3, 2, 4, 2, 2
    Q, K = 0.7 * rng.standard_normal((n, d)), 0.7 * rng.standard_normal((n, d))
    V = rng.standard_normal((n, dv))
    tq, tk = 0.6 * rng.standard_normal((p, t, d, m)), 0.6 * rng.standard_normal((p, t, d, m))
    g = -np.abs(0.5 * rng.standard_normal(n))
    G = rng.standard_normal((n, dv))
    kw = dict(square=square, normalize=normalize, delta=0.5)
    got = O.gated_causal_bwd(Q, K, V, tq, tk, g, G, **kw)
    args = [Q, K, V, tq, tk, g]
    h = 1e-6
    for which, grad in zip(range(6), got):
        x = args[which]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[which], am[which] = xp, xm
            num[idx] = (_gated_loss(*ap, G, **kw) - _gated_loss(*am, G, **kw)) / (2 * h)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-7), which


def test_gated_bwd_zero_gate_is_causal_bwd():
    """With log_gate = 0 the feature and value gradients are the ungated ones."""
    rng = np.random.default_rng(75)
    n, m, dv = 11, 5, 3
    Pq, Pk = np.abs(rng.standard_normal((n, m))), np.abs(rng.standard_normal((n, m)))
    V, G = rng.standard_normal((n, dv)), rng.standard_normal((n, dv))
    want = O.causal_attn_bwd(Pq, Pk, V, G, normalize=True, delta=0.3)
    got = O.gated_attn_bwd(Pq, Pk, V, G, np.zeros(n), normalize=True, delta=0.3)
    for a, b in zip(got[:3], want):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("normalize", [False, True])
def test_gated_bwd_recurrent_equals_materialised(normalize):
    rng = np.random.default_rng(76 + normalize)
    n, m, dv = 13, 4, 3
    Pq, Pk = np.abs(rng.standard_normal((n, m))), np.abs(rng.standard_normal((n, m)))
    V, G = rng.standard_normal((n, dv)), rng.standard_normal((n, dv))
    g = -np.abs(rng.standard_normal(n))
    a = O.gated_attn_bwd(Pq, Pk, V, G, g, normalize=normalize, delta=0.2)
    b = O.gated_attn_bwd_recurrent(Pq, Pk, V, G, g, normalize=normalize, delta=0.2)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=1e-11, atol=1e-12)


def test_gated_bwd_gate_gradient_closed_form():
    """Scalar features (Pq = Pk = 1), v = 1, G = 1, no normaliser, constant
    decay a: out_i = sum_{k=0..i} a^k, so L = sum_i sum_{k<=i} a^k and
    d/dg_l of the product chain: g_l appears in every weight a^(i-j) with
    j < l <= i, each contributing a^(i-j), so dg_l = sum_{i>=l} sum_{j<l} a^(i-j)."""
    n, a = 9, 0.7
    g = np.full(n, np.log(a))
    ones = np.ones((n, 1))
    _, _, _, dg = O.gated_attn_bwd(ones, ones, ones, ones, g)
    want = np.array([sum(a ** (i - j) for i in range(l, n) for j in range(l))
                     for l in range(n)])
    assert np.allclose(dg, want, rtol=1e-13, atol=1e-15)


# ---- causal backward from an initial state -----------------------------------

def _state_loss(Q, K, V, tq, tk, S0, z0, G, **kw):
    # the chunked recurrent form (an independent formulation of the forward)
    out = O.causal_chunked(Q, K, V, tq, tk, chunk=4, S0=S0, z0=z0, **kw)[0]
    return float((G * out).sum())


@pytest.mark.parametrize("square,normalize", [(False, False), (True, True)])
def test_causal_bwd_state_central_differences(square, normalize):
    """Every entry of Q, K, V, Theta_q, Theta_k, S0 and z0 against central
    differences of sum(G * causal_quadratic(..., S0, z0))."""
    rng = np.random.default_rng(80 + normalize)
    n, d, dv, m, p, t = 6, 3, 2, 4, 2, 2
    Q, K = 0.7 * rng.standard_normal((n, d)), 0.7 * rng.standard_normal((n, d))
    V = rng.standard_normal((n, dv))
    tq, tk = 0.6 * rng.standard_normal((p, t, d, m)), 0.6 * rng.standard_normal((p, t, d, m))
    S0 = 0.3 * rng.standard_normal((m, dv))
    z0 = np.abs(0.3 * rng.standard_normal(m))
    G = rng.standard_normal((n, dv))
    kw = dict(square=square, normalize=normalize, delta=0.5)
    got = O.causal_bwd_state(Q, K, V, tq, tk, G, S0, z0, **kw)
    args = [Q, K, V, tq, tk, S0, z0]
    order = [0, 1, 2, 3, 4, 5, 6]
    h = 1e-6
    for which, grad in zip(order, got):
        x = args[which]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[which], am[which] = xp, xm
            num[idx] = (_state_loss(*ap, G, **kw) - _state_loss(*am, G, **kw)) / (2 * h)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-7), which


def test_causal_bwd_zero_state_is_causal_bwd():
    rng = np.random.default_rng(83)
    n, m, dv = 9, 4, 3
    Pq, Pk = np.abs(rng.standard_normal((n, m))), np.abs(rng.standard_normal((n, m)))
    V, G = rng.standard_normal((n, dv)), rng.standard_normal((n, dv))
    want = O.causal_attn_bwd(Pq, Pk, V, G, normalize=True, delta=0.3)
    got = O.causal_attn_bwd_state(Pq, Pk, V, G, np.zeros((m, dv)), np.zeros(m), normalize=True,
                                  delta=0.3)
    for a, b in zip(got[:3], want):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_causal_bwd_state_is_prefix_gradient():
    """The initial state is what a prefix leaves behind: with S0, z0 built from
    a prefix of k tokens, dS0 and dz0 chained back through the prefix's
    S = Pk_pre^T V_pre, z = Pk_pre^T 1 give the prefix keys' and values'
    gradient contributions of the whole sequence's backward (rows k.. of G)."""
    rng = np.random.default_rng(84)
    n, k, m, dv = 10, 4, 3, 2
    Pq, Pk = np.abs(rng.standard_normal((n, m))), np.abs(rng.standard_normal((n, m)))
    V, G = rng.standard_normal((n, dv)), rng.standard_normal((n, dv))
    G[:k] = 0.0  # only the continuation's outputs carry loss
    full = O.causal_attn_bwd(Pq, Pk, V, G, normalize=True, delta=0.2)
    S0, z0 = Pk[:k].T @ V[:k], Pk[:k].sum(axis=0)
    part = O.causal_attn_bwd_state(Pq[k:], Pk[k:], V[k:], G[k:], S0, z0, normalize=True,
                                   delta=0.2)
    # continuation rows match
    assert np.allclose(part[0], full[0][k:], rtol=1e-11, atol=1e-12)
    assert np.allclose(part[1], full[1][k:], rtol=1e-11, atol=1e-12)
    assert np.allclose(part[2], full[2][k:], rtol=1e-11, atol=1e-12)
    # prefix rows through the state: dPk_pre = V_pre dS0^T + dz0, dV_pre = Pk_pre dS0
    assert np.allclose(V[:k] @ part[3].T + part[4][None, :], full[1][:k], rtol=1e-11, atol=1e-12)
    assert np.allclose(Pk[:k] @ part[3], full[2][:k], rtol=1e-11, atol=1e-12)


# ---- gated backward from an initial state -------------------------------------

def _gated_state_loss(Q, K, V, tq, tk, g, S0, z0, G, **kw):
    out, _, _ = O.gated_recurrent(Q, K, V, tq, tk, g, S0=S0, z0=z0, **kw)
    return float((G * out).sum())


@pytest.mark.parametrize("normalize", [False, True])
def test_gated_bwd_state_central_differences(normalize):
    """Every entry of Q, K, V, Theta, the log gates, S0 and z0 against central
    differences of sum(G * gated_recurrent(..., S0, z0)) (the token-by-token
    form, independent of the materialised backward)."""
    rng = np.random.default_rng(90 + normalize)
    n, d, dv, m, p, t = 6, 3, 2, 4, 2, 2
    Q, K = 0.7 * rng.standard_normal((n, d)), 0.7 * rng.standard_normal((n, d))
    V = rng.standard_normal((n, dv))
    tq, tk = 0.6 * rng.standard_normal((p, t, d, m)), 0.6 * rng.standard_normal((p, t, d, m))
    g = -np.abs(0.5 * rng.standard_normal(n))
    S0 = 0.3 * rng.standard_normal((m, dv))
    z0 = np.abs(0.3 * rng.standard_normal(m))
    G = rng.standard_normal((n, dv))
    kw = dict(square=True, normalize=normalize, delta=0.5)
    got = O.gated_causal_bwd_state(Q, K, V, tq, tk, g, G, S0, z0, **kw)
    args = [Q, K, V, tq, tk, g, S0, z0]
    h = 1e-6
    for which, grad in enumerate(got):
        x = args[which]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[which], am[which] = xp, xm
            num[idx] = (_gated_state_loss(*ap, G, **kw) - _gated_state_loss(*am, G, **kw)) / (2 * h)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-7), which


def test_gated_bwd_zero_state_is_gated_bwd():
    rng = np.random.default_rng(93)
    n, m, dv = 9, 4, 3
    Pq, Pk = np.abs(rng.standard_normal((n, m))), np.abs(rng.standard_normal((n, m)))
    V, G = rng.standard_normal((n, dv)), rng.standard_normal((n, dv))
    g = -np.abs(rng.standard_normal(n))
    want = O.gated_attn_bwd(Pq, Pk, V, G, g, normalize=True, delta=0.3)
    got = O.gated_attn_bwd_state(Pq, Pk, V, G, g, np.zeros((m, dv)), np.zeros(m), normalize=True,
                                 delta=0.3)
    for a, b in zip(got[:4], want):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
