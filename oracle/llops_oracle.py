"""Plain fp64 CPU oracle for the LLoPS linear-attention hot path.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module. The product path (the HIP
library and its Python binding) never does, and this module imports nothing
from it. Inputs arrive as plain numpy arrays; everything here runs in float64
with no intermediate rounding, no blocking and no fusion beyond what each
definition states.

Sources (titles of the pages the method is described on):
  [LLoPS-notes]  "Learnable Low-Rank Polynomial Sketch for Effective Linear
                 Attention" -- papernotes.org reading notes (NeurIPS 2026).
  [LLoPS-arXiv]  the same paper's text (arXiv 2610.14219), signal-papers reader.
  [SLAY-notes]   "SLAY: Geometry-aware Spherical Linearized Attention with
                 Yat-kernel" notes -- only its normalised linear-attention form.
  [LowRank-blog] blog post on low-rank attention, Linformer and Performer --
                 associativity and the causal cumulative-sum remark.

Readings taken where the pages are silent (each also pinned by a test where
the mathematics allows; see tests/test_oracle_pins.py):
  * Theta_{j,r} is d x m and feature i is column i ([LLoPS-notes] key design 2).
  * Lambda weights are folded into Theta (no separate lambda argument).
  * Squaring, when asked for, is applied after the sum over r.
  * Normaliser: out_i = num_i / (phi_Q(q_i) . z_i + delta), delta added once.
  * Causal mask is inclusive (key j contributes to query i iff j <= i); the
    decode step adds the new key/value to the state before reading it.
  * No 1/sqrt(d) scaling inside the method; the kernel is (q^T k)^p.
  * Gated state update (named as future work in [LLoPS-notes] conclusion,
    with Mamba2's semiseparable matrix as the example): one scalar decay
    a_i = exp(g_i) per token and head multiplies the whole state (S and z)
    before token i is added, so key j reaches query i >= j with weight
    exp(g_{j+1} + ... + g_i).
parity unpinned: the delta placement and the inclusive diagonal are
conventions (the pages fix neither); the tests only check that every path
applies them consistently.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Feature map
# --------------------------------------------------------------------------
def featmap(X, theta, square: bool = False) -> np.ndarray:
    """phi(X) = sum_r prod_j (X Theta_{j,r}), optionally squared element-wise.

    X: [n, d]; theta: [p, t, d, m]. Returns [n, m] float64.
    [LLoPS-notes] key design 2: psi_p(Q) W_hat = sum_r prod_j Q Theta_{j,r}
    (p*t low-dimensional products, then a Hadamard product over j and a sum
    over the t rank components). Squaring: [LLoPS-notes] training strategy
    (non-negativity) and [LLoPS-arXiv] Sec. 3 non-negativity paragraph.
    """
    X = _f64(X)
    theta = _f64(theta)
    p, t, d, m = theta.shape
    assert X.shape[-1] == d
    F = np.zeros(X.shape[:-1] + (m,))
    for r in range(t):
        prod = np.ones(X.shape[:-1] + (m,))
        for j in range(p):
            prod = prod * (X @ theta[j, r])
        F = F + prod
    if square:
        F = F * F
    return F


def featmap_bwd(X, theta, dphi, square: bool = False):
    """Gradients of phi = featmap(X, theta, square) for an upstream gradient
    dphi: returns (dX, dtheta), the derivatives of L = sum(dphi * phi).

    X: [n, d]; theta: [p, t, d, m]; dphi: [n, m]. Float64.
    Theta is trained end to end ([LLoPS-notes] training strategy;
    [LLoPS-arXiv] Sec. 3). The chain rule through the definition of featmap:
    with Y_{j,r} = X Theta_{j,r} and s = sum_r prod_j Y_{j,r},
      ds = dphi * 2 s (squared) or dphi,
      dY_{j,r} = ds * prod_{j' != j} Y_{j',r},
      dX = sum_{j,r} dY_{j,r} Theta_{j,r}^T,  dTheta_{j,r} = X^T dY_{j,r}.
    """
    X = _f64(X)
    theta = _f64(theta)
    G = _f64(dphi)
    p, t, d, m = theta.shape
    Y = [[X @ theta[j, r] for r in range(t)] for j in range(p)]
    s = np.zeros(X.shape[:-1] + (m,))
    for r in range(t):
        prod = np.ones_like(s)
        for j in range(p):
            prod = prod * Y[j][r]
        s = s + prod
    ds = G * (2.0 * s) if square else G
    dX = np.zeros_like(X)
    dtheta = np.zeros_like(theta)
    for r in range(t):
        for j in range(p):
            other = np.ones_like(s)
            for jj in range(p):
                if jj != j:
                    other = other * Y[jj][r]
            dY = ds * other
            dX = dX + dY @ theta[j, r].T
            dtheta[j, r] = X.T @ dY
    return dX, dtheta


# --------------------------------------------------------------------------
# Exact polynomial machinery (explicit d^p expansion; tiny d only)
# --------------------------------------------------------------------------
def psi(X, p: int) -> np.ndarray:
    """psi_p(x) = vec(x^{(x)p}) for every row of X: [n, d] -> [n, d^p].

    [LLoPS-arXiv] Sec. 1-3: the exact degree-p monomial feature map; index
    (a_1, ..., a_p) sits at position a_1 d^{p-1} + ... + a_p (np.kron order).
    """
    X = _f64(X)
    out = []
    for x in X:
        v = np.array([1.0])
        for _ in range(p):
            v = np.kron(v, x)
        out.append(v)
    return np.array(out)


def w_hat(theta) -> np.ndarray:
    """W_hat = sum_r Theta_{1,r} (.)col ... (.)col Theta_{p,r}: [d^p, m].

    Column i of the column-wise Kronecker product is the Kronecker product of
    the i-th columns, in the same order psi() uses.
    [LLoPS-notes] key design 2 (equation for W_hat); [LLoPS-arXiv] Eq. 8.
    """
    theta = _f64(theta)
    p, t, d, m = theta.shape
    W = np.zeros((d ** p, m))
    for r in range(t):
        for i in range(m):
            col = np.array([1.0])
            for j in range(p):
                col = np.kron(col, theta[j, r, :, i])
            W[:, i] += col
    return W


def poly_kernel(Q, K, p: int) -> np.ndarray:
    """A = (Q K^T)^{*p}, the degree-p polynomial kernel matrix, no scaling.

    [LLoPS-arXiv] kappa(q, k) = (q^T k)^p; [LLoPS-notes] key design 1.
    """
    return (_f64(Q) @ _f64(K).T) ** p


def eckart_young_floor(Q, K, p: int, m: int) -> float:
    """sum_{i>m} sigma_i^2 of A = (Q K^T)^{*p}: the least squared Frobenius
    error any rank-m product phi_Q phi_K^T can reach.
    [LLoPS-notes] key design 1 (Eckart-Young-Mirsky bound)."""
    s = np.linalg.svd(poly_kernel(Q, K, p), compute_uv=False)
    return float(np.sum(s[m:] ** 2))


def optimal_linear_sketch(Q, K, p: int, m: int):
    """Theorem 3.1's construction: W1, W2 in R^{d^p x m} with
    psi_p(Q) W1 = U_m Sigma_m^{1/2} and psi_p(K) W2 = V_m Sigma_m^{1/2},
    found by least squares (the proof shows an exact solution exists).
    [LLoPS-arXiv] Appendix A.1; [LLoPS-notes] key design 1."""
    A = poly_kernel(Q, K, p)
    U, s, Vt = np.linalg.svd(A)
    rs = np.sqrt(s[:m])
    W1 = np.linalg.lstsq(psi(Q, p), U[:, :m] * rs, rcond=None)[0]
    W2 = np.linalg.lstsq(psi(K, p), Vt[:m].T * rs, rcond=None)[0]
    return W1, W2


# --------------------------------------------------------------------------
# Linear attention, one (batch, head) slice
# --------------------------------------------------------------------------
def linattn(Q, K, V, theta_q, theta_k, square=False, normalize=False, delta=0.0):
    """Non-causal: out = phi_Q (phi_K^T V) [/ (phi_Q (phi_K^T 1) + delta)].

    [LLoPS-notes] overall framework: Attn = phi_Q(Q) (phi_K(K)^T V) by
    associativity; [LowRank-blog] Performer section for the normalised
    numerator/denominator form; [SLAY-notes] key design 3 for the +delta.
    """
    Pq = featmap(Q, theta_q, square)
    Pk = featmap(K, theta_k, square)
    V = _f64(V)
    num = Pq @ (Pk.T @ V)
    if not normalize:
        return num
    den = Pq @ Pk.sum(axis=0) + delta
    return num / den[:, None]


def causal_quadratic(Q, K, V, theta_q, theta_k, square=False, normalize=False,
                     delta=0.0):
    """Causal, materialised: M = tril(phi_Q phi_K^T) (diagonal kept),
    out = M V [/ (M 1 + delta)]. O(n^2); small n only.
    [LLoPS-arXiv] Sec. 1 (attention as (phi(Q) phi(K)^T) V); causal masking
    per the causal-LM use in [LLoPS-notes] training strategy."""
    Pq = featmap(Q, theta_q, square)
    Pk = featmap(K, theta_k, square)
    M = np.tril(Pq @ Pk.T)
    num = M @ _f64(V)
    if not normalize:
        return num
    return num / (M.sum(axis=1) + delta)[:, None]


def causal_chunked(Q, K, V, theta_q, theta_k, square=False, normalize=False,
                   delta=0.0, chunk=64, S0=None, z0=None):
    """Causal, recurrent over chunks of `chunk` tokens.

    State S (m x dv) and z (m) hold phi_K^T V and phi_K^T 1 of all earlier
    chunks; within a chunk the masked product is explicit:
      num_c = tril(Pq_c Pk_c^T) V_c + Pq_c S,  den_c = tril(..) 1 + Pq_c z + delta
      then S += Pk_c^T V_c, z += Pk_c^T 1.
    [LowRank-blog] Linformer-vs-Performer table (causal masking by
    incremental cumulative sums); [LLoPS-arXiv] Sec. 1 (streaming computation
    with a constant-size state). Returns (out, S_final, z_final).
    """
    Pq = featmap(Q, theta_q, square)
    Pk = featmap(K, theta_k, square)
    V = _f64(V)
    n, m = Pq.shape
    dv = V.shape[1]
    S = np.zeros((m, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros(m) if z0 is None else _f64(z0).copy()
    out = np.zeros((n, dv))
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        q, k, v = Pq[c0:c1], Pk[c0:c1], V[c0:c1]
        A = np.tril(q @ k.T)
        num = A @ v + q @ S
        if normalize:
            den = A.sum(axis=1) + q @ z + delta
            out[c0:c1] = num / den[:, None]
        else:
            out[c0:c1] = num
        S = S + k.T @ v
        z = z + k.sum(axis=0)
    return out, S, z


def attn_bwd(Pq, Pk, V, G, normalize=False, delta=0.0, causal=True):
    """Gradients (dPq, dPk, dV) of L = sum(G * out) for out = M V [/ (M 1 + delta)]
    over given features, M = Pq Pk^T, lower-triangular (diagonal kept) when
    causal. The chain rule through the materialised form of causal_quadratic
    and linattn ([LLoPS-arXiv] Sec. 1; [LowRank-blog] Performer section for
    the normalised form, [SLAY-notes] key design 3 for the +delta):
      normalised:  dnum = G / den,  dden = -sum_cols(G * out) / den
      plain:       dnum = G,        dden = 0
      dM = dnum V^T + dden 1^T (lower triangle when causal)
      dPq = dM Pk,  dPk = dM^T Pq,  dV = M^T dnum.
    """
    Pq, Pk, V, G = _f64(Pq), _f64(Pk), _f64(V), _f64(G)
    M = Pq @ Pk.T
    if causal:
        M = np.tril(M)
    if normalize:
        den = M.sum(axis=1) + delta
        out = (M @ V) / den[:, None]
        dnum = G / den[:, None]
        dden = -(G * out).sum(axis=1) / den
    else:
        dnum = G
        dden = np.zeros(Pq.shape[0])
    dM = dnum @ V.T + dden[:, None]
    if causal:
        dM = np.tril(dM)
    return dM @ Pk, dM.T @ Pq, M.T @ dnum


def attn_bwd_factored(Pq, Pk, V, G, normalize=False, delta=0.0):
    """Non-causal attn_bwd without the n x n matrix: by associativity
    ([LLoPS-arXiv] Sec. 1) with S = Pk^T V and z = Pk^T 1,
      num = Pq S,  den = Pq z + delta,
      dPq = dnum S^T + dden z^T,
      dPk = V (dnum^T Pq) + 1 (dden^T Pq),
      dV  = Pk (Pq^T dnum).
    Exact (up to rounding order) for any n; used where n^2 does not fit."""
    Pq, Pk, V, G = _f64(Pq), _f64(Pk), _f64(V), _f64(G)
    S = Pk.T @ V
    z = Pk.sum(axis=0)
    if normalize:
        den = Pq @ z + delta
        out = (Pq @ S) / den[:, None]
        dnum = G / den[:, None]
        dden = -(G * out).sum(axis=1) / den
    else:
        dnum = G
        dden = np.zeros(Pq.shape[0])
    dPq = dnum @ S.T + np.outer(dden, z)
    dPk = V @ (dnum.T @ Pq) + np.outer(np.ones(Pk.shape[0]), dden @ Pq)
    dV = Pk @ (Pq.T @ dnum)
    return dPq, dPk, dV


def linattn_bwd(Q, K, V, theta_q, theta_k, G, square=False, normalize=False, delta=0.0):
    """Gradients (dQ, dK, dV, dTheta_q, dTheta_k) of L = sum(G * out) for
    out = linattn(Q, K, V, theta_q, theta_k, ...): attn_bwd without the mask,
    then featmap_bwd on each side."""
    Pq = featmap(Q, theta_q, square)
    Pk = featmap(K, theta_k, square)
    dPq, dPk, dV = attn_bwd(Pq, Pk, V, G, normalize, delta, causal=False)
    dQ, dtq = featmap_bwd(Q, theta_q, dPq, square)
    dK, dtk = featmap_bwd(K, theta_k, dPk, square)
    return dQ, dK, dV, dtq, dtk


def causal_attn_bwd(Pq, Pk, V, G, normalize=False, delta=0.0):
    """Gradients (dPq, dPk, dV) of L = sum(G * out) for the causal contraction
    over given features, out = M V [/ (M 1 + delta)] with M = tril(Pq Pk^T).

    The chain rule through the materialised form of causal_quadratic
    ([LLoPS-arXiv] Sec. 1; the normalised form of [LowRank-blog] Performer
    section with [SLAY-notes] key design 3's +delta):
      normalised:  dnum = G / den,  dden = -sum_cols(G * out) / den
      plain:       dnum = G,        dden = 0
      dM = tril(dnum V^T + dden 1^T)
      dPq = dM Pk,  dPk = dM^T Pq,  dV = M^T dnum.
    """
    Pq, Pk, V, G = _f64(Pq), _f64(Pk), _f64(V), _f64(G)
    M = np.tril(Pq @ Pk.T)
    if normalize:
        den = M.sum(axis=1) + delta
        out = (M @ V) / den[:, None]
        dnum = G / den[:, None]
        dden = -(G * out).sum(axis=1) / den
    else:
        dnum = G
        dden = np.zeros(Pq.shape[0])
    dM = np.tril(dnum @ V.T + dden[:, None])
    return dM @ Pk, dM.T @ Pq, M.T @ dnum


def causal_attn_bwd_state(Pq, Pk, V, G, S0, z0, normalize=False, delta=0.0):
    """causal_attn_bwd for the contraction continued from an initial state
    (S0 [m, dv], z0 [m]; causal_quadratic's S0/z0): with
      num = M V + Pq S0,  den = M 1 + Pq z0 + delta,
    dnum and dden as before, dM = tril(dnum V^T + dden 1^T), and
      dPq = dM Pk + dnum S0^T + dden z0^T,  dPk = dM^T Pq,  dV = M^T dnum,
      dS0 = Pq^T dnum,  dz0 = Pq^T dden
    ([LLoPS-arXiv] Sec. 1 streaming form; [LowRank-blog] Performer section;
    [SLAY-notes] key design 3). Returns (dPq, dPk, dV, dS0, dz0)."""
    Pq, Pk, V, G = _f64(Pq), _f64(Pk), _f64(V), _f64(G)
    S0, z0 = _f64(S0), _f64(z0)
    M = np.tril(Pq @ Pk.T)
    num = M @ V + Pq @ S0
    if normalize:
        den = M.sum(axis=1) + Pq @ z0 + delta
        out = num / den[:, None]
        dnum = G / den[:, None]
        dden = -(G * out).sum(axis=1) / den
    else:
        dnum = G
        dden = np.zeros(Pq.shape[0])
    dM = np.tril(dnum @ V.T + dden[:, None])
    dPq = dM @ Pk + dnum @ S0.T + np.outer(dden, z0)
    return dPq, dM.T @ Pq, M.T @ dnum, Pq.T @ dnum, Pq.T @ dden


def causal_bwd_state(Q, K, V, theta_q, theta_k, G, S0, z0, square=False, normalize=False,
                     delta=0.0):
    """causal_bwd from an initial state: (dQ, dK, dV, dTheta_q, dTheta_k, dS0, dz0)."""
    Pq = featmap(Q, theta_q, square)
    Pk = featmap(K, theta_k, square)
    dPq, dPk, dV, dS0, dz0 = causal_attn_bwd_state(Pq, Pk, V, G, S0, z0, normalize, delta)
    dQ, dtq = featmap_bwd(Q, theta_q, dPq, square)
    dK, dtk = featmap_bwd(K, theta_k, dPk, square)
    return dQ, dK, dV, dtq, dtk, dS0, dz0


def causal_bwd_state_bh(Q, K, V, theta_q, theta_k, G, S0, z0, **kw):
    """causal_bwd_state over [B, H, n, .] tensors, S0 [B, H, m, dv], z0 [B, H, m];
    a shared theta's gradient sums over the heads."""
    theta_q, theta_k = np.asarray(theta_q), np.asarray(theta_k)
    B, H = Q.shape[:2]
    dQ, dK, dV = np.zeros(Q.shape), np.zeros(K.shape), np.zeros(V.shape)
    dtq, dtk = np.zeros(theta_q.shape), np.zeros(theta_k.shape)
    dS0, dz0 = np.zeros(np.shape(S0)), np.zeros(np.shape(z0))
    for b in range(B):
        for h in range(H):
            r = causal_bwd_state(Q[b, h], K[b, h], V[b, h], _theta_for(theta_q, h),
                                 _theta_for(theta_k, h), G[b, h], S0[b, h], z0[b, h], **kw)
            dQ[b, h], dK[b, h], dV[b, h] = r[0], r[1], r[2]
            dS0[b, h], dz0[b, h] = r[5], r[6]
            if theta_q.ndim == 5:
                dtq[h] += r[3]
            else:
                dtq += r[3]
            if theta_k.ndim == 5:
                dtk[h] += r[4]
            else:
                dtk += r[4]
    return dQ, dK, dV, dtq, dtk, dS0, dz0


def causal_attn_bwd_chunked(Pq, Pk, V, G, normalize=False, delta=0.0, chunk=256):
    """causal_attn_bwd without the n x n matrix, for long sequences: the same
    sums split at chunk boundaries. Prefix states S = sum Pk^T V, z = sum Pk
    of earlier chunks give num, den and dPq; suffix states R = sum Pq^T dnum,
    r = sum Pq^T dden of later chunks give dPk and dV; inside a chunk the
    masked products are explicit ([LowRank-blog] causal masking by running
    sums, taken in both directions)."""
    Pq, Pk, V, G = _f64(Pq), _f64(Pk), _f64(V), _f64(G)
    n, m = Pq.shape
    dv = V.shape[1]
    dnum = np.zeros((n, dv))
    dden = np.zeros(n)
    dPq = np.zeros((n, m))
    S, z = np.zeros((m, dv)), np.zeros(m)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        q, k, v, g = Pq[c0:c1], Pk[c0:c1], V[c0:c1], G[c0:c1]
        A = np.tril(q @ k.T)
        num = A @ v + q @ S
        if normalize:
            den = A.sum(axis=1) + q @ z + delta
            out = num / den[:, None]
            dn = g / den[:, None]
            dd = -(g * out).sum(axis=1) / den
        else:
            dn, dd = g, np.zeros(c1 - c0)
        dnum[c0:c1], dden[c0:c1] = dn, dd
        P = np.tril(dn @ v.T + dd[:, None])
        dPq[c0:c1] = dn @ S.T + np.outer(dd, z) + P @ k
        S = S + k.T @ v
        z = z + k.sum(axis=0)
    dPk = np.zeros((n, m))
    dV = np.zeros((n, dv))
    Rs, r = np.zeros((m, dv)), np.zeros(m)
    for c0 in reversed(range(0, n, chunk)):
        c1 = min(n, c0 + chunk)
        q, k, v = Pq[c0:c1], Pk[c0:c1], V[c0:c1]
        dn, dd = dnum[c0:c1], dden[c0:c1]
        A = np.tril(q @ k.T)
        P = np.tril(dn @ v.T + dd[:, None])
        dPk[c0:c1] = v @ Rs.T + r[None, :] + P.T @ q
        dV[c0:c1] = k @ Rs + A.T @ dn
        Rs = Rs + q.T @ dn
        r = r + q.T @ dd
    return dPq, dPk, dV


def causal_bwd(Q, K, V, theta_q, theta_k, G, square=False, normalize=False, delta=0.0):
    """Gradients (dQ, dK, dV, dTheta_q, dTheta_k) of L = sum(G * out) for
    out = causal_quadratic(Q, K, V, theta_q, theta_k, ...): causal_attn_bwd
    for the feature gradients, then featmap_bwd on each side (Theta is trained
    end to end: [LLoPS-notes] training strategy; [LLoPS-arXiv] Sec. 3)."""
    Pq = featmap(Q, theta_q, square)
    Pk = featmap(K, theta_k, square)
    dPq, dPk, dV = causal_attn_bwd(Pq, Pk, V, G, normalize, delta)
    dQ, dtq = featmap_bwd(Q, theta_q, dPq, square)
    dK, dtk = featmap_bwd(K, theta_k, dPk, square)
    return dQ, dK, dV, dtq, dtk


def state_from_prefix(K, V, theta_k, square=False):
    """S = phi_K^T V and z = phi_K^T 1 over a prefix (the state a causal pass
    over these tokens leaves behind). [LLoPS-arXiv] Sec. 1 (constant state)."""
    Pk = featmap(K, theta_k, square)
    return Pk.T @ _f64(V), Pk.sum(axis=0)


def decode(S0, z0, q_steps, k_steps, v_steps, theta_q, theta_k, square=False,
           normalize=True, delta=0.0):
    """Single-token recurrent steps for one (batch, head) slice.

    Each step: S += phi_k v^T; z += phi_k; o = phi_q^T S [/ (phi_q^T z + delta)]
    (state updated before it is read, matching the inclusive causal mask).
    q_steps, k_steps: [steps, d]; v_steps: [steps, dv].
    Returns (outs [steps, dv], S, z).
    [LLoPS-arXiv] Sec. 1 (recurrent memory state); [LowRank-blog] Performer
    section (sums over keys shared by all queries, updated incrementally).
    """
    S = _f64(S0).copy()
    z = _f64(z0).copy()
    outs = []
    for q, k, v in zip(_f64(q_steps), _f64(k_steps), _f64(v_steps)):
        fq = featmap(q[None], theta_q, square)[0]
        fk = featmap(k[None], theta_k, square)[0]
        S = S + np.outer(fk, v)
        z = z + fk
        o = fq @ S
        if normalize:
            o = o / (fq @ z + delta)
        outs.append(o)
    return np.array(outs), S, z


# --------------------------------------------------------------------------
# Batched wrappers over [B, H, n, *] with per-head (or shared) Theta
# --------------------------------------------------------------------------
def gated_causal_quadratic(Q, K, V, theta_q, theta_k, log_gate, square=False, normalize=False,
                           delta=0.0, S0=None, z0=None):
    """Causal attention with a per-token scalar decay, materialised: with
    c = cumsum(log_gate),
      M_ij = exp(c_i - c_j) (phi_Q,i . phi_K,j) for j <= i, else 0,
      num_i = (M V)_i + exp(c_i) phi_Q,i S0,  den_i = (M 1)_i + exp(c_i) phi_Q,i z0 + delta,
      out = num [/ den].
    The semiseparable (decay-masked) form of Mamba2 that [LLoPS-notes]
    conclusion names for combining the sketch with forgetting gates, on the
    attention of [LLoPS-arXiv] Sec. 1. O(n^2); small n only."""
    Pq = featmap(Q, theta_q, square)
    Pk = featmap(K, theta_k, square)
    V = _f64(V)
    c = np.cumsum(_f64(log_gate))
    n = Pq.shape[0]
    i, j = np.arange(n)[:, None], np.arange(n)[None, :]
    W = np.where(j <= i, np.exp(np.where(j <= i, c[:, None] - c[None, :], 0.0)), 0.0)
    M = W * (Pq @ Pk.T)
    num = M @ V
    den = M.sum(axis=1)
    if S0 is not None:
        num = num + np.exp(c)[:, None] * (Pq @ _f64(S0))
    if z0 is not None:
        den = den + np.exp(c) * (Pq @ _f64(z0))
    if not normalize:
        return num
    return num / (den + delta)[:, None]


def gated_recurrent(Q, K, V, theta_q, theta_k, log_gate, square=False, normalize=False,
                    delta=0.0, S0=None, z0=None):
    """The same gated attention token by token (the recurrent form of
    [LLoPS-arXiv] Sec. 1 with the decay of [LLoPS-notes] conclusion):
      S <- exp(g_i) S + phi_K,i v_i^T,  z <- exp(g_i) z + phi_K,i,
      out_i = phi_Q,i S [/ (phi_Q,i z + delta)].
    Returns (out [n, dv], S, z)."""
    Pq = featmap(Q, theta_q, square)
    Pk = featmap(K, theta_k, square)
    V = _f64(V)
    g = _f64(log_gate)
    m, dv = Pq.shape[1], V.shape[1]
    S = np.zeros((m, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros(m) if z0 is None else _f64(z0).copy()
    out = np.zeros((Pq.shape[0], dv))
    for t in range(Pq.shape[0]):
        a = np.exp(g[t])
        S = a * S + np.outer(Pk[t], V[t])
        z = a * z + Pk[t]
        o = Pq[t] @ S
        out[t] = o / (Pq[t] @ z + delta) if normalize else o
    return out, S, z


def gated_recurrent_bh(Q, K, V, theta_q, theta_k, log_gate, S0=None, z0=None, **kw):
    """gated_recurrent over [B, H, n, .] tensors, log_gate [B, H, n].
    Returns (out [B,H,n,dv], S [B,H,m,dv], z [B,H,m])."""
    B, H, n, _ = Q.shape
    m = np.asarray(theta_q).shape[-1]
    dv = V.shape[-1]
    out, S, z = np.zeros((B, H, n, dv)), np.zeros((B, H, m, dv)), np.zeros((B, H, m))
    for b in range(B):
        for h in range(H):
            out[b, h], S[b, h], z[b, h] = gated_recurrent(
                Q[b, h], K[b, h], V[b, h], _theta_for(theta_q, h), _theta_for(theta_k, h),
                log_gate[b, h], S0=None if S0 is None else S0[b, h],
                z0=None if z0 is None else z0[b, h], **kw)
    return out, S, z


def gated_attn_bwd(Pq, Pk, V, G, log_gate, normalize=False, delta=0.0):
    """Gradients (dPq, dPk, dV, dg) of L = sum(G * out) for the gated causal
    contraction from a zero state, out = M V [/ (M 1 + delta)] with
    M_ij = W_ij (Pq_i . Pk_j), W_ij = exp(c_i - c_j) for j <= i (else 0) and
    c = cumsum(log_gate): the chain rule through the materialised form of
    gated_causal_quadratic ([LLoPS-notes] limitations and outlook for the
    gate; [LLoPS-arXiv] Sec. 1 attention form; [SLAY-notes] key design 3):
      dnum, dden as in causal_attn_bwd;  dM = tril(dnum V^T + dden 1^T),
      dPq = (dM * W) Pk,  dPk = (dM * W)^T Pq,  dV = M^T dnum,
      dc_i = sum_j (dM * M)_ij - sum_k (dM * M)_ki   (c_i enters row i with +,
             column i with -),  dg_l = sum_{i >= l} dc_i   (c_i = sum_{l <= i} g_l)."""
    Pq, Pk, V, G = _f64(Pq), _f64(Pk), _f64(V), _f64(G)
    c = np.cumsum(_f64(log_gate))
    n = Pq.shape[0]
    i, j = np.arange(n)[:, None], np.arange(n)[None, :]
    W = np.where(j <= i, np.exp(np.where(j <= i, c[:, None] - c[None, :], 0.0)), 0.0)
    M = W * (Pq @ Pk.T)
    if normalize:
        den = M.sum(axis=1) + delta
        out = (M @ V) / den[:, None]
        dnum = G / den[:, None]
        dden = -(G * out).sum(axis=1) / den
    else:
        dnum = G
        dden = np.zeros(n)
    dM = np.tril(dnum @ V.T + dden[:, None])
    dA = dM * W
    X = dM * M
    dc = X.sum(axis=1) - X.sum(axis=0)
    dg = np.cumsum(dc[::-1])[::-1]
    return dA @ Pk, dA.T @ Pq, M.T @ dnum, dg


def gated_attn_bwd_recurrent(Pq, Pk, V, G, log_gate, normalize=False, delta=0.0):
    """gated_attn_bwd without the n x n matrix, for long sequences: the same
    sums as running states. Forward, token by token: S_i = a_i S_{i-1} +
    Pk_i V_i^T, z_i = a_i z_i-1 + Pk_i (a_i = exp(g_i)) give num, den and
    dPq_i = S_i dnum_i + dden_i z_i. Backward over the tokens: R_j = Pq_j dnum_j^T
    + a_{j+1} R_{j+1}, r_j = dden_j Pq_j + a_{j+1} r_{j+1} give dPk_j = R_j V_j + r_j
    and dV_j = R_j^T Pk_j. The gate gradient uses (dM * M) row sums = Pq_i . dPq_i
    and column sums = Pk_j . dPk_j, so dc = rowdot(Pq, dPq) - rowdot(Pk, dPk)."""
    Pq, Pk, V, G = _f64(Pq), _f64(Pk), _f64(V), _f64(G)
    a = np.exp(_f64(log_gate))
    n, m = Pq.shape
    dv = V.shape[1]
    S, z = np.zeros((m, dv)), np.zeros(m)
    dnum, dden, dPq = np.zeros((n, dv)), np.zeros(n), np.zeros((n, m))
    for t in range(n):
        S = a[t] * S + np.outer(Pk[t], V[t])
        z = a[t] * z + Pk[t]
        num = Pq[t] @ S
        if normalize:
            den = Pq[t] @ z + delta
            dnum[t] = G[t] / den
            dden[t] = -(G[t] @ (num / den)) / den
        else:
            dnum[t] = G[t]
        dPq[t] = S @ dnum[t] + dden[t] * z
    R, r = np.zeros((m, dv)), np.zeros(m)
    dPk, dV = np.zeros((n, m)), np.zeros((n, dv))
    for t in reversed(range(n)):
        nxt = a[t + 1] if t + 1 < n else 0.0
        R = nxt * R + np.outer(Pq[t], dnum[t])
        r = nxt * r + dden[t] * Pq[t]
        dPk[t] = R @ V[t] + r
        dV[t] = R.T @ Pk[t]
    dc = (Pq * dPq).sum(axis=1) - (Pk * dPk).sum(axis=1)
    dg = np.cumsum(dc[::-1])[::-1]
    return dPq, dPk, dV, dg


def gated_attn_bwd_state(Pq, Pk, V, G, log_gate, S0, z0, normalize=False, delta=0.0):
    """gated_attn_bwd for the contraction continued from an initial state
    (gated_causal_quadratic's S0/z0, which reach query i with weight exp(c_i)):
      num = M V + exp(c) * (Pq S0),  den = M 1 + exp(c) * (Pq z0) + delta,
      dPq_i = ((dM * W) Pk)_i + exp(c_i) (S0 dnum_i + dden_i z0),
      dS0 = sum_i exp(c_i) Pq_i dnum_i^T,  dz0 = sum_i exp(c_i) dden_i Pq_i,
    and the gate term: the state's contribution to row i, X_i0 =
    exp(c_i) (dnum_i . S0^T Pq_i + dden_i Pq_i . z0), joins row i's sum in dc_i.
    Returns (dPq, dPk, dV, dg, dS0, dz0)."""
    Pq, Pk, V, G = _f64(Pq), _f64(Pk), _f64(V), _f64(G)
    S0, z0 = _f64(S0), _f64(z0)
    c = np.cumsum(_f64(log_gate))
    e = np.exp(c)
    n = Pq.shape[0]
    i, j = np.arange(n)[:, None], np.arange(n)[None, :]
    W = np.where(j <= i, np.exp(np.where(j <= i, c[:, None] - c[None, :], 0.0)), 0.0)
    M = W * (Pq @ Pk.T)
    num = M @ V + e[:, None] * (Pq @ S0)
    if normalize:
        den = M.sum(axis=1) + e * (Pq @ z0) + delta
        out = num / den[:, None]
        dnum = G / den[:, None]
        dden = -(G * out).sum(axis=1) / den
    else:
        dnum = G
        dden = np.zeros(n)
    dM = np.tril(dnum @ V.T + dden[:, None])
    dA = dM * W
    X = dM * M
    x0 = e * ((dnum * (Pq @ S0)).sum(axis=1) + dden * (Pq @ z0))
    dc = X.sum(axis=1) - X.sum(axis=0) + x0
    dg = np.cumsum(dc[::-1])[::-1]
    dPq = dA @ Pk + e[:, None] * (dnum @ S0.T + np.outer(dden, z0))
    dS0 = (e[:, None] * Pq).T @ dnum
    dz0 = (e[:, None] * Pq).T @ dden
    return dPq, dA.T @ Pq, M.T @ dnum, dg, dS0, dz0


def gated_causal_bwd_state(Q, K, V, theta_q, theta_k, log_gate, G, S0, z0, square=False,
                           normalize=False, delta=0.0):
    """gated_causal_bwd from an initial state:
    (dQ, dK, dV, dTheta_q, dTheta_k, dlog_gate, dS0, dz0)."""
    Pq = featmap(Q, theta_q, square)
    Pk = featmap(K, theta_k, square)
    dPq, dPk, dV, dg, dS0, dz0 = gated_attn_bwd_state(Pq, Pk, V, G, log_gate, S0, z0, normalize,
                                                      delta)
    dQ, dtq = featmap_bwd(Q, theta_q, dPq, square)
    dK, dtk = featmap_bwd(K, theta_k, dPk, square)
    return dQ, dK, dV, dtq, dtk, dg, dS0, dz0


def gated_causal_bwd(Q, K, V, theta_q, theta_k, log_gate, G, square=False, normalize=False,
                     delta=0.0, recurrent=False):
    """Gradients (dQ, dK, dV, dTheta_q, dTheta_k, dlog_gate) of L = sum(G * out)
    for out = gated_causal_quadratic(...) from a zero state: the feature
    gradients (materialised, or the running-state form when recurrent), then
    featmap_bwd on each side."""
    Pq = featmap(Q, theta_q, square)
    Pk = featmap(K, theta_k, square)
    fn = gated_attn_bwd_recurrent if recurrent else gated_attn_bwd
    dPq, dPk, dV, dg = fn(Pq, Pk, V, G, log_gate, normalize, delta)
    dQ, dtq = featmap_bwd(Q, theta_q, dPq, square)
    dK, dtk = featmap_bwd(K, theta_k, dPk, square)
    return dQ, dK, dV, dtq, dtk, dg


def gated_causal_bwd_bh(Q, K, V, theta_q, theta_k, log_gate, G, **kw):
    """gated_causal_bwd over [B, H, n, .] tensors (log_gate [B, H, n]); a
    shared theta's gradient sums over the heads."""
    theta_q, theta_k = np.asarray(theta_q), np.asarray(theta_k)
    B, H = Q.shape[:2]
    dQ, dK, dV = np.zeros(Q.shape), np.zeros(K.shape), np.zeros(V.shape)
    dtq, dtk = np.zeros(theta_q.shape), np.zeros(theta_k.shape)
    dg = np.zeros(np.shape(log_gate))
    for b in range(B):
        for h in range(H):
            gq, gk, gv, tq, tk, gg = gated_causal_bwd(
                Q[b, h], K[b, h], V[b, h], _theta_for(theta_q, h), _theta_for(theta_k, h),
                log_gate[b, h], G[b, h], **kw)
            dQ[b, h], dK[b, h], dV[b, h], dg[b, h] = gq, gk, gv, gg
            if theta_q.ndim == 5:
                dtq[h] += tq
            else:
                dtq += tq
            if theta_k.ndim == 5:
                dtk[h] += tk
            else:
                dtk += tk
    return dQ, dK, dV, dtq, dtk, dg


def _theta_for(theta, h):
    theta = np.asarray(theta)
    return theta[h] if theta.ndim == 5 else theta


def featmap_bh(X, theta, square=False) -> np.ndarray:
    """featmap over X [B, H, n, d] with theta [H, p, t, d, m] or [p, t, d, m]."""
    B, H = X.shape[:2]
    m = np.asarray(theta).shape[-1]
    out = np.zeros((B, H, X.shape[2], m))
    for b in range(B):
        for h in range(H):
            out[b, h] = featmap(X[b, h], _theta_for(theta, h), square)
    return out


def featmap_bwd_bh(X, theta, dphi, square=False):
    """featmap_bwd over X [B, H, n, d] and dphi [B, H, n, m]; theta [H, p, t,
    d, m] or shared [p, t, d, m] (whose gradient then sums over all heads)."""
    theta = np.asarray(theta)
    B, H = X.shape[:2]
    dX = np.zeros(X.shape)
    dth = np.zeros(theta.shape)
    for b in range(B):
        for h in range(H):
            gx, gt = featmap_bwd(X[b, h], _theta_for(theta, h), dphi[b, h], square)
            dX[b, h] = gx
            if theta.ndim == 5:
                dth[h] += gt
            else:
                dth += gt
    return dX, dth


def linattn_bwd_bh(Q, K, V, theta_q, theta_k, G, **kw):
    """linattn_bwd over [B, H, n, .] tensors (shared theta: summed over heads)."""
    return _bwd_bh(linattn_bwd, Q, K, V, theta_q, theta_k, G, **kw)


def causal_bwd_bh(Q, K, V, theta_q, theta_k, G, **kw):
    """causal_bwd over [B, H, n, .] tensors; a shared theta's gradient sums
    over all heads. Returns (dQ, dK, dV, dTheta_q, dTheta_k)."""
    return _bwd_bh(causal_bwd, Q, K, V, theta_q, theta_k, G, **kw)


def _bwd_bh(fn, Q, K, V, theta_q, theta_k, G, **kw):
    theta_q, theta_k = np.asarray(theta_q), np.asarray(theta_k)
    B, H = Q.shape[:2]
    dQ, dK, dV = np.zeros(Q.shape), np.zeros(K.shape), np.zeros(V.shape)
    dtq, dtk = np.zeros(theta_q.shape), np.zeros(theta_k.shape)
    for b in range(B):
        for h in range(H):
            gq, gk, gv, tq, tk = fn(Q[b, h], K[b, h], V[b, h], _theta_for(theta_q, h),
                                    _theta_for(theta_k, h), G[b, h], **kw)
            dQ[b, h], dK[b, h], dV[b, h] = gq, gk, gv
            if theta_q.ndim == 5:
                dtq[h] += tq
            else:
                dtq += tq
            if theta_k.ndim == 5:
                dtk[h] += tk
            else:
                dtk += tk
    return dQ, dK, dV, dtq, dtk


def linattn_bh(Q, K, V, theta_q, theta_k, **kw) -> np.ndarray:
    B, H, n, _ = Q.shape
    out = np.zeros((B, H, n, V.shape[-1]))
    for b in range(B):
        for h in range(H):
            out[b, h] = linattn(Q[b, h], K[b, h], V[b, h], _theta_for(theta_q, h),
                                _theta_for(theta_k, h), **kw)
    return out


def causal_bh(Q, K, V, theta_q, theta_k, chunk=64, S0=None, z0=None, **kw):
    """Returns (out [B,H,n,dv], S [B,H,m,dv], z [B,H,m])."""
    B, H, n, _ = Q.shape
    m = np.asarray(theta_q).shape[-1]
    dv = V.shape[-1]
    out = np.zeros((B, H, n, dv))
    S = np.zeros((B, H, m, dv))
    z = np.zeros((B, H, m))
    for b in range(B):
        for h in range(H):
            s0 = None if S0 is None else S0[b, h]
            zz = None if z0 is None else z0[b, h]
            out[b, h], S[b, h], z[b, h] = causal_chunked(
                Q[b, h], K[b, h], V[b, h], _theta_for(theta_q, h),
                _theta_for(theta_k, h), chunk=chunk, S0=s0, z0=zz, **kw)
    return out, S, z
