"""GPU parity of every C-ABI entry point against the fp64 oracle on small
seeded inputs that still span several tiles, segments and ragged tails, plus
the edge cases (n = 0, n = 1, p = 1, t = 1, shared and aliased Theta, state
continuation, decode after prefill, bitwise repeatability)."""
import numpy as np
import pytest

from learnable_polynomial_feature_amd.workloads import Workload, generate
from oracle import llops_oracle as O

from _util import (TOL_BF16, TOL_F32, TOL_FEAT_BF16_IN, TOL_FEAT_BF16_OUT, TOL_ROW_BF16,
                    announce, dev, host, rel_fro, row_rel_max)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _w(B, H, n, d, dv, m, p, t, dtype="bf16", square=True, normalize=True, delta=1e-6, chunk=64,
       qk="gauss", seed=0):
    return Workload("case", batch=B, heads=H, n=n, d=d, dv=dv, p=p, t=t, m=m, dtype=dtype,
                    causal=True, square=square, normalize=normalize, delta=delta, chunk=chunk,
                    qk_dist=qk, seed=seed)


def _tdt(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def _inputs(w, shared=False):
    x = generate(w)
    if shared:
        x["theta_q"] = x["theta_q"][0]
        x["theta_k"] = x["theta_k"][0]
    tdt = _tdt(w)
    d = {k: dev(v, tdt) for k, v in x.items()}
    return x, d


# ---------------------------------------------------------------------------
# feature map
# ---------------------------------------------------------------------------
FEAT_CASES = [
    # B, H, n, d, m, p, t, square, shared, out_bf16
    (2, 3, 300, 64, 64, 2, 4, True, False, False),
    (1, 2, 513, 128, 256, 2, 4, True, False, False),
    (2, 2, 200, 64, 128, 3, 8, True, False, False),
    (1, 1, 100, 16, 32, 2, 2, False, False, False),
    (1, 2, 77, 48, 48, 1, 3, False, True, False),
    (3, 2, 50, 32, 16, 4, 1, True, False, True),
    (128, 4, 1, 128, 256, 2, 4, True, False, False),
    (1, 1, 600, 256, 64, 2, 2, False, False, False),
    (1, 1, 64, 128, 32, 8, 1, False, False, False),
    (2, 1, 257, 96, 80, 3, 5, True, True, True),
    # the unrolled 256-row-tile kernels, with ragged tiles, batch boundaries
    # inside a tile and an odd number of 32-feature blocks (bf16 phi is
    # stored in block pairs)
    (2, 2, 1100, 128, 256, 2, 4, True, False, False),
    (2, 2, 1100, 128, 256, 2, 4, True, False, True),
    (3, 1, 1000, 128, 64, 2, 1, False, True, True),
    (1, 2, 2100, 64, 64, 2, 4, True, False, True),
    (2, 1, 1500, 64, 128, 3, 8, True, False, False),
    (1, 1, 4096, 128, 80, 2, 4, False, False, False),
    (1, 1, 4096, 128, 80, 2, 4, True, False, True),
    (5, 3, 613, 128, 48, 2, 4, True, False, False),
    # few row tiles: feature blocks split over workgroups (one block each,
    # then two per workgroup with a single block left in the last group)
    (1, 3, 700, 128, 96, 2, 4, True, False, True),
    (2, 2, 300, 128, 160, 2, 1, False, False, True),
    (1, 8, 12800, 128, 160, 2, 1, True, False, True),
    # p = 4 on the unrolled kernels with four distinct Theta_j (each j, r is
    # its own seeded draw): the 256-row-tile kernels (> 1024 rows per head)
    # and the few-row kernels that read Theta in place (<= 1024 rows)
    (1, 2, 2100, 128, 256, 4, 1, True, False, True),
    (1, 2, 2100, 128, 256, 4, 1, False, True, False),
    (2, 2, 1100, 64, 128, 4, 1, False, False, False),
    (128, 4, 1, 128, 256, 4, 1, True, False, False),
    (300, 2, 1, 64, 64, 4, 1, True, False, True),
    # head dims that are multiples of 16 but not of 32 (generic kernel,
    # operands zeroed past d)
    (2, 2, 300, 80, 64, 2, 2, True, False, False),
    (1, 1, 200, 112, 48, 3, 1, False, False, True),
    (1, 1, 150, 240, 32, 2, 2, True, True, False),
]


@pytest.mark.parametrize("case", FEAT_CASES, ids=[str(c) for c in FEAT_CASES])
def test_featmap_bf16(lib, case):
    B, H, n, d, m, p, t, square, shared, out_bf16 = case
    w = _w(B, H, n, d, 16, m, p, t, square=square)
    x, g = _inputs(w, shared)
    announce(f"featmap bf16 {case}")
    odt = torch.bfloat16 if out_bf16 else torch.float32
    phi = lib.llops_featmap(g["Q"], g["theta_q"], square=square, out_dtype=odt)
    torch.cuda.synchronize()
    want = O.featmap_bh(x["Q"], x["theta_q"], square=square)
    err = rel_fro(host(phi), want)
    assert err <= (TOL_FEAT_BF16_OUT if out_bf16 else TOL_FEAT_BF16_IN), err


@pytest.mark.parametrize("case", [(1, 2, 3000, 128, 256, 2, 4), (2, 1, 1500, 64, 128, 3, 8),
                                  (1, 1, 300, 64, 64, 2, 4)])
def test_featmap_bf16_out_is_rounded_f32_out(lib, case):
    """Storing phi as bf16 rounds the same fp32 value the fp32 output holds
    (round to nearest even), bit for bit."""
    B, H, n, d, m, p, t = case
    w = _w(B, H, n, d, 16, m, p, t)
    _, g = _inputs(w)
    announce(f"featmap bf16 vs f32 out {case}")
    f32 = lib.llops_featmap(g["Q"], g["theta_q"], square=True, out_dtype=torch.float32)
    b16 = lib.llops_featmap(g["Q"], g["theta_q"], square=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(f32.to(torch.bfloat16), b16)


@pytest.mark.parametrize("case", [(2, 3, 37, 16, 32, 2, 2, True), (1, 1, 20, 7, 5, 3, 2, False),
                                  (2, 2, 64, 64, 64, 1, 1, True)])
def test_featmap_f32(lib, case):
    B, H, n, d, m, p, t, square = case
    w = _w(B, H, n, d, 4, m, p, t, dtype="f32", square=square)
    x, g = _inputs(w)
    announce(f"featmap f32 {case}")
    phi = lib.llops_featmap(g["Q"], g["theta_q"], square=square)
    torch.cuda.synchronize()
    err = rel_fro(host(phi), O.featmap_bh(x["Q"], x["theta_q"], square=square))
    assert err <= TOL_F32, err


def test_featmap_empty(lib):
    X = torch.zeros((2, 3, 0, 64), dtype=torch.bfloat16, device="cuda")
    th = torch.zeros((3, 2, 2, 64, 32), dtype=torch.bfloat16, device="cuda")
    phi = lib.llops_featmap(X, th)
    torch.cuda.synchronize()
    assert phi.shape == (2, 3, 0, 32)


# ---------------------------------------------------------------------------
# causal and non-causal attention
# ---------------------------------------------------------------------------
CAUSAL_CASES = [
    # B, H, n, d, dv, m, p, t, square, normalize, chunk
    (2, 3, 300, 64, 64, 64, 2, 4, True, True, 64),
    (2, 3, 300, 64, 64, 64, 2, 4, True, True, 32),
    (1, 2, 1000, 128, 128, 256, 2, 4, True, True, 128),
    (2, 2, 517, 64, 64, 128, 3, 8, True, True, 64),
    (1, 2, 200, 64, 32, 32, 2, 2, False, False, 64),
    (1, 3, 129, 32, 16, 32, 1, 1, True, True, 16),
    (2, 1, 90, 64, 48, 96, 2, 3, True, True, 64),
    (1, 1, 1, 64, 64, 64, 2, 2, True, True, 64),
    (3, 2, 33, 128, 128, 256, 2, 4, True, True, 64),
    (2, 2, 1500, 128, 128, 256, 2, 4, True, True, 128),
    (1, 2, 2500, 64, 64, 128, 3, 8, True, True, 64),
    (1, 2, 300, 80, 64, 64, 2, 2, True, True, 64),
]


@pytest.mark.parametrize("case", CAUSAL_CASES, ids=[str(c) for c in CAUSAL_CASES])
def test_causal_bf16(lib, case):
    B, H, n, d, dv, m, p, t, square, normalize, chunk = case
    w = _w(B, H, n, d, dv, m, p, t, square=square, normalize=normalize, chunk=chunk)
    x, g = _inputs(w)
    announce(f"causal bf16 {case}")
    out, S, z = lib.llops_linattn_causal_fwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"],
                                             square=square, normalize=normalize, delta=1e-6,
                                             chunk=chunk, return_state=True)
    torch.cuda.synchronize()
    ro, rS, rz = O.causal_bh(x["Q"], x["K"], x["V"], x["theta_q"], x["theta_k"], chunk=64,
                             square=square, normalize=normalize, delta=1e-6)
    assert rel_fro(host(out), ro) <= TOL_BF16
    if normalize:  # delta decides the first rows: bound every row
        assert row_rel_max(host(out), ro) <= TOL_ROW_BF16, row_rel_max(host(out), ro)
    assert rel_fro(host(S), rS) <= TOL_BF16
    assert rel_fro(host(z), rz) <= TOL_BF16


@pytest.mark.parametrize("case", [(1, 1, 256, 16, 16, 32, 2, 2, False, False, 0),
                                  (2, 2, 150, 16, 8, 24, 3, 2, True, True, 16),
                                  (1, 2, 300, 32, 20, 40, 2, 3, True, True, 128),
                                  (1, 1, 70, 5, 3, 7, 2, 2, False, True, 32)])
def test_causal_f32(lib, case):
    B, H, n, d, dv, m, p, t, square, normalize, chunk = case
    w = _w(B, H, n, d, dv, m, p, t, dtype="f32", square=square, normalize=normalize,
           chunk=chunk, delta=1e-3)
    x, g = _inputs(w)
    announce(f"causal f32 {case}")
    out, S, z = lib.llops_linattn_causal_fwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"],
                                             square=square, normalize=normalize, delta=1e-3,
                                             chunk=chunk, return_state=True)
    torch.cuda.synchronize()
    ro, rS, rz = O.causal_bh(x["Q"], x["K"], x["V"], x["theta_q"], x["theta_k"], chunk=64,
                             square=square, normalize=normalize, delta=1e-3)
    assert rel_fro(host(out), ro) <= TOL_F32
    assert rel_fro(host(S), rS) <= TOL_F32
    assert rel_fro(host(z), rz) <= TOL_F32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("normalize", [True, False])
def test_noncausal(lib, dtype, normalize):
    if dtype == "bf16":
        w = _w(2, 3, 300, 64, 64, 64, 2, 4, square=True, normalize=normalize)
        tol = TOL_BF16
    else:
        w = _w(1, 1, 256, 16, 16, 32, 2, 2, dtype="f32", square=False, normalize=normalize,
               delta=1e-3)
        tol = TOL_F32
    x, g = _inputs(w)
    announce(f"noncausal {dtype} normalize={normalize}")
    out = lib.llops_linattn_fwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"],
                                square=w.square, normalize=normalize, delta=w.delta)
    torch.cuda.synchronize()
    want = O.linattn_bh(x["Q"], x["K"], x["V"], x["theta_q"], x["theta_k"], square=w.square,
                        normalize=normalize, delta=w.delta)
    assert rel_fro(host(out), want) <= tol


# fp32 non-causal shapes. The first five take the one-launch kernel for small
# sequences (d = 16, m = 32, p = 2, t = 2, n <= 1024, dv a multiple of 4), with
# a ragged last 256-row tile, one row, dv = 4 and 8, and a shared Theta; the
# rest take the segment passes (n above 1024; other (d, m, p, t)).
# Normalised cases with an unsquared map stay short: there phi_Q z can come
# near zero, and a longer sum leaves fp32 short of the 1e-5 bound on both paths
F32_NONCAUSAL = [
    # B, H, n, d, dv, m, p, t, square, normalize, shared
    (1, 1, 1, 16, 16, 32, 2, 2, False, True, False),
    (2, 3, 33, 16, 8, 32, 2, 2, True, True, False),
    (1, 2, 64, 16, 16, 32, 2, 2, False, True, True),
    (2, 2, 130, 16, 4, 32, 2, 2, True, False, False),
    (3, 1, 700, 16, 16, 32, 2, 2, True, True, False),
    (1, 2, 1500, 16, 16, 32, 2, 2, True, True, False),
    (2, 3, 100, 16, 12, 32, 3, 1, True, False, False),
    (1, 2, 64, 8, 16, 16, 2, 2, False, True, True),
    (1, 1, 200, 10, 6, 24, 2, 2, True, True, False),
]


@pytest.mark.parametrize("case", F32_NONCAUSAL, ids=[str(c) for c in F32_NONCAUSAL])
def test_noncausal_f32_shapes(lib, case):
    B, H, n, d, dv, m, p, t, square, normalize, shared = case
    w = _w(B, H, n, d, dv, m, p, t, dtype="f32", square=square, normalize=normalize, delta=1e-3)
    x, g = _inputs(w, shared=shared)
    announce(f"noncausal f32 {case}")
    out = lib.llops_linattn_fwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"],
                                square=square, normalize=normalize, delta=1e-3)
    torch.cuda.synchronize()
    want = O.linattn_bh(x["Q"], x["K"], x["V"], x["theta_q"], x["theta_k"], square=square,
                        normalize=normalize, delta=1e-3)
    assert rel_fro(host(out), want) <= TOL_F32
    assert row_rel_max(host(out), want) <= 10 * TOL_F32


@pytest.mark.parametrize("shape", [(2, 2, 333, 64, 64, 128, 3, 2), (1, 3, 200, 64, 64, 64, 2, 2),
                                   (1, 2, 150, 128, 48, 96, 2, 2)])
def test_noncausal_bf16_normalised_shapes(lib, shape):
    """Every (m, dv) kernel variant, including the split of the normaliser
    state over waves, against the plain non-causal definition."""
    B, H, n, d, dv, m, p, t = shape
    w = _w(B, H, n, d, dv, m, p, t, square=True, normalize=True)
    x, g = _inputs(w)
    announce(f"noncausal bf16 normalised {shape}")
    out = lib.llops_linattn_fwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"], square=True,
                                normalize=True, delta=1e-6)
    torch.cuda.synchronize()
    want = O.linattn_bh(x["Q"], x["K"], x["V"], x["theta_q"], x["theta_k"], square=True,
                        normalize=True, delta=1e-6)
    assert rel_fro(host(out), want) <= TOL_BF16


def test_noncausal_bf16_large_head(lib):
    w = _w(1, 2, 700, 128, 128, 256, 2, 4, square=True, normalize=True)
    x, g = _inputs(w)
    announce("noncausal bf16 m=256 dv=128")
    out = lib.llops_linattn_fwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"], square=True,
                                normalize=True, delta=1e-6)
    torch.cuda.synchronize()
    want = O.linattn_bh(x["Q"], x["K"], x["V"], x["theta_q"], x["theta_k"], square=True,
                        normalize=True, delta=1e-6)
    assert rel_fro(host(out), want) <= TOL_BF16


def test_causal_shared_and_aliased_theta(lib):
    w = _w(2, 2, 150, 64, 64, 64, 2, 2)
    x, g = _inputs(w, shared=True)
    announce("causal shared theta, theta_q is theta_k")
    out = lib.llops_linattn_causal_fwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_q"],
                                       square=True, normalize=True, delta=1e-6)
    torch.cuda.synchronize()
    ro, _, _ = O.causal_bh(x["Q"], x["K"], x["V"], x["theta_q"], x["theta_q"], chunk=64,
                           square=True, normalize=True, delta=1e-6)
    assert rel_fro(host(out), ro) <= TOL_BF16


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causal_state_continuation(lib, dtype):
    w = _w(2, 2, 300, 64, 64, 64, 2, 3, dtype=dtype, delta=1e-3)
    x, g = _inputs(w)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    kw = dict(square=True, normalize=True, delta=1e-3)
    announce(f"causal continuation {dtype}")
    full, Sf, zf = lib.llops_linattn_causal_fwd(g["Q"], g["K"], g["V"], g["theta_q"],
                                                g["theta_k"], return_state=True, **kw)
    n1 = 130
    a, S1, z1 = lib.llops_linattn_causal_fwd(g["Q"][:, :, :n1], g["K"][:, :, :n1],
                                             g["V"][:, :, :n1], g["theta_q"], g["theta_k"],
                                             return_state=True, **kw)
    b, S2, z2 = lib.llops_linattn_causal_fwd(g["Q"][:, :, n1:], g["K"][:, :, n1:],
                                             g["V"][:, :, n1:], g["theta_q"], g["theta_k"],
                                             S0=S1, z0=z1, return_state=True, **kw)
    torch.cuda.synchronize()
    ro, rS, rz = O.causal_bh(x["Q"], x["K"], x["V"], x["theta_q"], x["theta_k"], chunk=64, **kw)
    got = np.concatenate([host(a), host(b)], axis=2)
    assert rel_fro(got, ro) <= tol
    assert rel_fro(host(S2), rS) <= tol
    assert rel_fro(host(z2), rz) <= tol
    assert rel_fro(got, host(full)) <= tol


def test_causal_empty_sequence_passes_state_through(lib):
    w = _w(2, 2, 0, 64, 32, 64, 2, 2)
    B, H, m, dv = 2, 2, 64, 32
    Q = torch.zeros((B, H, 0, 64), dtype=torch.bfloat16, device="cuda")
    V = torch.zeros((B, H, 0, dv), dtype=torch.bfloat16, device="cuda")
    th = torch.zeros((H, 2, 2, 64, m), dtype=torch.bfloat16, device="cuda")
    S0 = torch.randn((B, H, m, dv), device="cuda")
    z0 = torch.rand((B, H, m), device="cuda")
    announce("causal n=0")
    out, S, z = lib.llops_linattn_causal_fwd(Q, Q, V, th, th, S0=S0, z0=z0, square=True,
                                             normalize=True, delta=1e-6, return_state=True)
    torch.cuda.synchronize()
    assert out.shape == (B, H, 0, dv)
    assert torch.equal(S, S0) and torch.equal(z, z0)
    _, S, z = lib.llops_linattn_causal_fwd(Q, Q, V, th, th, return_state=True)
    torch.cuda.synchronize()
    assert float(S.abs().max()) == 0.0 and float(z.abs().max()) == 0.0
    del w


def test_causal_bitwise_repeatable(lib):
    w = _w(1, 4, 777, 128, 128, 256, 2, 4)
    _, g = _inputs(w)
    announce("causal repeatability")
    args = (g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"])
    o1 = lib.llops_linattn_causal_fwd(*args, square=True, normalize=True, delta=1e-6)
    o2 = lib.llops_linattn_causal_fwd(*args, square=True, normalize=True, delta=1e-6)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", [(4, 3, 128, 128, 256, 2, 4, "bf16", 40),
                                  (3, 2, 64, 64, 64, 3, 2, "bf16", 33),
                                  (2, 2, 16, 10, 24, 2, 2, "f32", 20),
                                  (2, 1, 32, 6, 16, 2, 1, "f32", 5)])
def test_decode(lib, case):
    """Steps from an oracle-built prefix state: outputs every step, final S, z."""
    B, H, d, dv, m, p, t, dtype, prefix = case
    steps = 5
    w = _w(B, H, prefix + steps, d, dv, m, p, t, dtype=dtype, delta=1e-6)
    x, g = _inputs(w)
    S0 = np.zeros((B, H, m, dv))
    z0 = np.zeros((B, H, m))
    thq = x["theta_q"]
    thk = x["theta_k"]
    for b in range(B):
        for h in range(H):
            S0[b, h], z0[b, h] = O.state_from_prefix(x["K"][b, h, :prefix], x["V"][b, h, :prefix],
                                                     thk[h], square=True)
    S = torch.from_numpy(S0.astype(np.float32)).cuda()
    z = torch.from_numpy(z0.astype(np.float32)).cuda()
    S0r, z0r = S0.astype(np.float32), z0.astype(np.float32)
    announce(f"decode {case}")
    outs = []
    for s in range(steps):
        i = prefix + s
        outs.append(lib.llops_decode_step(g["Q"][:, :, i], g["K"][:, :, i], g["V"][:, :, i],
                                          g["theta_q"], g["theta_k"], S, z, square=True,
                                          normalize=True, delta=1e-6))
    torch.cuda.synchronize()
    got = np.stack([host(o) for o in outs], axis=2)  # [B, H, steps, dv]
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    want = np.zeros_like(got)
    Sw = np.zeros((B, H, m, dv))
    zw = np.zeros((B, H, m))
    for b in range(B):
        for h in range(H):
            sl = slice(prefix, prefix + steps)
            want[b, h], Sw[b, h], zw[b, h] = O.decode(S0r[b, h], z0r[b, h], x["Q"][b, h, sl],
                                                      x["K"][b, h, sl], x["V"][b, h, sl], thq[h],
                                                      thk[h], square=True, normalize=True,
                                                      delta=1e-6)
    assert rel_fro(got, want) <= tol
    assert rel_fro(host(S), Sw) <= tol
    assert rel_fro(host(z), zw) <= tol


def test_decode_after_prefill_matches_prefill_rows(lib):
    w = _w(2, 2, 105, 128, 128, 256, 2, 4)
    x, g = _inputs(w)
    kw = dict(square=True, normalize=True, delta=1e-6)
    announce("decode after prefill")
    n1 = 100
    full = lib.llops_linattn_causal_fwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"], **kw)
    _, S, z = lib.llops_linattn_causal_fwd(g["Q"][:, :, :n1], g["K"][:, :, :n1],
                                           g["V"][:, :, :n1], g["theta_q"], g["theta_k"],
                                           return_state=True, **kw)
    outs = [lib.llops_decode_step(g["Q"][:, :, i], g["K"][:, :, i], g["V"][:, :, i],
                                  g["theta_q"], g["theta_k"], S, z, **kw) for i in range(n1, 105)]
    torch.cuda.synchronize()
    got = np.stack([host(o) for o in outs], axis=2)
    assert rel_fro(got, host(full)[:, :, n1:]) <= TOL_BF16
    ro, _, _ = O.causal_bh(x["Q"], x["K"], x["V"], x["theta_q"], x["theta_k"], chunk=64, **kw)
    assert rel_fro(got, ro[:, :, n1:]) <= TOL_BF16


def test_bad_workspace_raises_before_launch(lib):
    w = _w(1, 1, 64, 64, 64, 64, 2, 2)
    _, g = _inputs(w)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(lib.LlopsError, match="WORKSPACE"):
        lib.llops_linattn_causal_fwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"],
                                     workspace=small)
