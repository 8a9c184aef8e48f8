"""GPU parity of llops_linattn_gated_causal_bwd (gradients of sum(dO * out)
with respect to Q, K, V, Theta_q, Theta_k and the log gates) against the
fp64 oracle's chain rule through the decay-masked form, on seeded inputs with
ragged tails: plain and normalised, squared and not, t = 1 and 4, shared
Theta, strong decay, n = 1, no rows, zero gates against the ungated backward,
and 1 x 32 x 65536 on sampled heads (the running-state oracle, pinned to the
materialised one). Normalised cases use the squared map, as for the ungated
backward."""
import numpy as np
import pytest

from learnable_polynomial_feature_amd.workloads import (WORKLOADS, Workload, dout, generate,
                                                         log_gates)
from oracle import llops_oracle as O

from _util import TOL_BF16, announce, dev, host, rel_fro

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAMES = ("dQ", "dK", "dV", "dtheta_q", "dtheta_k", "dlog_gate")


def _w(B, H, n, d, dv, m, t, square, normalize, seed=0):
    return Workload("gbwd", batch=B, heads=H, n=n, d=d, dv=dv, p=2, t=t, m=m, dtype="bf16",
                    causal=True, square=square, normalize=normalize, delta=1e-6, chunk=64,
                    seed=seed)


CASES = [
    # B, H, n, d, dv, m, t, square, normalize, shared, mu (gate u ~ N(mu, 1))
    (1, 2, 300, 64, 64, 64, 4, True, True, False, 3.0),
    (2, 1, 257, 128, 128, 256, 4, True, True, False, 4.0),
    (1, 2, 500, 128, 64, 128, 1, False, False, True, 2.0),
    (1, 2, 400, 64, 64, 64, 4, True, True, False, 0.0),
    (1, 1, 1, 128, 128, 256, 4, True, False, False, 4.0),
    (1, 1, 2048, 128, 128, 256, 4, True, True, False, 4.0),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_gated_bwd(lib, case):
    B, H, n, d, dv, m, t, square, normalize, shared, mu = case
    w = _w(B, H, n, d, dv, m, t, square, normalize)
    x = generate(w)
    if shared:
        x["theta_q"], x["theta_k"] = x["theta_q"][0], x["theta_k"][0]
    G = dout(w)
    lg = log_gates(w, mu=mu)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    announce(f"gated_bwd {case}")
    got = lib.llops_linattn_gated_causal_bwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"],
                                             dev(lg, torch.float32), dev(G, torch.float32),
                                             square=square, normalize=normalize, delta=w.delta)
    torch.cuda.synchronize()
    want = O.gated_causal_bwd_bh(x["Q"], x["K"], x["V"], x["theta_q"], x["theta_k"], lg, G,
                                 square=square, normalize=normalize, delta=w.delta)
    errs = {nm: rel_fro(host(a), b) for nm, a, b in zip(NAMES, got, want)}
    print(f"[gated_bwd] {case} {errs}", flush=True)
    for nm, err in errs.items():
        assert err <= TOL_BF16, (nm, err)



@pytest.mark.parametrize("case", [CASES[0], CASES[1]], ids=[str(CASES[0]), str(CASES[1])])
def test_gated_bwd_reversed_form(lib, case, monkeypatch):
    """The reversed-copy form of the suffix sums (the fallback for phi too long
    for a 32-bit view), selected with LLOPS_BWD_REVERSED=1, against the oracle."""
    monkeypatch.setenv("LLOPS_BWD_REVERSED", "1")
    test_gated_bwd(lib, case)

@pytest.mark.parametrize("case", [CASES[1], CASES[4], CASES[5]],
                         ids=[str(CASES[1]), str(CASES[4]), str(CASES[5])])
@pytest.mark.parametrize("state", [False, True], ids=["no_state", "state"])
def test_gated_bwd_narrow_equals_padded(lib, case, state, monkeypatch):
    """On the m = 256, dv = 128 kernels the gated chain-rule passes read
    [dnum | dden | 0] from a narrow copy and [V | 1 | 0] from V itself;
    LLOPS_BWD_PADDED=1 selects the padded copies. Every gradient, the
    log-gate one and (from an initial state) dS0, dz0 included, agrees bit
    for bit."""
    B, H, n, d, dv, m, t, square, normalize, shared, mu = case
    w = _w(B, H, n, d, dv, m, t, square, normalize, seed=7)
    x = generate(w)
    G = dev(dout(w), torch.float32)
    lg = dev(log_gates(w, mu=mu), torch.float32)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    rng = np.random.default_rng(41)
    S0 = dev((0.01 * rng.standard_normal((B, H, m, dv))).astype(np.float32), torch.float32)
    z0 = dev(np.abs(0.01 * rng.standard_normal((B, H, m))).astype(np.float32), torch.float32)
    announce(f"gated_bwd narrow vs padded {case} state={state}")

    def run():
        if state:
            out = lib.llops_linattn_gated_causal_bwd_state(
                g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"], lg, G, S0=S0, z0=z0,
                square=square, normalize=normalize, delta=w.delta)
        else:
            out = lib.llops_linattn_gated_causal_bwd(g["Q"], g["K"], g["V"], g["theta_q"],
                                                     g["theta_k"], lg, G, square=square,
                                                     normalize=normalize, delta=w.delta)
        torch.cuda.synchronize()
        return out
    narrow = run()
    monkeypatch.setenv("LLOPS_BWD_PADDED", "1")
    padded = run()
    assert len(narrow) == len(padded)
    for i, (a, b) in enumerate(zip(narrow, padded)):
        assert torch.equal(a, b), i


def test_gated_bwd_zero_gate_matches_ungated(lib):
    """log_gate = 0: the same gradients as llops_linattn_causal_bwd (different
    kernels and rounding order), and the gate gradient against the oracle."""
    w = _w(1, 2, 700, 128, 128, 256, 4, True, True)
    x = generate(w)
    G = dout(w)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    zero = np.zeros((1, 2, 700), np.float32)
    announce("gated_bwd zero gate")
    got = lib.llops_linattn_gated_causal_bwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"],
                                             dev(zero, torch.float32), dev(G, torch.float32),
                                             square=True, normalize=True, delta=w.delta)
    ref = lib.llops_linattn_causal_bwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"],
                                       dev(G, torch.float32), square=True, normalize=True,
                                       delta=w.delta)
    torch.cuda.synchronize()
    for nm, a, b in zip(NAMES, got[:5], ref):
        assert rel_fro(host(a), host(b)) <= 1e-2, nm
    want = O.gated_causal_bwd_bh(x["Q"], x["K"], x["V"], x["theta_q"], x["theta_k"], zero, G,
                                 square=True, normalize=True, delta=w.delta)
    assert rel_fro(host(got[5]), want[5]) <= TOL_BF16


def test_gated_bwd_no_rows(lib):
    w = _w(1, 2, 0, 64, 64, 64, 4, True, True)
    th = dev(generate(w.replace(n=1))["theta_q"], torch.bfloat16)
    Q = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    V = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    G = torch.empty((1, 2, 0, 64), dtype=torch.float32, device="cuda")
    lg = torch.empty((1, 2, 0), dtype=torch.float32, device="cuda")
    announce("gated_bwd n=0")
    dQ, dK, dV, dtq, dtk, dg = lib.llops_linattn_gated_causal_bwd(Q, Q, V, th, th, lg, G,
                                                                  square=True, normalize=True,
                                                                  delta=1e-6)
    torch.cuda.synchronize()
    assert dQ.numel() == 0 and dV.numel() == 0 and dg.numel() == 0
    assert torch.count_nonzero(dtq).item() == 0 and torch.count_nonzero(dtk).item() == 0


@pytest.mark.slow
def test_gated_bwd_full_size_sampled(lib):
    """1 x 32 x 65536 (d = dv = 128, m = 256, p = 2, t = 4, squared,
    normalised), retention-biased gates: all heads on the GPU; heads 0 and 31
    against the running-state fp64 oracle."""
    w = WORKLOADS["causal_long_n65536"]
    x = generate(w)
    G = dout(w)
    lg = log_gates(w, mu=4.0)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    announce("gated_bwd full size")
    got = lib.llops_linattn_gated_causal_bwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"],
                                             dev(lg, torch.float32), dev(G, torch.float32),
                                             square=w.square, normalize=w.normalize,
                                             delta=w.delta)
    torch.cuda.synchronize()
    for h in (0, 31):
        want = O.gated_causal_bwd(x["Q"][0, h], x["K"][0, h], x["V"][0, h], x["theta_q"][h],
                                  x["theta_k"][h], lg[0, h], G[0, h], square=w.square,
                                  normalize=w.normalize, delta=w.delta, recurrent=True)
        sel = (got[0][0, h], got[1][0, h], got[2][0, h], got[3][h], got[4][h], got[5][0, h])
        errs = {nm: rel_fro(host(a), b) for nm, a, b in zip(NAMES, sel, want)}
        print(f"[gated_bwd full] head {h} {errs}", flush=True)
        for nm, err in errs.items():
            assert err <= TOL_BF16, (h, nm, err)


def test_gated_bwd_shared_aliased_theta(lib):
    """One shared Theta passed as both theta_q and theta_k: the two gradients
    come back apart, each summed over the heads."""
    w = _w(2, 3, 200, 64, 64, 64, 4, True, True)
    x = generate(w)
    th = x["theta_q"][0]
    G = dout(w)
    lg = log_gates(w, mu=2.0)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    gth = dev(th, torch.bfloat16)
    announce("gated_bwd shared aliased theta")
    got = lib.llops_linattn_gated_causal_bwd(g["Q"], g["K"], g["V"], gth, gth,
                                             dev(lg, torch.float32), dev(G, torch.float32),
                                             square=True, normalize=True, delta=w.delta)
    torch.cuda.synchronize()
    want = O.gated_causal_bwd_bh(x["Q"], x["K"], x["V"], th, th, lg, G, square=True,
                                 normalize=True, delta=w.delta)
    for nm, a, b in zip(NAMES, got, want):
        assert rel_fro(host(a), b) <= TOL_BF16, nm


@pytest.mark.parametrize("case", [
    # B, H, n, d, dv, m, t, square, normalize, mu
    (1, 2, 300, 64, 64, 64, 4, True, True, 3.0),
    (2, 1, 257, 128, 128, 256, 4, True, True, 4.0),
    (1, 2, 500, 128, 64, 128, 1, False, False, 2.0),
    (1, 2, 400, 64, 64, 64, 4, True, True, 0.0),
])
def test_gated_bwd_from_initial_state(lib, case):
    """llops_linattn_gated_causal_bwd_state: the gated forward continued from
    (S0, z0); all eight gradients against the fp64 chain rule."""
    B, H, n, d, dv, m, t, square, normalize, mu = case
    w = _w(B, H, n, d, dv, m, t, square, normalize)
    x = generate(w)
    G = dout(w)
    lg = log_gates(w, mu=mu)
    rng = np.random.default_rng(41)
    S0 = (0.01 * rng.standard_normal((B, H, m, dv))).astype(np.float32)
    z0 = np.abs(0.01 * rng.standard_normal((B, H, m))).astype(np.float32)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    announce(f"gated_bwd_state {case}")
    got = lib.llops_linattn_gated_causal_bwd_state(
        g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"], dev(lg, torch.float32),
        dev(G, torch.float32), S0=dev(S0, torch.float32), z0=dev(z0, torch.float32),
        square=square, normalize=normalize, delta=w.delta)
    torch.cuda.synchronize()
    names = NAMES + ("dS0", "dz0")
    dtq, dtk = np.zeros(x["theta_q"].shape), np.zeros(x["theta_k"].shape)
    for b in range(B):
        for h in range(H):
            want = O.gated_causal_bwd_state(x["Q"][b, h], x["K"][b, h], x["V"][b, h],
                                            x["theta_q"][h], x["theta_k"][h], lg[b, h], G[b, h],
                                            S0[b, h], z0[b, h], square=square,
                                            normalize=normalize, delta=w.delta)
            dtq[h] += want[3]
            dtk[h] += want[4]
            sel = (got[0][b, h], got[1][b, h], got[2][b, h], None, None, got[5][b, h],
                   got[6][b, h], got[7][b, h])
            for nm, a, r in zip(names, sel, want):
                if a is None:
                    continue
                err = rel_fro(host(a), r)
                assert err <= TOL_BF16, (b, h, nm, err)
    assert rel_fro(host(got[3]), dtq) <= TOL_BF16
    assert rel_fro(host(got[4]), dtk) <= TOL_BF16


def test_gated_bwd_state_without_state_is_gated_bwd(lib):
    """No initial state: the same numbers as llops_linattn_gated_causal_bwd bit for bit."""
    w = _w(1, 2, 300, 64, 64, 64, 4, True, True)
    x = generate(w)
    G = dout(w)
    lg = log_gates(w, mu=3.0)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    announce("gated_bwd_state without state")
    a = lib.llops_linattn_gated_causal_bwd_state(g["Q"], g["K"], g["V"], g["theta_q"],
                                                 g["theta_k"], dev(lg, torch.float32),
                                                 dev(G, torch.float32), square=True,
                                                 normalize=True, delta=w.delta)
    b = lib.llops_linattn_gated_causal_bwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"],
                                           dev(lg, torch.float32), dev(G, torch.float32),
                                           square=True, normalize=True, delta=w.delta)
    torch.cuda.synchronize()
    for x1, x2 in zip(a[:6], b):
        assert torch.equal(x1, x2)
