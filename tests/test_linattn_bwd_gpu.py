"""GPU parity of llops_linattn_bwd (gradients of sum(dO * out) for the
non-causal LLoPS attention) against the fp64 oracle's chain rule on seeded
inputs with ragged tails, plain and normalised, squared and not, t = 1 and 4,
shared Theta, n = 1, no rows, and at 1 x 32 x 65536 on sampled heads (the
factored oracle, pinned to the materialised one).

Normalised cases use the squared (non-negative) map for the reason the causal
backward's tests give: with signed features the denominator can pass through
zero, where neither the output nor its gradient is well conditioned. The
n = 1 case is plain: normalised, a lone token's output is its own value and
dphi_Q is a difference of two terms that cancel."""
import numpy as np
import pytest

from learnable_polynomial_feature_amd.workloads import WORKLOADS, Workload, dout, generate
from oracle import llops_oracle as O

from _util import TOL_BF16, announce, dev, host, rel_fro

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _w(B, H, n, d, dv, m, t, square, normalize, seed=0):
    return Workload("ncbwd", batch=B, heads=H, n=n, d=d, dv=dv, p=2, t=t, m=m, dtype="bf16",
                    causal=False, square=square, normalize=normalize, delta=1e-6, chunk=64,
                    seed=seed)


CASES = [
    # B, H, n, d, dv, m, t, square, normalize, shared
    (1, 2, 300, 64, 64, 64, 4, True, True, False),
    (2, 1, 257, 128, 128, 256, 4, True, True, False),
    (1, 2, 500, 128, 64, 128, 1, False, False, True),
    (2, 2, 100, 64, 32, 64, 1, True, False, False),
    (1, 1, 1, 128, 128, 256, 4, True, False, False),
    (1, 1, 2048, 128, 128, 256, 4, True, True, False),
    (1, 3, 1000, 64, 128, 128, 4, True, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_linattn_bwd(lib, case):
    B, H, n, d, dv, m, t, square, normalize, shared = case
    w = _w(B, H, n, d, dv, m, t, square, normalize)
    x = generate(w)
    if shared:
        x["theta_q"], x["theta_k"] = x["theta_q"][0], x["theta_k"][0]
    G = dout(w)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    announce(f"linattn_bwd {case}")
    got = lib.llops_linattn_bwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"],
                                dev(G, torch.float32), square=square, normalize=normalize,
                                delta=w.delta)
    torch.cuda.synchronize()
    want = O.linattn_bwd_bh(x["Q"], x["K"], x["V"], x["theta_q"], x["theta_k"], G,
                            square=square, normalize=normalize, delta=w.delta)
    for name, a, b in zip(("dQ", "dK", "dV", "dtheta_q", "dtheta_k"), got, want):
        err = rel_fro(host(a), b)
        assert err <= TOL_BF16, (name, err)


NARROW = [CASES[1], CASES[4], CASES[5]]


@pytest.mark.parametrize("case", NARROW, ids=[str(c) for c in NARROW])
def test_linattn_bwd_narrow_equals_padded(lib, case, monkeypatch):
    """As for the causal backward: the non-causal chain-rule passes on narrow
    operands agree bit for bit with the padded copies (LLOPS_BWD_PADDED=1)."""
    B, H, n, d, dv, m, t, square, normalize, shared = case
    w = _w(B, H, n, d, dv, m, t, square, normalize)
    x = generate(w)
    G = dev(dout(w), torch.float32)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    announce(f"linattn_bwd narrow vs padded {case}")

    def run():
        out = lib.llops_linattn_bwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"], G,
                                    square=square, normalize=normalize, delta=w.delta)
        torch.cuda.synchronize()
        return out
    narrow = run()
    monkeypatch.setenv("LLOPS_BWD_PADDED", "1")
    padded = run()
    for name, a, b in zip(("dQ", "dK", "dV", "dtheta_q", "dtheta_k"), narrow, padded):
        assert torch.equal(a, b), name


def test_linattn_bwd_no_rows(lib):
    w = _w(1, 2, 0, 64, 64, 64, 4, True, True)
    th = dev(generate(w.replace(n=1))["theta_q"], torch.bfloat16)
    Q = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    V = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    G = torch.empty((1, 2, 0, 64), dtype=torch.float32, device="cuda")
    announce("linattn_bwd n=0")
    dQ, dK, dV, dtq, dtk = lib.llops_linattn_bwd(Q, Q, V, th, th, G, square=True, normalize=True,
                                                 delta=1e-6)
    torch.cuda.synchronize()
    assert dQ.numel() == 0 and dV.numel() == 0
    assert torch.count_nonzero(dtq).item() == 0 and torch.count_nonzero(dtk).item() == 0


@pytest.mark.slow
def test_linattn_bwd_full_size_sampled(lib):
    """1 x 32 x 65536 non-causal (d=dv=128, m=256, p=2, t=4, squared,
    normalised): all heads on the GPU; heads 0 and 31 against the factored
    fp64 oracle."""
    w = WORKLOADS["causal_long_n65536"].replace(causal=False)
    x = generate(w)
    G = dout(w)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    announce("linattn_bwd full size")
    dQ, dK, dV, dtq, dtk = lib.llops_linattn_bwd(
        g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"], dev(G, torch.float32),
        square=w.square, normalize=w.normalize, delta=w.delta)
    torch.cuda.synchronize()
    for h in (0, 31):
        q, k, v, tq, tk = x["Q"][0, h], x["K"][0, h], x["V"][0, h], x["theta_q"][h], x["theta_k"][h]
        Pq, Pk = O.featmap(q, tq, w.square), O.featmap(k, tk, w.square)
        dPq, dPk, rdV = O.attn_bwd_factored(Pq, Pk, v, G[0, h], normalize=w.normalize,
                                            delta=w.delta)
        rdQ, rtq = O.featmap_bwd(q, tq, dPq, w.square)
        rdK, rtk = O.featmap_bwd(k, tk, dPk, w.square)
        for name, a, b in (("dQ", dQ[0, h], rdQ), ("dK", dK[0, h], rdK), ("dV", dV[0, h], rdV),
                           ("dtheta_q", dtq[h], rtq), ("dtheta_k", dtk[h], rtk)):
            err = rel_fro(host(a), b)
            assert err <= TOL_BF16, (h, name, err)
