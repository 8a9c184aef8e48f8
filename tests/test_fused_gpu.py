"""The causal forward with phi_Q projected inside the output pass
(LLOPS_FUSED_Q=1) against the default two-kernel path (feature maps of Q and
K through HBM, then the segment passes) and against the oracle.

The fused pass runs the feature map's products and epilogue in the feature
map kernel's order and the read-out in the output pass's order, so the two
paths must agree bit for bit: outputs and final states, across ragged
sequence ends, segments whose chunk count is odd, several segments per
sequence, an initial state, shared Theta and both fused shapes (m, dv, d,
p, t) = (256, 128, 128, 2, 4) and (128, 64, 64, 3, 8)."""
import numpy as np
import pytest

from learnable_polynomial_feature_amd.workloads import Workload, generate
from oracle import llops_oracle as O

from _util import TOL_BF16, TOL_ROW_BF16, announce, dev, host, rel_fro, row_rel_max

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    # B, H, n, d, dv, m, p, t, square, normalize, shared, state
    (1, 2, 1500, 128, 128, 256, 2, 4, True, True, False, False),
    (2, 3, 1100, 128, 128, 256, 2, 4, True, True, False, True),
    (1, 1, 5000, 128, 128, 256, 2, 4, True, True, True, False),
    (3, 1, 1057, 128, 128, 256, 2, 4, False, False, False, False),
    (1, 2, 4097, 128, 128, 256, 2, 4, True, False, False, True),
    (2, 2, 2500, 64, 64, 128, 3, 8, True, True, False, False),
    (1, 3, 3001, 64, 64, 128, 3, 8, True, True, True, True),
]


def _run(lib, g, c, S0, z0):
    B, H, n, d, dv, m, p, t, square, normalize, shared, state = c
    return lib.llops_linattn_causal_fwd(g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"],
                                        square=square, normalize=normalize, delta=1e-6,
                                        chunk=64, S0=S0, z0=z0, return_state=True)


def _inputs(c, seed=0):
    B, H, n, d, dv, m, p, t, square, normalize, shared, state = c
    w = Workload("fused", batch=B, heads=H, n=n, d=d, dv=dv, p=p, t=t, m=m, dtype="bf16",
                 causal=True, square=square, normalize=normalize, delta=1e-6, chunk=64,
                 seed=seed)
    x = generate(w)
    if shared:
        x["theta_q"], x["theta_k"] = x["theta_q"][0], x["theta_k"][0]
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    S0 = z0 = None
    if state:  # a positive prefix state, as a previous call would leave it
        rng = np.random.default_rng(5)
        S0 = torch.from_numpy(rng.standard_normal((B, H, m, dv)).astype(np.float32)).cuda()
        z0 = torch.from_numpy((rng.random((B, H, m)) * 8 + 1).astype(np.float32)).cuda()
    return x, g, S0, z0


@pytest.mark.parametrize("c", CASES, ids=[str(c) for c in CASES])
def test_fused_equals_two_kernel_path(lib, c, monkeypatch):
    x, g, S0, z0 = _inputs(c)
    announce(f"two-kernel causal {c}")
    monkeypatch.delenv("LLOPS_FUSED_Q", raising=False)
    plain = _run(lib, g, c, S0, z0)
    torch.cuda.synchronize()
    monkeypatch.setenv("LLOPS_FUSED_Q", "1")
    announce(f"fused causal {c}")
    fused = _run(lib, g, c, S0, z0)
    torch.cuda.synchronize()
    for a, b, name in zip(fused, plain, ("out", "S_final", "z_final")):
        assert torch.isfinite(a).all(), name
        assert torch.equal(a, b), (name, (a - b).abs().max().item())


@pytest.mark.parametrize("c", [CASES[1], CASES[5]], ids=["m256_state", "p3_m128"])
def test_fused_against_oracle(lib, c, monkeypatch):
    B, H, n, d, dv, m, p, t, square, normalize, shared, state = c
    monkeypatch.setenv("LLOPS_FUSED_Q", "1")
    x, g, S0, z0 = _inputs(c, seed=3)
    announce(f"fused causal vs oracle {c}")
    out, S, z = _run(lib, g, c, S0, z0)
    torch.cuda.synchronize()
    kw = dict(square=square, normalize=normalize, delta=1e-6)
    ro, rS, rz = O.causal_bh(x["Q"], x["K"], x["V"], x["theta_q"], x["theta_k"], chunk=64,
                             S0=None if S0 is None else host(S0),
                             z0=None if z0 is None else host(z0), **kw)
    assert rel_fro(host(out), ro) <= TOL_BF16
    assert row_rel_max(host(out), ro) <= TOL_ROW_BF16, row_rel_max(host(out), ro)
    assert rel_fro(host(S), rS) <= TOL_BF16
    assert rel_fro(host(z), rz) <= TOL_BF16


def test_fused_long_workload(lib, monkeypatch):
    """The long workload (1 x 32 x 65536, d = dv = 128, m = 256, p = 2, t = 4,
    squared, normalised) on the fused path: equal to the two-kernel path on
    the whole output and final state, and four heads against the oracle."""
    from learnable_polynomial_feature_amd.workloads import WORKLOADS
    w = WORKLOADS["causal_long_n65536"]
    x = generate(w)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    del x
    kw = dict(square=w.square, normalize=w.normalize, delta=w.delta, chunk=w.chunk,
              return_state=True)
    args = (g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"])
    announce("long workload, two-kernel path")
    monkeypatch.delenv("LLOPS_FUSED_Q", raising=False)
    plain = lib.llops_linattn_causal_fwd(*args, **kw)
    torch.cuda.synchronize()
    monkeypatch.setenv("LLOPS_FUSED_Q", "1")
    announce("long workload, fused path")
    fused = lib.llops_linattn_causal_fwd(*args, **kw)
    torch.cuda.synchronize()
    for a, b, name in zip(fused, plain, ("out", "S_final", "z_final")):
        assert torch.equal(a, b), name
    del plain, g
    out, S, z = fused
    for h in (0, 9, 22, 31):
        xs = generate(w, heads=[h])
        ro, rS, rz = O.causal_chunked(xs["Q"][0, 0], xs["K"][0, 0], xs["V"][0, 0],
                                      xs["theta_q"][0], xs["theta_k"][0], square=w.square,
                                      normalize=w.normalize, delta=w.delta, chunk=w.chunk)
        o = host(out[0, h])
        assert rel_fro(o, ro) <= TOL_BF16, h
        assert row_rel_max(o, ro) <= TOL_ROW_BF16, h
        assert rel_fro(host(S[0, h]), rS) <= TOL_BF16, h
        assert rel_fro(host(z[0, h]), rz) <= TOL_BF16, h
