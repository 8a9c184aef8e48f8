"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph on a side
stream, the library launching on the capturing stream) against the same
steps run eagerly: three replays, each from a restored state with eager work
and synchronisations in between, must equal the eager results bit for bit
(same kernels, same order, deterministic reductions)."""
import numpy as np
import pytest

from learnable_polynomial_feature_amd.workloads import Workload, generate

from _util import announce, dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("gated", [False, True])
def test_decode_graph_replays_equal_eager(lib, gated):
    B, H, d, dv, m, steps = 16, 4, 128, 128, 256, 5
    w = Workload("graph", batch=B, heads=H, n=steps, d=d, dv=dv, p=2, t=4, m=m, dtype="bf16",
                 causal=True, square=True, normalize=True, delta=1e-6, chunk=64)
    x = generate(w)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    rng = np.random.default_rng(4)
    S0 = torch.from_numpy((0.05 * rng.standard_normal((B, H, m, dv))).astype(np.float32)).cuda()
    z0 = torch.from_numpy(np.abs(0.05 * rng.standard_normal((B, H, m))).astype(np.float32)).cuda()
    lg = torch.from_numpy(np.log(rng.uniform(0.5, 1.0, (steps, B, H))).astype(np.float32)).cuda()
    kw = dict(square=True, normalize=True, delta=1e-6)
    outs = torch.zeros((steps, B, H, dv), dtype=torch.float32, device="cuda")

    def run(S, z):
        for s in range(steps):
            if gated:
                lib.llops_gated_decode_step(g["Q"][:, :, s], g["K"][:, :, s], g["V"][:, :, s],
                                            g["theta_q"], g["theta_k"], lg[s], S, z, out=outs[s],
                                            **kw)
            else:
                lib.llops_decode_step(g["Q"][:, :, s], g["K"][:, :, s], g["V"][:, :, s],
                                      g["theta_q"], g["theta_k"], S, z, out=outs[s], **kw)

    announce(f"decode graph vs eager, gated={gated}")
    S, z = S0.clone(), z0.clone()
    run(S, z)
    torch.cuda.synchronize()
    want = (outs.clone(), S.clone(), z.clone())
    S.copy_(S0)
    z.copy_(z0)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        run(S, z)
    torch.cuda.synchronize()
    for rep in range(3):
        S.copy_(S0)
        z.copy_(z0)
        outs.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, want[0]), rep
        assert torch.equal(S, want[1]) and torch.equal(z, want[2]), rep
        _ = (S * 2).sum().item()  # eager work between replays


@pytest.mark.parametrize("fused", [False, True])
def test_causal_graph_replays_equal_eager(lib, fused, monkeypatch):
    """A whole causal forward call (feature maps, segment passes, scan, output
    pass) captured once and replayed three times, with eager work between the
    replays, equals the eager call bit for bit; on the two-kernel path and on
    the fused output pass."""
    if fused:
        monkeypatch.setenv("LLOPS_FUSED_Q", "1")
    else:
        monkeypatch.delenv("LLOPS_FUSED_Q", raising=False)
    w = Workload("graph_causal", batch=1, heads=4, n=3000, d=128, dv=128, p=2, t=4, m=256,
                 dtype="bf16", causal=True, square=True, normalize=True, delta=1e-6, chunk=64)
    x = generate(w)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    kw = dict(square=True, normalize=True, delta=1e-6, chunk=64)
    shape = lib.make_shape(batch=1, heads=4, n=3000, d=128, dv=128, m=256, p=2, t=4, square=1,
                           normalize=1, delta=1e-6, chunk=64)
    ws = torch.empty(lib.llops_workspace_bytes(shape, lib.ENTRY_CAUSAL), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((1, 4, 3000, 128), dtype=torch.float32, device="cuda")
    Sf = torch.empty((1, 4, 256, 128), dtype=torch.float32, device="cuda")
    zf = torch.empty((1, 4, 256), dtype=torch.float32, device="cuda")
    args = (g["Q"], g["K"], g["V"], g["theta_q"], g["theta_k"])

    def call():
        lib.llops_linattn_causal_fwd(*args, out=out, S_final=Sf, z_final=zf, workspace=ws, **kw)

    announce(f"causal graph vs eager, fused={fused}")
    call()
    torch.cuda.synchronize()
    want = (out.clone(), Sf.clone(), zf.clone())
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        Sf.zero_()
        zf.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want[0]), rep
        assert torch.equal(Sf, want[1]) and torch.equal(zf, want[2]), rep
        _ = (out * 2).sum().item()  # eager work between replays
