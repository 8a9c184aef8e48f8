"""llops_decode_step_noalloc (scratch in the library's static per-GPU buffer,
no workspace) against llops_decode_step (caller workspace) through the C ABI:
the same kernels on the same inputs, so outputs and updated states must agree
bit for bit. Two calls in a row, the second with a smaller batch and fewer
heads, so the second reads a buffer the first left full of its own values."""
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

D, DV, M, P, T = 128, 128, 256, 2, 4


def _inputs(B, H, seed, d=D, dv=DV, m=M, p=P, t=T):
    g = torch.Generator(device="cpu").manual_seed(seed)
    bf = lambda *s, scale=1.0: (torch.randn(*s, generator=g) * scale).to(torch.bfloat16).cuda()
    q, k, v = bf(B, H, d), bf(B, H, d), bf(B, H, dv)
    thq, thk = bf(H, p, t, d, m, scale=d ** -0.5), bf(H, p, t, d, m, scale=d ** -0.5)
    S = torch.randn(B, H, m, dv, generator=g).cuda()
    z = (torch.rand(B, H, m, generator=g) * 4 + 1).cuda()  # positive: denominators away from 0
    return q, k, v, thq, thk, S, z


def _both(lib, B, H, seed):
    q, k, v, thq, thk, S, z = _inputs(B, H, seed)
    kw = dict(square=True, normalize=True, delta=1e-6)
    S1, z1, S2, z2 = S.clone(), z.clone(), S.clone(), z.clone()
    print(f"[gpu-case] decode_step_noalloc B={B} H={H}", flush=True)
    want = lib.llops_decode_step(q, k, v, thq, thk, S1, z1, **kw)
    got = lib.llops_decode_step_noalloc(q, k, v, thq, thk, S2, z2, **kw)
    torch.cuda.synchronize()
    return (want, S1, z1), (got, S2, z2)


def test_noalloc_decode_equals_workspace_decode_twice(lib):
    for B, H, seed in ((128, 32, 1), (16, 8, 2)):
        (want, S1, z1), (got, S2, z2) = _both(lib, B, H, seed)
        assert torch.isfinite(want).all()
        assert torch.equal(got, want), (B, H, (got - want).abs().max().item())
        assert torch.equal(S2, S1), (B, H)
        assert torch.equal(z2, z1), (B, H)


def test_noalloc_decode_rejects_oversized_scratch(lib):
    """512 x 8 slices at m = 1024 need 32 MiB of phi scratch: refused before
    any launch, and the state is left as it was."""
    B, H = 512, 8
    q, k, v, thq, thk, S, z = _inputs(B, H, 3, d=16, dv=4, m=1024, p=2, t=1)
    S0 = S.clone()
    with pytest.raises(lib.LlopsError) as e:
        lib.llops_decode_step_noalloc(q, k, v, thq, thk, S, z, square=True, normalize=True,
                                      delta=1e-6)
    assert e.value.status == 2 and "static" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
