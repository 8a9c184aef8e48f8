"""Host-side checks of the Python binding: every shape, dtype or layout
mismatch between arguments raises before anything reaches the library.

The tensors here are host tensors. A call whose arguments pass every metadata
check stops at the device check instead ("must be a device tensor"), so each
case below asserts the message of its own mismatch: if that check were
missing, the call would fall through to the device check and the test would
fail. No GPU is needed and nothing is launched."""
import pytest

torch = pytest.importorskip("torch")

from learnable_polynomial_feature_amd import _lib as L  # noqa: E402

B, H, n, d, dv, m, p, t = 2, 3, 8, 16, 16, 32, 2, 2


def bf(*s):
    return torch.zeros(s, dtype=torch.bfloat16)


def f32(*s):
    return torch.zeros(s, dtype=torch.float32)


def attn_args(**over):
    a = dict(Q=bf(B, H, n, d), K=bf(B, H, n, d), V=bf(B, H, n, dv), theta_q=bf(H, p, t, d, m),
             theta_k=bf(H, p, t, d, m))
    a.update(over)
    return a


def dec_args(**over):
    a = dict(q=bf(B, H, d), k=bf(B, H, d), v=bf(B, H, dv), theta_q=bf(H, p, t, d, m),
             theta_k=bf(H, p, t, d, m), S=f32(B, H, m, dv), z=f32(B, H, m))
    a.update(over)
    return a


def raises(fn, match):
    with pytest.raises((ValueError, TypeError), match=match):
        fn()


def noncontig(*s):
    """A float32 tensor of shape s that is not contiguous."""
    return f32(*s[:-2], s[-1], s[-2]).transpose(-1, -2)


# ---- consistent arguments reach the device check --------------------------
def test_consistent_arguments_stop_at_the_device_check():
    raises(lambda: L.llops_featmap(bf(B, H, n, d), bf(H, p, t, d, m)), "device tensor")
    a = attn_args()
    raises(lambda: L.llops_linattn_fwd(*a.values()), "device tensor")
    raises(lambda: L.llops_linattn_causal_fwd(*a.values(), out=f32(B, H, n, dv)), "device tensor")
    raises(lambda: L.llops_linattn_causal_bwd(*a.values(), f32(B, H, n, dv)), "device tensor")
    dc = dec_args()
    raises(lambda: L.llops_decode_step(**dc), "device tensor")
    raises(lambda: L.llops_gated_decode_step(log_gate=f32(B, H), **dc), "device tensor")


# ---- feature map -------------------------------------------------------------
@pytest.mark.parametrize("kw,match", [
    # a bf16 buffer where fp32 phi is asked for: twice its bytes would be written
    (dict(out=bf(B, H, n, m)), "out must be torch.float32"),
    (dict(out=bf(B, H, n, m), out_dtype=torch.float32), "out must be torch.float32"),
    (dict(out=f32(B, H, n, m), out_dtype=torch.bfloat16), "out must be torch.bfloat16"),
    (dict(out=f32(B, H, n, m + 16)), "out must have shape"),
    (dict(out=noncontig(B, H, n, m)), "contiguous"),
    (dict(workspace=torch.zeros(64, 2, dtype=torch.uint8).t()), "workspace must be contiguous"),
    (dict(workspace=[0]), "workspace must be a torch.Tensor"),
    (dict(out_dtype=torch.float16), "out_dtype"),
])
def test_featmap_buffers(kw, match):
    raises(lambda: L.llops_featmap(bf(B, H, n, d), bf(H, p, t, d, m), **kw), match)


def test_featmap_inputs():
    raises(lambda: L.llops_featmap(bf(B, H, n, d), bf(H, p, t, d + 16, m)), "d and dtype")
    raises(lambda: L.llops_featmap(bf(B, H, n, d), f32(H, p, t, d, m)), "d and dtype")
    raises(lambda: L.llops_featmap(bf(B, H, n, d), bf(H + 1, p, t, d, m)), "heads")
    raises(lambda: L.llops_featmap(bf(H, n, d), bf(H, p, t, d, m)), "batch, heads, n, d")


def test_featmap_bwd_buffers():
    X, th = bf(B, H, n, d), bf(H, p, t, d, m)
    raises(lambda: L.llops_featmap_bwd(X, th, f32(B, H, n, m + 16)), "dphi must have shape")
    raises(lambda: L.llops_featmap_bwd(X, th, f32(B, H, n, m), dX=bf(B, H, n, d)),
           "dX must be torch.float32")
    raises(lambda: L.llops_featmap_bwd(X, th, f32(B, H, n, m), dtheta=f32(H, p, t, d, m + 16)),
           "dtheta must have shape")


# ---- attention -----------------------------------------------------------------
@pytest.mark.parametrize("over,match", [
    (dict(K=bf(B, H, n + 1, d)), "Q, K must be"),
    (dict(V=bf(B, H, n + 1, dv)), "Q, K must be"),
    (dict(theta_k=bf(H, p, t + 1, d, m)), "same shape"),
    (dict(theta_k=bf(p, t, d, m)), "same shape"),
    (dict(theta_q=bf(H, p, t, d + 16, m), theta_k=bf(H, p, t, d + 16, m)), "must match"),
    (dict(V=f32(B, H, n, dv)), "one dtype"),
    (dict(theta_k=f32(H, p, t, d, m)), "one dtype"),
])
def test_attention_inputs(over, match):
    a = attn_args(**over)
    raises(lambda: L.llops_linattn_fwd(*a.values()), match)
    raises(lambda: L.llops_linattn_causal_fwd(*a.values()), match)


@pytest.mark.parametrize("kw,match", [
    (dict(out=f32(B, H, n, dv + 16)), "out must have shape"),
    (dict(out=bf(B, H, n, dv)), "out must be torch.float32"),
    (dict(out=noncontig(B, H, n, dv)), "contiguous"),
    (dict(S0=f32(B, H, m, dv + 16)), "S0 must have shape"),
    (dict(z0=bf(B, H, m)), "z0 must be torch.float32"),
    (dict(S_final=bf(B, H, m, dv)), "S_final must be torch.float32"),
    (dict(z_final=f32(B, H, m + 16)), "z_final must have shape"),
    (dict(S_final=noncontig(B, H, m, dv)), "contiguous"),
    (dict(workspace=torch.zeros(64, 2, dtype=torch.uint8).t()), "workspace must be contiguous"),
])
def test_causal_buffers(kw, match):
    raises(lambda: L.llops_linattn_causal_fwd(*attn_args().values(), **kw), match)


def test_gated_and_backward_buffers():
    a = attn_args()
    raises(lambda: L.llops_linattn_gated_causal_fwd(*a.values(), f32(B, H, n + 1)),
           "log_gate must have shape")
    raises(lambda: L.llops_linattn_gated_causal_fwd(*a.values(), bf(B, H, n)),
           "log_gate must be torch.float32")
    raises(lambda: L.llops_linattn_causal_bwd(*a.values(), bf(B, H, n, dv)),
           "dO must be torch.float32")
    raises(lambda: L.llops_linattn_bwd(*a.values(), f32(B, H, n, dv + 16)), "dO must have shape")
    raises(lambda: L.llops_linattn_causal_bwd_state(*a.values(), f32(B, H, n, dv),
                                                    S0=f32(B, H, m + 16, dv)),
           "S0 must have shape")
    raises(lambda: L.llops_linattn_gated_causal_bwd(*a.values(), f32(B, H, n - 1),
                                                    f32(B, H, n, dv)),
           "log_gate must have shape")


# ---- decode --------------------------------------------------------------------
@pytest.mark.parametrize("over,match", [
    (dict(theta_k=bf(H, p, t + 1, d, m)), "same shape"),
    (dict(theta_k=bf(p, t, d, m)), "same shape"),
    (dict(theta_k=bf(H, p, t, d, m + 16)), "same shape"),
    (dict(theta_q=bf(H, p, t, d + 16, m), theta_k=bf(H, p, t, d + 16, m)), "must match"),
    (dict(v=f32(B, H, dv)), "one dtype"),
    (dict(theta_k=f32(H, p, t, d, m)), "one dtype"),
    (dict(k=bf(B, H, d + 16)), "q, k must be"),
    (dict(S=f32(B, H, m, dv + 16)), "S must have shape"),
    (dict(S=bf(B, H, m, dv)), "S must be torch.float32"),
    (dict(S=noncontig(B, H, m, dv)), "contiguous"),
    (dict(z=f32(B, H, m + 16)), "z must have shape"),
])
def test_decode_arguments(over, match):
    raises(lambda: L.llops_decode_step(**dec_args(**over)), match)


def test_decode_buffers():
    dc = dec_args()
    raises(lambda: L.llops_decode_step(**dc, out=bf(B, H, dv)), "out must be torch.float32")
    raises(lambda: L.llops_decode_step(**dc, out=f32(B, H, dv + 16)), "out must have shape")
    raises(lambda: L.llops_gated_decode_step(log_gate=f32(B, H, 1), **dc),
           "log_gate must have shape")
    raises(lambda: L.llops_gated_decode_step(log_gate=None, **dc), "log_gate is required")
