"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, the ctypes struct matches llops_shape_t, and invalid calls
return their documented status before any launch (no GPU needed: these calls
fail validation, so no device pointer is ever touched)."""
import ctypes
import os
import re
import subprocess

import pytest

from learnable_polynomial_feature_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llops.h")

FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10008)


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# Calls below pass placeholder pointers that only validation ever sees. They
# never run where a GPU is visible, so a validation gap cannot turn into a
# launch on a real device.
fake_ptr = pytest.mark.skipif(_gpu_visible(), reason="placeholder pointers: host-only test")


@pytest.fixture(scope="module")
def L():
    return _lib.library()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(llops_\w+)\s*\(", src,
                                 flags=re.M)))


def test_header_functions_are_exported(L):
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (llops_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def test_shape_struct_layout_matches_header(tmp_path):
    """Compile a tiny C program against include/llops.h and compare
    sizeof/offsetof with the ctypes mirror."""
    fields = [f for f, _ in _lib.Shape._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", '#include "llops.h"', "int main(){",
            'printf("%zu\\n", sizeof(llops_shape_t));']
    prog += [f'printf("%zu\\n", offsetof(llops_shape_t, {f}));' for f in fields]
    prog += ["return 0;}"]
    c = str(tmp_path / "llops_layout_check.c")
    exe = str(tmp_path / "llops_layout_check")
    with open(c, "w") as f:
        f.write("\n".join(prog))
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", c, "-o", exe], check=True)
    vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(_lib.Shape)
    for f, off in zip(fields, vals[1:]):
        assert getattr(_lib.Shape, f).offset == off, f


def _shape(**kw):
    """llops_shape_t built field by field (no coercion of out-of-range values)."""
    base = dict(batch=2, heads=3, n=100, d=64, dv=64, m=64, p=2, t=2, square=1, normalize=1,
                delta=1e-6, chunk=64, theta_per_head=1, in_dtype=_lib.BF16, out_dtype=_lib.F32)
    base.update(kw)
    s = _lib.Shape()
    for k, v in base.items():
        setattr(s, k, v)
    return s


def _err(L):
    return L.llops_last_error().decode()


def test_status_strings(L):
    for code, name in _lib.STATUS.items():
        assert L.llops_status_str(code).decode() == name


@pytest.mark.parametrize("bad,code", [
    (dict(p=0), 1), (dict(t=0), 1), (dict(d=0), 1), (dict(m=0), 1), (dict(n=-1), 1),
    (dict(batch=-1), 1), (dict(in_dtype=7), 1), (dict(out_dtype=2), 1), (dict(square=2), 1),
    (dict(chunk=48), 1), (dict(p=9), 2), (dict(t=65), 2), (dict(d=512), 2), (dict(m=2048), 2),
    (dict(d=40), 2), (dict(m=24), 2),
])
@fake_ptr
def test_featmap_validation(L, bad, code):
    s = _shape(**bad)
    st = L.llops_featmap(ctypes.byref(s), FAKE, FAKE, FAKE, None, 0, None)
    assert st == code, _err(L)


@fake_ptr
def test_featmap_null_and_alignment(L):
    s = _shape()
    assert L.llops_featmap(None, FAKE, FAKE, FAKE, None, 0, None) == 1
    assert L.llops_featmap(ctypes.byref(s), None, FAKE, FAKE, None, 0, None) == 1
    assert "X is null" in _err(L)
    assert L.llops_featmap(ctypes.byref(s), FAKE, MISALIGNED, FAKE, None, 0, None) == 1
    assert "aligned" in _err(L)
    # fp32 inputs cannot produce a bf16 phi
    s = _shape(in_dtype=_lib.F32, out_dtype=_lib.BF16)
    assert L.llops_featmap(ctypes.byref(s), FAKE, FAKE, FAKE, None, 0, None) == 2


@fake_ptr
def test_featmap_workspace(L):
    """Shapes with an unrolled bf16 kernel need scratch for the repacked
    Theta (heads * p * t * d * m bf16); the rest need none."""
    s = _shape(batch=1, heads=4, n=4096, d=128, m=256, p=2, t=4)
    need = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_FEATMAP)
    assert need == 4 * 2 * 4 * 128 * 256 * 2
    assert L.llops_featmap(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, need - 1, None) == 3
    assert "workspace" in _err(L)
    assert L.llops_featmap(ctypes.byref(s), FAKE, FAKE, FAKE, None, need, None) == 1
    shared = _shape(batch=1, heads=4, n=4096, d=128, m=256, p=2, t=4, theta_per_head=0)
    assert L.llops_workspace_bytes(ctypes.byref(shared), _lib.ENTRY_FEATMAP) == need // 4
    # up to 1024 rows per head the unrolled shapes read Theta in place (no
    # repacked copy); f32 inputs and shapes without an unrolled kernel need none
    few = _shape(batch=1, heads=4, n=1024, d=128, m=256, p=2, t=4)
    assert L.llops_workspace_bytes(ctypes.byref(few), _lib.ENTRY_FEATMAP) == 0
    more = _shape(batch=1, heads=4, n=1025, d=128, m=256, p=2, t=4)
    assert L.llops_workspace_bytes(ctypes.byref(more), _lib.ENTRY_FEATMAP) == need
    for other in (_shape(in_dtype=_lib.F32), _shape(n=4096, d=96, m=64)):
        assert L.llops_workspace_bytes(ctypes.byref(other), _lib.ENTRY_FEATMAP) == 0
    # the attention entry points hold two repacked copies (Theta_q and Theta_k)
    a = _shape(batch=1, heads=4, n=4096, d=128, dv=128, m=256, p=2, t=4)
    big = L.llops_workspace_bytes(ctypes.byref(a), _lib.ENTRY_CAUSAL)
    assert big >= 2 * need


@pytest.mark.parametrize("bad,code", [
    (dict(delta=-1.0), 1), (dict(delta=float("nan")), 1), (dict(delta=float("inf")), 1),
    (dict(dv=0), 1), (dict(out_dtype=_lib.BF16), 2), (dict(m=48), 2), (dict(m=512), 2),
    (dict(dv=256), 2), (dict(dv=24), 2),
])
@fake_ptr
def test_attention_validation(L, bad, code):
    s = _shape(**bad)
    ws = L.llops_workspace_bytes(ctypes.byref(_shape()), _lib.ENTRY_CAUSAL)
    st = L.llops_linattn_causal_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                    FAKE, None, None, FAKE, ws, None)
    assert st == code, _err(L)
    st = L.llops_linattn_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
    assert st == code, _err(L)


@fake_ptr
def test_delta_ignored_without_normaliser(L):
    s = _shape(normalize=0, delta=-1.0)
    ws = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_CAUSAL)
    # passes validation, then fails on the too-small workspace (no launch)
    st = L.llops_linattn_causal_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                    FAKE, None, None, FAKE, ws - 1, None)
    assert st == 3, _err(L)


@fake_ptr
def test_workspace_checks(L):
    s = _shape()
    for entry, call in ((_lib.ENTRY_CAUSAL, "causal"), (_lib.ENTRY_LINATTN, "lin"),
                        (_lib.ENTRY_DECODE, "dec")):
        need = L.llops_workspace_bytes(ctypes.byref(s), entry)
        assert need > 0
        if call == "causal":
            st = L.llops_linattn_causal_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                            None, FAKE, None, None, FAKE, need - 1, None)
        elif call == "lin":
            st = L.llops_linattn_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     need - 1, None)
        else:
            st = L.llops_decode_step(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, need - 1, None)
        assert st == 3, _err(L)
        assert "workspace" in _err(L)
    # a workspace is required when its size is non-zero
    need = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_CAUSAL)
    st = L.llops_linattn_causal_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                    FAKE, None, None, None, need, None)
    assert st == 1
    assert L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_FEATMAP) == 0
    assert L.llops_workspace_bytes(ctypes.byref(s), 10) == 0
    assert L.llops_workspace_bytes(ctypes.byref(_shape(p=0)), _lib.ENTRY_CAUSAL) == 0


def test_workspace_sizes_follow_layout(L):
    """bf16 phi_Q and phi_K plus fp32 per-segment states, 256-byte aligned."""
    s = _lib.make_shape(batch=1, heads=32, n=65536, d=128, dv=128, m=256, p=2, t=4, square=1,
                        normalize=1, delta=1e-6, chunk=128)
    need = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_CAUSAL)
    phi = 32 * 65536 * 256 * 2
    per = 256 * 128 + 256
    assert need >= 2 * phi + 32 * per * 4
    assert need <= 2 * phi + 32 * 64 * per * 4 + 1024
    s32 = _lib.make_shape(batch=1, heads=1, n=256, d=16, dv=16, m=32, p=2, t=2,
                          in_dtype=_lib.F32)
    need32 = L.llops_workspace_bytes(ctypes.byref(s32), _lib.ENTRY_LINATTN)
    assert need32 >= 2 * 256 * 32 * 4
    dec = _lib.make_shape(batch=128, heads=32, n=1, d=128, dv=128, m=256, p=2, t=4)
    # phi_q and phi_k in fp32 (128 rows per head: Theta is read in place)
    assert L.llops_workspace_bytes(ctypes.byref(dec), _lib.ENTRY_DECODE) == 2 * 128 * 32 * 256 * 4


@fake_ptr
def test_decode_requires_state(L):
    s = _shape()
    need = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_DECODE)
    st = L.llops_decode_step(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                             FAKE, need, None)
    assert st == 1 and "S is null" in _err(L)


def test_binding_refuses_host_tensors():
    import torch
    X = torch.zeros(1, 1, 4, 16, dtype=torch.bfloat16)
    th = torch.zeros(1, 1, 16, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        _lib.llops_featmap(X, th)


def test_missing_library_raises(tmp_path):
    import importlib
    mod = importlib.import_module("learnable_polynomial_feature_amd._lib")
    saved = mod._LIB
    try:
        mod._LIB = None
        with pytest.raises(_lib.LlopsError, match="not found"):
            mod.library(str(tmp_path / "nope.so"))
    finally:
        mod._LIB = saved


def _bwd_shape(**kw):
    base = dict(batch=2, heads=3, n=100, d=64, m=64, p=2, t=4, square=1)
    base.update(kw)
    return _shape(**base)


@pytest.mark.parametrize("bad,code", [
    (dict(p=0), 1), (dict(m=0), 1), (dict(in_dtype=7), 1), (dict(square=2), 1), (dict(n=-1), 1),
    (dict(t=2), 2), (dict(p=3), 2), (dict(p=1), 2), (dict(d=96), 2), (dict(m=48), 2),
    (dict(in_dtype=_lib.F32), 2), (dict(p=9), 2),
])
@fake_ptr
def test_featmap_bwd_validation(L, bad, code):
    s = _bwd_shape(**bad)
    st = L.llops_featmap_bwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == code, _err(L)


@fake_ptr
def test_featmap_bwd_pointers_and_workspace(L):
    s = _bwd_shape(batch=1, heads=4, n=4096, d=128, m=256, t=4)
    need = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_FEATMAP_BWD)
    slot = 4 * 2 * 4 * 256 * 128 * 4  # one fp32 partial dTheta for every head
    ds = 1 * 4 * 4096 * 256 * 2  # t > 1 and squared: ds of every row in bf16 (whole 256-row tiles)
    pack = 2 * 4 * 128 * 256 * 2  # one head's Theta in bf16, in fragment order
    assert need > ds and (need - ds - 4 * pack) % slot == 0
    plain = _bwd_shape(batch=1, heads=4, n=4096, d=128, m=256, t=4, square=0)
    assert L.llops_workspace_bytes(ctypes.byref(plain), _lib.ENTRY_FEATMAP_BWD) == need - ds
    shared = _bwd_shape(batch=1, heads=4, n=4096, d=128, m=256, t=4, theta_per_head=0)
    assert L.llops_workspace_bytes(ctypes.byref(shared), _lib.ENTRY_FEATMAP_BWD) == need - 3 * pack
    ragged = _bwd_shape(batch=1, heads=4, n=4000, d=128, m=256, t=4)  # ds rounds up to 4096 rows
    assert L.llops_workspace_bytes(ctypes.byref(ragged), _lib.ENTRY_FEATMAP_BWD) - ds == \
        L.llops_workspace_bytes(ctypes.byref(_bwd_shape(batch=1, heads=4, n=4000, d=128, m=256,
                                                        t=4, square=0)), _lib.ENTRY_FEATMAP_BWD)
    args = [FAKE] * 5
    assert L.llops_featmap_bwd(ctypes.byref(s), *args, FAKE, need - 1, None) == 3
    assert "workspace" in _err(L)
    assert L.llops_featmap_bwd(ctypes.byref(s), *args, None, need, None) == 1
    for i, name in enumerate(("X", "theta", "dphi", "dX", "dtheta")):
        a = list(args)
        a[i] = None
        assert L.llops_featmap_bwd(ctypes.byref(s), *a, FAKE, need, None) == 1
        assert f"{name} is null" in _err(L)
        a[i] = MISALIGNED
        assert L.llops_featmap_bwd(ctypes.byref(s), *a, FAKE, need, None) == 1
        assert "aligned" in _err(L)
    # no rows: X, dphi and dX may be null (dtheta is still written, as zeros)
    empty = _bwd_shape(batch=1, heads=4, n=0, d=128, m=256, t=4)
    assert L.llops_workspace_bytes(ctypes.byref(empty), _lib.ENTRY_FEATMAP_BWD) == 0
    assert L.llops_featmap_bwd(ctypes.byref(empty), None, FAKE, None, None, None, None, 0,
                               None) == 1
    assert "dtheta is null" in _err(L)
    # t = 1 keeps one partial per wave and chunk
    t1 = _bwd_shape(batch=1, heads=4, n=4096, d=128, m=256, t=1)
    need1 = L.llops_workspace_bytes(ctypes.byref(t1), _lib.ENTRY_FEATMAP_BWD)
    pack1 = 2 * 1 * 128 * 256 * 2
    assert need1 > 0 and (need1 - 4 * pack1) % (4 * 4 * 2 * 1 * 256 * 128 * 4) == 0


def _cbwd_shape(**kw):
    base = dict(batch=1, heads=2, n=300, d=64, dv=64, m=64, p=2, t=4, square=1, normalize=1)
    base.update(kw)
    return _shape(**base)


@pytest.mark.parametrize("bad,code", [
    (dict(p=0), 1), (dict(dv=0), 1), (dict(delta=-1.0), 1), (dict(n=-1), 1),
    (dict(in_dtype=_lib.F32), 2), (dict(t=2), 2), (dict(p=3), 2), (dict(m=96), 2),
    (dict(m=192), 2), (dict(d=96), 2), (dict(dv=144), 2), (dict(out_dtype=_lib.BF16), 2),
])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@fake_ptr
def test_attn_bwd_validation(L, bad, code, causal):
    s = _cbwd_shape(**bad)
    fn, entry = _attn_bwd_entry(L, causal)
    st = fn(ctypes.byref(s), *([FAKE] * 11), FAKE, 1 << 40, None)
    assert st == code, _err(L)
    assert L.llops_workspace_bytes(ctypes.byref(s), entry) == 0


def _attn_bwd_entry(L, causal):
    if causal:
        return L.llops_linattn_causal_bwd, _lib.ENTRY_CAUSAL_BWD
    return L.llops_linattn_bwd, _lib.ENTRY_LINATTN_BWD


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@fake_ptr
def test_attn_bwd_pointers_and_workspace(L, causal):
    fn, entry = _attn_bwd_entry(L, causal)
    s = _cbwd_shape(batch=2, heads=3, n=1000, d=128, dv=128, m=256)
    need = L.llops_workspace_bytes(ctypes.byref(s), entry)
    R = 2 * 3 * 1000
    # at least: phi_Q, phi_K (bf16), fp32 num and M 1, a and b (the causal
    # pass also keeps reversed copies of a, b, phi_Q and phi_K)
    floor = R * 256 * (2 + 2) + R * (128 + 16) * 4 + 2 * R * 192 * 2
    if causal:
        floor += 2 * R * 192 * 2 + 2 * R * 256 * 2
    assert need >= floor
    plain = _cbwd_shape(batch=2, heads=3, n=1000, d=128, dv=128, m=256, normalize=0)
    assert L.llops_workspace_bytes(ctypes.byref(plain), entry) < need
    args = [FAKE] * 11
    assert fn(ctypes.byref(s), *args, FAKE, need - 1, None) == 3
    names = ("Q", "K", "V", "theta_q", "theta_k", "dO", "dQ", "dK", "dV", "dtheta_q", "dtheta_k")
    for i, name in enumerate(names):
        a = list(args)
        a[i] = None
        assert fn(ctypes.byref(s), *a, FAKE, need, None) == 1
        assert f"{name} is null" in _err(L)


@fake_ptr
def test_noncausal_bwd_workspace_below_causal(L):
    s = _cbwd_shape(batch=2, heads=3, n=1000, d=128, dv=128, m=256)
    c = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_CAUSAL_BWD)
    nc = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_LINATTN_BWD)
    assert 0 < nc < c


# ---- gated causal attention and gated decode -------------------------------

@pytest.mark.parametrize("bad,code", [
    (dict(m=96), 2), (dict(dv=32), 2), (dict(m=256, dv=64), 2),
    (dict(delta=-1.0), 1), (dict(dv=0), 1), (dict(m=512), 2),
])
@fake_ptr
def test_gated_validation(L, bad, code):
    """bf16 gated attention runs on the (m, dv) in {(256,128), (128,64),
    (64,64)} kernels; anything else is refused before any launch."""
    s = _shape(**bad)
    ws = L.llops_workspace_bytes(ctypes.byref(_shape()), _lib.ENTRY_GATED_CAUSAL)
    assert ws > 0
    assert L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_GATED_CAUSAL) == 0
    st = L.llops_linattn_gated_causal_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          None, None, FAKE, None, None, FAKE, ws, None)
    assert st == code, _err(L)


@fake_ptr
def test_gated_pointers_and_workspace(L):
    s = _shape()
    need = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_GATED_CAUSAL)
    # the gate is required, 4-byte aligned; a 16-byte-misaligned gate is fine
    st = L.llops_linattn_gated_causal_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                          None, None, FAKE, None, None, FAKE, need, None)
    assert st == 1 and "log_gate is null" in _err(L)
    st = L.llops_linattn_gated_causal_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE,
                                          ctypes.c_void_p(0x10002), None, None, FAKE, None, None,
                                          FAKE, need, None)
    assert st == 1 and "log_gate" in _err(L)
    st = L.llops_linattn_gated_causal_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE,
                                          ctypes.c_void_p(0x10004), None, None, FAKE, None, None,
                                          FAKE, need - 1, None)
    assert st == 3 and "workspace" in _err(L)
    st = L.llops_linattn_gated_causal_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          MISALIGNED, None, FAKE, None, None, FAKE, need, None)
    assert st == 1 and "S0" in _err(L)


@fake_ptr
def test_gated_f32_any_shape(L):
    """fp32 inputs take the fp32 gated kernels for shapes the bf16 kernels
    refuse; a short workspace still stops the call before any launch."""
    s = _shape(in_dtype=_lib.F32, m=96, dv=24, d=20)
    need = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_GATED_CAUSAL)
    assert need > 0
    st = L.llops_linattn_gated_causal_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          None, None, FAKE, None, None, FAKE, need - 1, None)
    assert st == 3, _err(L)


def test_gated_workspace_layout(L):
    """The gated workspace is the causal one plus the chunk-local gate sums
    (rows padded to 32 tokens) and one fp32 gate sum per segment."""
    s = _lib.make_shape(batch=1, heads=32, n=65536, d=128, dv=128, m=256, p=2, t=4, square=1,
                        normalize=1, delta=1e-6, chunk=128)
    base = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_CAUSAL)
    gated = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_GATED_CAUSAL)
    assert base + 32 * 65536 * 4 <= gated <= base + 32 * 65536 * 4 + 32 * 512 * 4 + 512
    r = _lib.make_shape(batch=2, heads=3, n=33, d=64, dv=64, m=64, p=2, t=2)
    gr = L.llops_workspace_bytes(ctypes.byref(r), _lib.ENTRY_GATED_CAUSAL)
    assert gr >= L.llops_workspace_bytes(ctypes.byref(r), _lib.ENTRY_CAUSAL) + 6 * 64 * 4
    dec = _lib.make_shape(batch=128, heads=32, n=1, d=128, dv=128, m=256, p=2, t=4)
    assert (L.llops_workspace_bytes(ctypes.byref(dec), _lib.ENTRY_GATED_DECODE)
            == L.llops_workspace_bytes(ctypes.byref(dec), _lib.ENTRY_DECODE))


@fake_ptr
def test_gated_decode_requires_gate(L):
    s = _shape()
    need = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_GATED_DECODE)
    st = L.llops_gated_decode_step(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                   FAKE, FAKE, FAKE, need, None)
    assert st == 1 and "log_gate is null" in _err(L)
    st = L.llops_gated_decode_step(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, FAKE, need - 1, None)
    assert st == 3, _err(L)


@pytest.mark.parametrize("bad,code", [
    (dict(m=96), 2), (dict(p=3), 2), (dict(m=256, dv=64), 2), (dict(m=128, dv=128), 2),
    (dict(in_dtype=_lib.F32), 2), (dict(delta=-1.0), 1),
])
@fake_ptr
def test_gated_bwd_validation(L, bad, code):
    s = _shape(**{"t": 4, **bad})
    ws = L.llops_workspace_bytes(ctypes.byref(_shape(t=4)), _lib.ENTRY_GATED_CAUSAL_BWD)
    assert ws > 0
    assert L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_GATED_CAUSAL_BWD) == 0
    st = L.llops_linattn_gated_causal_bwd(ctypes.byref(s), *([FAKE] * 14), ws, None)
    assert st == code, _err(L)


@fake_ptr
def test_gated_bwd_pointers_and_workspace(L):
    s = _shape(t=4)
    need = L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_GATED_CAUSAL_BWD)
    assert need > L.llops_workspace_bytes(ctypes.byref(s), _lib.ENTRY_CAUSAL_BWD)
    args = [FAKE] * 14
    args[5] = None  # log_gate
    st = L.llops_linattn_gated_causal_bwd(ctypes.byref(s), *args, need, None)
    assert st == 1 and "log_gate is null" in _err(L)
    args = [FAKE] * 14
    args[12] = None  # dlog_gate (index 13 is ws)
    st = L.llops_linattn_gated_causal_bwd(ctypes.byref(s), *args, need, None)
    assert st == 1 and "dlog_gate is null" in _err(L)
    st = L.llops_linattn_gated_causal_bwd(ctypes.byref(s), *([FAKE] * 14), need - 1, None)
    assert st == 3 and "workspace" in _err(L)


@fake_ptr
def test_decode_noalloc_size_limit(L):
    """The allocation-free decode refuses a shape whose scratch exceeds its
    16 MiB static buffer, before touching any device (status UNSUPPORTED)."""
    big = _shape(batch=4096, heads=8, n=1, d=128, dv=128, m=256, p=2, t=4)
    st = L.llops_decode_step_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, None)
    assert st == 2 and "static" in _err(L), _err(L)
    # invalid shapes fail validation first
    st = L.llops_decode_step_noalloc(ctypes.byref(_shape(p=0)), FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, FAKE, None)
    assert st == 1
