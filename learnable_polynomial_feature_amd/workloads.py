"""Seeded synthetic inputs for the LLoPS hot path.

This module draws random numbers and rounds them to the storage dtype. It
holds none of the method's arithmetic (no feature map, no attention), so both
the HIP path's tests/bench and the CPU oracle may take their inputs from it.

Every tensor slice comes from its own counter-style stream,
``numpy.random.default_rng(SeedSequence([seed, tensor_id, *index]))``:
``index`` is ``(b, h)`` for per-sequence tensors, ``(h,)`` for Theta and
``(step,)`` for decode tokens. One head of a large workload can therefore be
regenerated on its own, bit for bit, without drawing the rest.

Distributions (the five workloads the hot path is measured on):
  Q, K  ~ N(0,1)/sqrt(d), or rows L2-normalised then scaled by 2
  V     ~ N(0,1) (the tiny fp32 case: N(0,1)/sqrt(d))
  Theta ~ N(0, 1/d), i.e. standard deviation 1/sqrt(d), one draw per head
  dphi  ~ N(0,1): the upstream gradient handed to the feature-map backward
  dO    ~ N(0,1): the upstream gradient of the attention output (float32)
  log gate g = log(sigmoid(u)), u ~ N(mu, 1) (float32, never rounded): a
        per-token state decay exp(g) in (0, 1); mu = 4 puts the median decay
        near 0.982, a retention-biased forgetting gate
Draws are float32; bf16 workloads round to bf16 with round-to-nearest-even and
keep the rounded values in float32 arrays (exactly representable), so the GPU
receives them losslessly and the oracle sees the identical numbers.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tensor ids for stream derivation
_T_Q, _T_K, _T_V, _T_THQ, _T_THK = 1, 2, 3, 4, 5
_T_PRE_K, _T_PRE_V, _T_STEP_Q, _T_STEP_K, _T_STEP_V = 6, 7, 8, 9, 10
_T_DPHI = 11
_T_DOUT = 12
_T_GATE, _T_STEP_GATE = 13, 14


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    n: int
    d: int
    dv: int
    p: int
    t: int
    m: int
    dtype: str            # "f32" or "bf16": storage of Q, K, V, Theta
    causal: bool
    square: bool
    normalize: bool
    delta: float
    chunk: int
    qk_dist: str = "gauss"        # "gauss": N(0,1)/sqrt(d); "l2x2": unit rows x 2
    v_scale: str = "unit"         # "unit": N(0,1); "inv_sqrt_d": N(0,1)/sqrt(d)
    prefix: int = 0               # decode: prefix length that builds S0, z0
    steps: int = 0                # decode: consecutive single-token steps
    seed: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def tokens(self) -> int:
        if self.steps:
            return self.batch * self.steps
        return self.batch * self.n


WORKLOADS = {
    "tiny_noncausal_f32": Workload(
        "tiny_noncausal_f32", batch=1, heads=1, n=256, d=16, dv=16, p=2, t=2, m=32,
        dtype="f32", causal=False, square=False, normalize=False, delta=0.0, chunk=0,
        v_scale="inv_sqrt_d"),
    "causal_p2_m64": Workload(
        "causal_p2_m64", batch=4, heads=12, n=2048, d=64, dv=64, p=2, t=4, m=64,
        dtype="bf16", causal=True, square=True, normalize=True, delta=1e-6, chunk=64),
    "causal_p3_m128": Workload(
        "causal_p3_m128", batch=2, heads=16, n=8192, d=64, dv=64, p=3, t=8, m=128,
        dtype="bf16", causal=True, square=True, normalize=True, delta=1e-6, chunk=64,
        qk_dist="l2x2"),
    "causal_long_n65536": Workload(
        "causal_long_n65536", batch=1, heads=32, n=65536, d=128, dv=128, p=2, t=4, m=256,
        dtype="bf16", causal=True, square=True, normalize=True, delta=1e-6, chunk=128),
    "decode_b128_h32": Workload(
        "decode_b128_h32", batch=128, heads=32, n=1, d=128, dv=128, p=2, t=4, m=256,
        dtype="bf16", causal=True, square=True, normalize=True, delta=1e-6, chunk=128,
        prefix=4096, steps=1000),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    out = (r.astype(np.uint32) << 16).view(np.float32)
    return out.reshape(x.shape)


def _stream(seed: int, tensor_id: int, *index: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor_id, *index]))


def _normal(seed, tensor_id, index, shape) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _stream(seed, tensor_id, *index).standard_normal(out=out, dtype=np.float32)
    return out


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _store(w: Workload, x: np.ndarray) -> np.ndarray:
    return round_bf16(x) if w.dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def qk_slice(w: Workload, which: str, b: int, h: int, n: int | None = None) -> np.ndarray:
    """One (b, h) slice of Q or K, shape [n, d], already in storage precision."""
    n = w.n if n is None else n
    tid = _T_Q if which == "q" else _T_K
    x = _normal(w.seed, tid, (b, h), (n, w.d))
    if w.qk_dist == "gauss":
        x = x / np.float32(np.sqrt(w.d))
    elif w.qk_dist == "l2x2":
        x64 = x.astype(np.float64)
        x64 = 2.0 * x64 / np.linalg.norm(x64, axis=1, keepdims=True)
        x = x64.astype(np.float32)
    else:
        raise ValueError(w.qk_dist)
    return _store(w, x)


def v_slice(w: Workload, b: int, h: int, n: int | None = None) -> np.ndarray:
    n = w.n if n is None else n
    x = _normal(w.seed, _T_V, (b, h), (n, w.dv))
    if w.v_scale == "inv_sqrt_d":
        x = x / np.float32(np.sqrt(w.d))
    return _store(w, x)


def theta_head(w: Workload, which: str, h: int) -> np.ndarray:
    """Theta for one head, shape [p, t, d, m], entries ~ N(0, 1/d)."""
    tid = _T_THQ if which == "q" else _T_THK
    x = _normal(w.seed, tid, (h,), (w.p, w.t, w.d, w.m)) / np.float32(np.sqrt(w.d))
    return _store(w, x)


def dphi_slice(w: Workload, b: int, h: int, bf16: bool = False) -> np.ndarray:
    """One (b, h) slice [n, m] of the feature map's upstream gradient, float32
    draws (rounded to bf16 values when ``bf16``)."""
    x = _normal(w.seed, _T_DPHI, (b, h), (w.n, w.m))
    return round_bf16(x) if bf16 else x


def dout_slice(w: Workload, b: int, h: int) -> np.ndarray:
    """One (b, h) slice [n, dv] of the attention output's upstream gradient."""
    return _normal(w.seed, _T_DOUT, (b, h), (w.n, w.dv))


def _log_sigmoid(u: np.ndarray) -> np.ndarray:
    # log(1 / (1 + exp(-u))) without overflow for large |u|
    u64 = u.astype(np.float64)
    return (np.minimum(u64, 0.0) - np.log1p(np.exp(-np.abs(u64)))).astype(np.float32)


def gate_slice(w: Workload, b: int, h: int, n: int | None = None, mu: float = 4.0) -> np.ndarray:
    """One (b, h) slice [n] of per-token log gates, log(sigmoid(N(mu, 1)))."""
    n = w.n if n is None else n
    return _log_sigmoid(_normal(w.seed, _T_GATE, (b, h), (n,)) + np.float32(mu))


def log_gates(w: Workload, heads: list[int] | None = None, batches: list[int] | None = None,
              mu: float = 4.0) -> np.ndarray:
    """Log gates [B', H', n] float32 for the selected batch rows and heads."""
    heads = list(range(w.heads)) if heads is None else list(heads)
    batches = list(range(w.batch)) if batches is None else list(batches)
    g = np.empty((len(batches), len(heads), w.n), np.float32)
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            g[bi, hi] = gate_slice(w, b, h, mu=mu)
    return g


def decode_step_gates(w: Workload, step: int, mu: float = 4.0) -> np.ndarray:
    """Step ``step``'s log gates [B, H], log(sigmoid(N(mu, 1)))."""
    return _log_sigmoid(_normal(w.seed, _T_STEP_GATE, (step,), (w.batch, w.heads))
                        + np.float32(mu))


def dout(w: Workload, heads: list[int] | None = None,
         batches: list[int] | None = None) -> np.ndarray:
    """dO [B', H', n, dv] float32 for the selected batch rows and heads."""
    heads = list(range(w.heads)) if heads is None else list(heads)
    batches = list(range(w.batch)) if batches is None else list(batches)
    G = np.empty((len(batches), len(heads), w.n, w.dv), np.float32)
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            G[bi, hi] = dout_slice(w, b, h)
    return G


def q_and_dphi(w: Workload, heads: list[int] | None = None,
               batches: list[int] | None = None, bf16_dphi: bool = False) -> dict:
    """Q [B', H', n, d] (the feature map's input X) and dphi [B', H', n, m]."""
    heads = list(range(w.heads)) if heads is None else list(heads)
    batches = list(range(w.batch)) if batches is None else list(batches)
    B, H = len(batches), len(heads)
    Q = np.empty((B, H, w.n, w.d), np.float32)
    G = np.empty((B, H, w.n, w.m), np.float32)

    def fill(bh):
        bi, hi = bh
        Q[bi, hi] = qk_slice(w, "q", batches[bi], heads[hi])
        G[bi, hi] = dphi_slice(w, batches[bi], heads[hi], bf16_dphi)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, [(bi, hi) for bi in range(B) for hi in range(H)]))
    return {"Q": Q, "dphi": G, "theta_q": np.stack([theta_head(w, "q", h) for h in heads])}


def generate(w: Workload, heads: list[int] | None = None,
             batches: list[int] | None = None) -> dict:
    """Q, K, V [B', H', n, d|dv] and theta_q, theta_k [H', p, t, d, m] for the
    selected batch rows and heads (all by default), in storage precision."""
    heads = list(range(w.heads)) if heads is None else list(heads)
    batches = list(range(w.batch)) if batches is None else list(batches)
    B, H = len(batches), len(heads)
    Q = np.empty((B, H, w.n, w.d), np.float32)
    K = np.empty((B, H, w.n, w.d), np.float32)
    V = np.empty((B, H, w.n, w.dv), np.float32)

    def fill(bh):
        bi, hi = bh
        b, h = batches[bi], heads[hi]
        Q[bi, hi] = qk_slice(w, "q", b, h)
        K[bi, hi] = qk_slice(w, "k", b, h)
        V[bi, hi] = v_slice(w, b, h)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, [(bi, hi) for bi in range(B) for hi in range(H)]))
    thq = np.stack([theta_head(w, "q", h) for h in heads])
    thk = np.stack([theta_head(w, "k", h) for h in heads])
    return {"Q": Q, "K": K, "V": V, "theta_q": thq, "theta_k": thk}


def decode_prefix(w: Workload, heads: list[int] | None = None,
                  batches: list[int] | None = None) -> dict:
    """The prefix keys and values [B', H', prefix, d|dv] whose sums build the
    decode state: K_pre ~ N(0,1), V_pre ~ N(0,1) (storage precision)."""
    heads = list(range(w.heads)) if heads is None else list(heads)
    batches = list(range(w.batch)) if batches is None else list(batches)
    B, H, L = len(batches), len(heads), w.prefix
    Kp = np.empty((B, H, L, w.d), np.float32)
    Vp = np.empty((B, H, L, w.dv), np.float32)

    def fill(bh):
        bi, hi = bh
        b, h = batches[bi], heads[hi]
        Kp[bi, hi] = _store(w, _normal(w.seed, _T_PRE_K, (b, h), (L, w.d)))
        Vp[bi, hi] = _store(w, _normal(w.seed, _T_PRE_V, (b, h), (L, w.dv)))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, [(bi, hi) for bi in range(B) for hi in range(H)]))
    return {"K_pre": Kp, "V_pre": Vp}


def decode_step_tokens(w: Workload, step: int) -> dict:
    """Step ``step``'s new tokens q, k, v: [B, H, d|dv], each ~ N(0,1)."""
    shp = (w.batch, w.heads)
    return {
        "q": _store(w, _normal(w.seed, _T_STEP_Q, (step,), shp + (w.d,))),
        "k": _store(w, _normal(w.seed, _T_STEP_K, (step,), shp + (w.d,))),
        "v": _store(w, _normal(w.seed, _T_STEP_V, (step,), shp + (w.dv,))),
    }


def decode_tokens(w: Workload, steps: int | None = None) -> dict:
    """All decode steps stacked: q, k [S, B, H, d], v [S, B, H, dv]."""
    steps = w.steps if steps is None else steps
    q = np.empty((steps, w.batch, w.heads, w.d), np.float32)
    k = np.empty_like(q)
    v = np.empty((steps, w.batch, w.heads, w.dv), np.float32)

    def fill(s):
        tok = decode_step_tokens(w, s)
        q[s], k[s], v[s] = tok["q"], tok["k"], tok["v"]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(steps)))
    return {"q": q, "k": k, "v": v}
