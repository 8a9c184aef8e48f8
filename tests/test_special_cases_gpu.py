"""GPU feature map on the special cases the LLoPS notes name (key design 2),
checked against their closed forms, not against the oracle.

- Flatten: one projection W shared by all p factors and t = 1 gives the
  element-wise power phi = (X W)^p.
- BASED (degree-2 part): Theta_1 column (a, b) = W column a and Theta_2
  column (a, b) = W column b give phi = vec((X W)(X W)^T), the outer product
  of the r-dimensional projection with itself (m = r^2).

The closed forms are evaluated here in float64 from the same bf16 inputs the
kernel receives; these are also the shapes the unrolled kernels gained for the
p = 4 and t = 1 variants (d = 64 and 128).
"""
import numpy as np
import pytest

from learnable_polynomial_feature_amd.workloads import round_bf16

from _util import TOL_FEAT_BF16_IN, TOL_FEAT_BF16_OUT, announce, dev, host, rel_fro

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _x(rng, B, H, n, d):
    return round_bf16(rng.standard_normal((B, H, n, d)).astype(np.float32) * 0.5)


def _proj(X, W):
    """(X W) per head in float64: X [B][H][n][d], W [H][d][r] -> [B][H][n][r]."""
    return np.einsum("bhnd,hdr->bhnr", X.astype(np.float64), W.astype(np.float64))


@pytest.mark.parametrize("B,H,n,d,m,p,out_bf16", [
    (1, 2, 1500, 128, 256, 2, False),
    (1, 2, 1500, 128, 256, 4, False),
    (2, 3, 700, 64, 128, 4, False),
    (1, 2, 900, 64, 64, 2, True),
    (64, 4, 1, 128, 256, 4, False),
])
def test_flatten_is_elementwise_power(lib, B, H, n, d, m, p, out_bf16):
    rng = np.random.default_rng(11)
    X = _x(rng, B, H, n, d)
    W = round_bf16(rng.standard_normal((H, d, m)).astype(np.float32) / np.sqrt(d))
    theta = np.ascontiguousarray(np.repeat(W[:, None, None], p, axis=1))  # [H][p][1][d][m]
    announce(f"flatten B={B} H={H} n={n} d={d} m={m} p={p} bf16_out={out_bf16}")
    odt = torch.bfloat16 if out_bf16 else torch.float32
    phi = lib.llops_featmap(dev(X, torch.bfloat16), dev(theta, torch.bfloat16), square=False,
                            out_dtype=odt)
    torch.cuda.synchronize()
    want = _proj(X, W) ** p
    err = rel_fro(host(phi), want)
    assert err <= (TOL_FEAT_BF16_OUT if out_bf16 else TOL_FEAT_BF16_IN), err


@pytest.mark.parametrize("B,H,n,d,r", [(1, 2, 1200, 128, 16), (2, 2, 500, 64, 8), (128, 2, 1, 128, 16)])
def test_based_is_outer_product(lib, B, H, n, d, r):
    rng = np.random.default_rng(12)
    X = _x(rng, B, H, n, d)
    W = round_bf16(rng.standard_normal((H, d, r)).astype(np.float32) / np.sqrt(d))
    m = r * r
    a = np.arange(m) // r
    b = np.arange(m) % r
    theta = np.empty((H, 2, 1, d, m), np.float32)
    theta[:, 0, 0] = W[:, :, a]
    theta[:, 1, 0] = W[:, :, b]
    announce(f"BASED B={B} H={H} n={n} d={d} r={r}")
    phi = lib.llops_featmap(dev(X, torch.bfloat16), dev(theta, torch.bfloat16), square=False,
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    y = _proj(X, W)
    want = (y[..., :, None] * y[..., None, :]).reshape(B, H, n, m)
    err = rel_fro(host(phi), want)
    assert err <= TOL_FEAT_BF16_IN, err
