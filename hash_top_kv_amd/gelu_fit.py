"""The GELU polynomial of the key and query encoders (csrc/encode_core.h), written out.

GELU(a) = a Phi(a) = max(a, 0) - x Phi(-x) with x = |a|.  The encoders compute
Phi(-x) = 2^R(x) with R a degree-5 polynomial in x, so one GELU costs five fused
multiply-adds, one base-2 exponential, an integer max and a final fused multiply-add.

R is chosen by a linear program over a dense grid of x in [0, 9] and a geometric grid
up to 10^4: it minimises the bound d such that
    |x 2^R(x) - x Phi(-x)| <= d     (bounds written on R through log2),
with R's leading coefficient negative, so that R falls without bound and 2^R
underflows to zero for large x (no clamp is needed).  The error is that of the GELU
itself, not of R: where x Phi(-x) is tiny, R may be far off.

    python hash_top_kv_amd/gelu_fit.py          # refit, and check the constants in encode_core.h

`check()` evaluates the constants exactly as the kernel does (fp32 Horner with fused
multiply-adds, fp32 exponential and result) and returns the largest absolute error
against GELU in float64 beyond the fp32 rounding of the result.
"""
from __future__ import annotations

import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ENCODE = os.path.join(HERE, "csrc", "encode_core.h")


def constants(path: str = ENCODE) -> np.ndarray:
    """kGelu0 .. kGelu5 as written in encode_core.h (float32)."""
    text = open(path).read()
    c = [float(re.search(rf"kGelu{k}\s*=\s*([-+0-9.eE]+)f", text).group(1)) for k in range(6)]
    return np.array(c, dtype=np.float32)


def _f32(v):
    with np.errstate(over="ignore", invalid="ignore"):
        return np.asarray(v, np.float64).astype(np.float32).astype(np.float64)


def gelu_kernel(a, c) -> np.ndarray:
    """The encoders' GELU in fp32 (each fused multiply-add rounded once)."""
    a = _f32(a)
    x = np.abs(a)
    r = np.full_like(x, np.float64(c[-1]))
    with np.errstate(over="ignore", invalid="ignore"):
        for k in range(len(c) - 2, -1, -1):
            r = _f32(r * x + np.float64(c[k]))
        g = _f32(np.exp2(r))
        return _f32(-x * g + np.maximum(a, 0.0))


def check(c=None) -> float:
    """Max |GELU_kernel - GELU| beyond the fp32 rounding of the result, over finite a."""
    from scipy.special import ndtr
    if c is None:
        c = constants()
    a = np.concatenate([np.linspace(-40, 40, 2_000_001), np.geomspace(40, 1e30, 1000),
                        -np.geomspace(40, 1e30, 1000)])
    a = _f32(a)
    exact = a * ndtr(a)
    err = np.abs(gelu_kernel(a, c) - exact) - np.abs(exact) * 2.0 ** -24
    return float(np.max(err))


def fit(deg: int = 5, xs: float = 9.0, xt: float = 1e4, n: int = 3000):
    """Smallest-error degree-`deg` R by bisection on the linear program's feasibility."""
    from scipy.optimize import linprog
    from scipy.special import ndtr

    x = np.concatenate([np.linspace(1e-4, xs, n), np.geomspace(xs, xt, 800)[1:]])
    xp = np.where(x < 38, x * ndtr(-x), 0.0)
    V = np.vander(x / xs, deg + 1, increasing=True)
    rs = np.maximum(1.0, np.max(np.abs(V), axis=1))

    def feasible(d):
        ok = xp - d > 0
        A = np.vstack([V / rs[:, None], -(V[ok] / rs[ok, None])])
        b = np.concatenate([np.log2((xp + d) / x) / rs, -np.log2((xp[ok] - d) / x[ok]) / rs[ok]])
        lead = np.zeros(deg + 1)
        lead[-1] = 1.0
        A = np.vstack([A, lead])
        b = np.concatenate([b, [-1e-9]])
        slack = np.concatenate([1.0 / rs, 1.0 / rs[ok], [0.0]])
        A2 = np.hstack([A, slack[:, None]])
        cobj = np.zeros(deg + 2)
        cobj[-1] = -1.0
        r = linprog(cobj, A_ub=A2, b_ub=b, bounds=[(None, None)] * (deg + 1) + [(None, 1.0)],
                    method="highs")
        if r.status != 0 or r.x[-1] < 0:
            return None
        return r.x[:deg + 1] / xs ** np.arange(deg + 1)

    lo, hi = 1e-9, 1e-3
    for _ in range(30):
        mid = np.sqrt(lo * hi)
        if feasible(mid) is not None:
            hi = mid
        else:
            lo = mid
    return feasible(hi), hi


if __name__ == "__main__":
    c, d = fit()
    print("fitted R:", ", ".join(f"{v:.9e}" for v in c), f"(bound on the grid {d:.2e})")
    print(f"fitted constants, fp32 kernel arithmetic: max error {check(np.float32(c)):.2e}")
    print(f"constants in encode_core.h: max error {check():.2e}")
