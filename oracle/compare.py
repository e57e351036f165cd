"""Tolerance checks of a GPU forward against the fp64 oracle (test infrastructure).

fp32 outputs: |gpu - ref| <= 1e-5 * (S + |bias|), where S = sum |f*w| over the
terms the oracle added for that output; an output with no present neighbour
(S == 0) must equal fp32(bias) exactly.

bf16 outputs: |gpu - ref| <= 2 ulp_bf16(ref), or the fp32 criterion above
(outputs that cancel to near zero carry fp32 accumulation error that is tiny
against S but many bf16 ulps of the small result).  ulp_bf16(x) =
2^(floor(log2|x|) - 7).  The number of outputs that fail the strict 2-ulp test
and the largest ulp error are reported alongside.
"""
from __future__ import annotations

import numpy as np


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.abs(np.asarray(x, dtype=np.float64))
    m, e = np.frexp(ax)                 # ax = m * 2^e, m in [0.5, 1)
    u = np.ldexp(1.0, e - 8)            # 2^(floor(log2 ax) - 7)
    return np.where(ax > 0, u, 0.0)


def check_forward(gpu, ref, S, bias, dtype: str) -> dict:
    """gpu: (n, Co) array of the GPU outputs (any float dtype, converted to f64);
    ref, S: (n, Co) fp64 from the oracle; bias: (Co,) float32 or None."""
    g = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    b = np.zeros(ref.shape[1]) if bias is None else np.abs(np.asarray(bias, dtype=np.float64))
    err = np.abs(g - ref)
    tol = 1e-5 * (S + b[None, :])
    norm_err = err / np.maximum(S + b[None, :], 1e-300)
    rep = {"n": int(g.size), "max_norm_err": float(norm_err.max()) if g.size else 0.0}
    if dtype == "f32":
        ok = err <= tol
        zero = S == 0
        if zero.any():
            bias32 = np.zeros(ref.shape[1]) if bias is None else np.asarray(bias, np.float32).astype(np.float64)
            ok[zero] &= (g == np.broadcast_to(bias32[None, :], g.shape))[zero]
    elif dtype == "bf16":
        u = ulp_bf16(ref)
        strict = err <= 2 * u
        ok = strict | (err <= tol)
        with np.errstate(divide="ignore", invalid="ignore"):
            ulps = np.where(u > 0, err / u, np.where(err > 0, np.inf, 0.0))
        rep["strict_2ulp_fail"] = int((~strict).sum())
        rep["max_ulp"] = float(ulps.max()) if g.size else 0.0
    else:
        raise ValueError(dtype)
    rep["fail"] = int((~ok).sum())
    if rep["fail"]:
        i = np.argwhere(~ok)[0]
        rep["first_fail"] = {"row": int(i[0]), "col": int(i[1]), "gpu": float(g[tuple(i)]),
                             "ref": float(ref[tuple(i)]), "S": float(S[tuple(i)])}
    return rep
