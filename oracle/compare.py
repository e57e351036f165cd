"""Tolerance checks of a GPU forward against the fp64 oracle (test infrastructure).

fp32 outputs: |gpu - ref| <= 1e-5 * (S + |bias|), where S = sum |f*w| over the
terms the oracle added for that output; an output with no present neighbour
(S == 0) must equal fp32(bias) exactly.

bf16 outputs: |gpu - ref| <= 2 ulp_bf16(ref), or the fp32 criterion above
(outputs that cancel to near zero carry fp32 accumulation error that is tiny
against S but many bf16 ulps of the small result).  An output with S == 0 must
equal bf16(bias) exactly: the accumulator is zero and the one rounding of the
fp32 bias to the output type (the page's kernel stores `(T)acc`) is exact
arithmetic.  ulp_bf16(x) is the spacing of bf16 values at |x|:
2^(floor(log2|x|) - 7) for normal |x| >= 2^-126, 2^-133 below (subnormals),
0 at x = 0.  The number of outputs that fail the strict 2-ulp test and the
largest ulp error are reported; more than max(16, strict_frac * outputs)
strict failures is itself a failure, since a systematic error (a wrong bias
rounding, a dropped term) shows first as many outputs outside 2 ulp.
"""
from __future__ import annotations

import numpy as np

STRICT_FLOOR = 16


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.abs(np.asarray(x, dtype=np.float64))
    m, e = np.frexp(ax)                 # ax = m * 2^e, m in [0.5, 1): floor(log2 ax) = e - 1
    e = np.maximum(e, -125)             # below 2^-126 the spacing stays that of the subnormals
    u = np.ldexp(1.0, e - 8)            # 2^(floor(log2 ax) - 7)
    return np.where(ax > 0, u, 0.0)


def bf16_round(x32: np.ndarray) -> np.ndarray:
    """fp32 values rounded to bf16 (nearest, ties to even) by the oracle's own
    pinned cast, returned as float64."""
    import torch
    import oracle
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x32, dtype=np.float32)))
    return oracle.cast(t, torch.bfloat16).to(torch.float64).numpy()


def check_forward(gpu, ref, S, bias, dtype: str, strict_frac: float = 1e-3) -> dict:
    """gpu: (n, Co) array of the GPU outputs (any float dtype, converted to f64);
    ref, S: (n, Co) fp64 from the oracle; bias: (Co,) float32 or None.
    rep["fail"] counts the outputs outside tolerance, plus (bf16) the strict
    2-ulp failures beyond the allowance."""
    g = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    b = np.zeros(ref.shape[1]) if bias is None else np.abs(np.asarray(bias, dtype=np.float64))
    err = np.abs(g - ref)
    tol = 1e-5 * (S + b[None, :])
    norm_err = err / np.maximum(S + b[None, :], 1e-300)
    rep = {"n": int(g.size), "max_norm_err": float(norm_err.max()) if g.size else 0.0}
    bias32 = np.zeros(ref.shape[1], np.float32) if bias is None else np.asarray(bias, np.float32)
    zero = S == 0
    excess = 0
    if dtype == "f32":
        ok = err <= tol
        if zero.any():
            ok[zero] = (g == np.broadcast_to(bias32.astype(np.float64)[None, :], g.shape))[zero]
    elif dtype == "bf16":
        u = ulp_bf16(ref)
        strict = err <= 2 * u
        ok = strict | (err <= tol)
        if zero.any():
            ok[zero] = (g == np.broadcast_to(bf16_round(bias32)[None, :], g.shape))[zero]
        with np.errstate(divide="ignore", invalid="ignore"):
            ulps = np.where(u > 0, err / u, np.where(err > 0, np.inf, 0.0))
        nstrict = int((~strict).sum())
        allowed = max(STRICT_FLOOR, int(strict_frac * g.size))
        excess = max(0, nstrict - allowed)
        rep["strict_2ulp_fail"] = nstrict
        rep["strict_2ulp_allowed"] = allowed
        rep["max_ulp"] = float(ulps.max()) if g.size else 0.0
    else:
        raise ValueError(dtype)
    rep["fail"] = int((~ok).sum()) + excess
    if (~ok).any():
        i = np.argwhere(~ok)[0]
        rep["first_fail"] = {"row": int(i[0]), "col": int(i[1]), "gpu": float(g[tuple(i)]),
                             "ref": float(ref[tuple(i)]), "S": float(S[tuple(i)])}
    return rep
