"""Element-wise acceptance test for bf16 GEMM outputs against the oracle.

An element passes iff |gpu - oracle| <= 2*ulp(oracle) + 1e-3*sqrt(K), where
ulp(v) is the spacing of bf16 values at the oracle's value v:
2^(max(floor(log2|v|), -126) - 7), and 2^-133 for v == 0.  Infinities must
match exactly; a NaN passes only against a NaN.
"""
from __future__ import annotations

import numpy as np


def bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact), by widening to float32 bits."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def ulp_bf16(v) -> np.ndarray:
    v = np.abs(np.asarray(v, dtype=np.float64))
    out = np.full(v.shape, 2.0 ** -133)
    nz = (v > 0) & np.isfinite(v)
    e = np.floor(np.log2(v[nz]))
    # log2 of an exact power of two is exact; guard the floor anyway
    e = np.where(2.0 ** e > v[nz], e - 1, e)
    e = np.maximum(e, -126)
    out[nz] = 2.0 ** (e - 7)
    return out


def tolerance_report(gpu_bits, ref_bits, K: int) -> dict:
    g = bits_to_f64(gpu_bits).reshape(-1)
    r = bits_to_f64(ref_bits).reshape(-1)
    tol = 2.0 * ulp_bf16(r) + 1e-3 * np.sqrt(max(K, 0))
    both_nan = np.isnan(g) & np.isnan(r)
    inf_ok = np.isinf(r) & (g == r)
    finite = np.isfinite(r) & np.isfinite(g)
    err = np.zeros_like(r)
    err[finite] = np.abs(g[finite] - r[finite])
    ok = both_nan | inf_ok | (finite & (err <= tol))
    ulps = np.zeros_like(r)
    ulps[finite] = err[finite] / ulp_bf16(r[finite])
    bad = np.flatnonzero(~ok)
    return {
        "n": int(r.size),
        "fail": int(bad.size),
        "first_bad": bad[:8].tolist(),
        "max_abs_err": float(err.max()) if r.size else 0.0,
        "max_ulp": float(ulps[finite].max()) if finite.any() else 0.0,
        "mean_ulp": float(ulps[finite].mean()) if finite.any() else 0.0,
        "exact": int(np.count_nonzero(finite & (err == 0))),
        "le1ulp": int(np.count_nonzero(finite & (ulps <= 1))),
        "le2ulp": int(np.count_nonzero(finite & (ulps <= 2))),
    }


def assert_within_tolerance(gpu_bits, ref_bits, K: int, what: str = "") -> dict:
    rep = tolerance_report(gpu_bits, ref_bits, K)
    assert rep["fail"] == 0, f"{what}: {rep['fail']} of {rep['n']} elements outside tolerance: {rep}"
    return rep
