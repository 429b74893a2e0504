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
    # error as a fraction of the allowed tolerance (<= 1 passes): unlike an
    # error in ulps it stays meaningful for outputs near zero, whose bf16 ulp
    # is far below the fp32 accumulation error the absolute slack covers
    ratio = np.zeros_like(r)
    ratio[finite] = err[finite] / tol[finite]
    ulps = np.zeros_like(r)
    ulps[finite] = err[finite] / ulp_bf16(r[finite])
    bad = np.flatnonzero(~ok)
    return {
        "n": int(r.size),
        "fail": int(bad.size),
        "first_bad": bad[:8].tolist(),
        "max_abs_err": float(err.max()) if r.size else 0.0,
        "max_err_over_tol": float(ratio[finite].max()) if finite.any() else 0.0,
        "mean_err_over_tol": float(ratio[finite].mean()) if finite.any() else 0.0,
        "exact": int(np.count_nonzero(finite & (err == 0))),
        "le1ulp": int(np.count_nonzero(finite & (ulps <= 1))),
        "le2ulp": int(np.count_nonzero(finite & (ulps <= 2))),
    }


def assert_within_tolerance(gpu_bits, ref_bits, K: int, what: str = "") -> dict:
    rep = tolerance_report(gpu_bits, ref_bits, K)
    assert rep["fail"] == 0, f"{what}: {rep['fail']} of {rep['n']} elements outside tolerance: {rep}"
    return rep


def q8_report(q_gpu, q_ref, t_exact, scale_per_elem, zp: int, K: int) -> dict:
    """Acceptance test for int8 codes against the oracle.

    The oracle decides each code from the exact epilogue value; the kernel
    from its fp32 accumulation, which may differ by about 1e-3*sqrt(K) in
    absolute terms and 2^-16 relative (the bf16 tolerance's fp32 error
    model).  So a code must equal the oracle's exactly unless the oracle's
    exact t = y*scale + zp lies within
        delta = |scale|*1e-3*sqrt(K) + 2^-16*|t - zp| + 2^-22*|t|
    of a rounding boundary (a half-integer), where the neighbouring code is
    also accepted.  Saturated codes have no boundary at the clamp (both
    sides of +-127.5 / -128.5 give the same code).  A NaN t must give 0.
    """
    g = np.asarray(q_gpu, dtype=np.int64).reshape(-1)
    r = np.asarray(q_ref, dtype=np.int64).reshape(-1)
    t = np.asarray(t_exact, dtype=np.float64).reshape(-1)
    s = np.abs(np.asarray(scale_per_elem, dtype=np.float64).reshape(-1))
    delta = s * 1e-3 * np.sqrt(max(K, 0)) + 2.0 ** -16 * np.abs(t - zp) + 2.0 ** -22 * np.abs(t)
    frac_dist = np.abs(t - (np.floor(t) + 0.5))
    near = np.isfinite(t) & (frac_dist <= delta)
    nan = np.isnan(t)
    ok = (g == r) | (near & (np.abs(g - r) <= 1))
    ok &= ~nan | ((g == 0) & (r == 0))
    bad = np.flatnonzero(~ok)
    return {"n": int(r.size), "fail": int(bad.size), "first_bad": bad[:8].tolist(),
            "exact": int(np.count_nonzero(g == r)), "near_boundary": int(np.count_nonzero(near)),
            "max_code_diff": int(np.abs(g - r).max()) if r.size else 0}


def assert_q8_within_tolerance(q_gpu, q_ref, t_exact, scale_per_elem, zp, K, what="") -> dict:
    rep = q8_report(q_gpu, q_ref, t_exact, scale_per_elem, zp, K)
    assert rep["fail"] == 0, f"{what}: {rep['fail']} of {rep['n']} int8 codes outside tolerance: {rep}"
    return rep
