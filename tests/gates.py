"""Comparison gates shared by the tests (GPU result or oracle variant vs the oracle).

Floating point: max-abs error <= 1e-5 (fp32) or 2e-2 (bf16) after widening
to float64, and relative RMS error ||x - ref|| / ||ref|| <= 1e-5 (fp32) or
1e-2 (bf16).  The relative gate is there because N(0, 1) inputs give
outputs of RMS about sqrt(e / L), small enough at long L that a wrong kernel
could pass the absolute gate alone.
"""
import numpy as np

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-2)}


def errors(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if out.shape != ref.shape:
        raise ValueError(f"shape mismatch {out.shape} vs {ref.shape}")
    diff = out - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    if not np.all(np.isfinite(out)):
        max_abs = rel = float("inf")
    return max_abs, rel


def passes(out, ref, dtype: str) -> bool:
    a, r = errors(out, ref)
    ta, tr = TOL[dtype]
    return a <= ta and r <= tr


def check(out, ref, dtype: str, what: str = ""):
    a, r = errors(out, ref)
    ta, tr = TOL[dtype]
    assert a <= ta and r <= tr, f"{what}: max_abs {a:.3e} (tol {ta}), rel_rms {r:.3e} (tol {tr})"
    return a, r
