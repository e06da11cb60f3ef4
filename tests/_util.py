"""Shared test helpers: library loading (building it when absent) and error metrics."""
import os

import numpy as np


def ensure_built():
    import mixture_experts_layer_deterministic_amd as m
    if not os.path.exists(m.LIB_PATH):
        from mixture_experts_layer_deterministic_amd import build
        build.build(verbose=False)
    return m


def rel_maxabs(got, ref):
    """max |got - ref| / max |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


def rel_maxabs_over_rms(got, ref):
    """max |got - ref| / rms(ref): reported next to the two bounded forms, not bounded itself.
    A single one-ulp bf16 rounding difference on one of the largest elements already puts it
    near 2^-8 max|ref| / rms(ref), about 1-3e-2 for these outputs."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.sqrt(np.mean(ref ** 2)), 1e-300))


def rel_rms(got, ref):
    """rms(got - ref) / rms(ref), which equals the relative Frobenius error."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.sqrt(np.sum((got - ref) ** 2)) / max(np.sqrt(np.sum(ref ** 2)), 1e-300))


# Tolerances of the layer's parity bar:
# - the bf16 layer output and input gradient are within 1e-2 relative error, measured both as
#   max-abs (normalised by max |ref|) and as RMS; max-abs over rms(ref) is printed as well;
# - weight, router and routing-weight gradients are within 2e-2 relative Frobenius error.
TOL_ACT = 1e-2
TOL_GRAD = 2e-2


def assert_act(name, got, ref, tol=TOL_ACT):
    a, b = rel_maxabs(got, ref), rel_rms(got, ref)
    c = rel_maxabs_over_rms(got, ref)
    print(f"  {name}: rel max-abs {a:.3e}  rel rms {b:.3e}  (max-abs/rms(ref) {c:.3e})")
    assert a <= tol and b <= tol, (name, a, b)


def assert_grad(name, got, ref, tol=TOL_GRAD):
    f = rel_rms(got, ref)
    print(f"  {name}: rel fro {f:.3e}")
    assert f <= tol, (name, f)
