"""Shared helpers of the GPU parity tests (no test functions here)."""
import sys

import numpy as np

from dual_window_attention_amd import inputs as I

# bf16 inputs: max |err| <= 2e-2 and relative L2 <= 1e-2 against fp64.
BF16_TOL = (2e-2, 1e-2)
# fp32 inputs: the fp32 arithmetic bound this build sets for itself.
F32_TOL = (1e-4, 1e-5)


def tol_for(dtype: str):
    return BF16_TOL if dtype == "bf16" else F32_TOL


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    err = np.abs(got - ref).max() if got.size else 0.0
    nrm = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / nrm if nrm > 0 else np.linalg.norm(got - ref)
    return float(err), float(rel)


def assert_close(got, ref, tol, what: str):
    err, rel = errors(got, ref)
    say(f"  {what}: max|err|={err:.3e} relL2={rel:.3e} (tol {tol[0]:g}, {tol[1]:g})")
    assert err <= tol[0] and rel <= tol[1], f"{what}: max|err|={err:.3e} relL2={rel:.3e}"


def assert_close_stored(got, ref, tol, what: str, dtype: str):
    """Intermediates the layer keeps in its storage type.  bf16 storage adds
    up to half an ulp (2^-9 relative) per rounding; such a tensor is held to
    the relative L2 bound and, per element, to tol_abs plus 2^-6 |ref|: each
    of O, the RMSNorm output and Z is rounded once on the way, and the two
    length-d_model dot products of the gate and up projections spread the
    input rounding (std ~2^-9/sqrt(3) per operand) over tens of millions of
    elements, whose tails reach several half-ulps.
    fp32 intermediates use ``tol``."""
    if dtype != "bf16":
        return assert_close(got, ref, tol, what)
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    ex = np.abs(got - ref) - (tol[0] + 2.0 ** -6 * np.abs(ref))
    worst = float(ex.max()) if ex.size else -1.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    say(f"  {what} (bf16-stored): worst excess={worst:.3e} relL2={rel:.3e}")
    assert worst <= 0 and rel <= tol[1], f"{what}: excess={worst:.3e} relL2={rel:.3e}"


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def attn_tensors(B, T, Hq, Hkv, D, dtype, seed, outlier=0.0):
    cfg = I.LayerConfig(name="case", dtype=dtype, batch=B, seq=T, n_q_heads=Hq,
                        n_kv_heads=Hkv, head_dim=D, w_teacher=1, w_student=1, seed=seed,
                        outlier_frac=outlier, outlier_scale=8.0)
    return I.attention_inputs(cfg)
