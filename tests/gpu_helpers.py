"""Shared helpers of the GPU parity tests (no test functions here).

Tolerance.  For bf16 inputs the bound is 1e-2 relative, in the L2 norm and
in the max norm, with the stated absolute bound 2e-2 as the floor of the
max norm:

    ||got - ref||_2   <= 1e-2 ||ref||_2
    ||got - ref||_inf <= max(2e-2, 1e-2 ||ref||_inf)

Error model behind it: the GPU path rounds its intermediates (O, the RMSNorm
output, Z, the conv outputs, R, the chunk writes and the per-chunk weights)
to bf16, each a relative perturbation of at most u = 2^-8 of the rounded
value, and accumulates in fp32.  An output element combines a handful of
such perturbations of terms no larger than the tensor's range, so its error
is a small multiple of u ||ref||_inf; 1e-2 ||ref||_inf = 2.56 u.  The
absolute 2e-2 is the bound stated for unit-scale activations and governs
every tensor whose values stay within +-2; beyond that an absolute bound
that does not grow with the values would ask the bf16 pipeline for more
significant bits than bf16 has (the spacing of bf16 values in [256, 512) is
2).  fp32 inputs use the same form with 1e-5 relative and a 1e-4 floor.
"""
import sys

import numpy as np

from dual_window_attention_amd import inputs as I

# (absolute floor of the max norm, relative bound in the L2 and max norms)
BF16_TOL = (2e-2, 1e-2)
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


def max_bound(ref, tol) -> float:
    """The max-norm bound: max(floor, rel * ||ref||_inf)."""
    ref = np.asarray(ref, dtype=np.float64)
    top = float(np.abs(ref).max()) if ref.size else 0.0
    return max(tol[0], tol[1] * top)


def assert_close(got, ref, tol, what: str):
    err, rel = errors(got, ref)
    bound = max_bound(ref, tol)
    say(f"  {what}: max|err|={err:.3e} (bound {bound:.3g}) relL2={rel:.3e} (bound {tol[1]:g})")
    assert err <= bound and rel <= tol[1], f"{what}: max|err|={err:.3e} relL2={rel:.3e}"


# bf16 unit roundoff: the largest relative error of one rounding to bf16
U_BF16 = 2.0 ** -8


def assert_correction(corr, corr_ref, y_ref, chunk: int, dtype: str, what: str = "correction"):
    """The fast-weight correction y - W_down0 z on its own, so that an error
    in the small part of y that the fast weight adds cannot hide in y's
    bound.  y_ref [B, T, d] is the reference MLP output.  The error has
    three parts:
      * the fast-weight path's own roundings: the relative bound of every
        other output, rel ||corr_ref||;
      * the one rounding of each per-chunk weight S_i (i >= 1) to bf16
        before the apply, which perturbs y_t = S_i z_t in proportion to y,
        not to the correction: a relative rounding error of at most u per
        weight entry has rms at most u/sqrt(3) and lands on y_t with rms at
        most u/sqrt(3) |y_t| (u = 2^-8; chunk 0 uses W_down0 itself);
      * the fp32 sums of the apply, relative 1e-5 (the fp32 bound) of y.
        ||corr - corr_ref|| <= rel ||corr_ref|| + (u/sqrt(3)) ||y_ref[t >= C]||
                               + 1e-5 ||y_ref||"""
    tol = tol_for(dtype)
    corr = np.asarray(corr, dtype=np.float64)
    corr_ref = np.asarray(corr_ref, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = float(np.linalg.norm(corr - corr_ref))
    nc = float(np.linalg.norm(corr_ref))
    snap = U_BF16 / np.sqrt(3.0) * float(np.linalg.norm(y_ref[:, chunk:])) if dtype == "bf16" else 0.0
    bound = tol[1] * nc + snap + F32_TOL[1] * float(np.linalg.norm(y_ref))
    say(f"  {what}: |err|={err:.3e} bound {bound:.3e} (|corr|={nc:.3e}, relL2 "
        f"{err / max(nc, 1e-300):.3e})")
    assert err <= bound, f"{what}: |err|={err:.3e} > {bound:.3e}"


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def attn_tensors(B, T, Hq, Hkv, D, dtype, seed, outlier=0.0):
    cfg = I.LayerConfig(name="case", dtype=dtype, batch=B, seq=T, n_q_heads=Hq,
                        n_kv_heads=Hkv, head_dim=D, w_teacher=1, w_student=1, seed=seed,
                        outlier_frac=outlier, outlier_scale=8.0)
    return I.attention_inputs(cfg)
