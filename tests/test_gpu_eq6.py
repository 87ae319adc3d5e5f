"""ttcd_fastweight_scan_eq6 (the unprojected write) on the GPU against the
fp64 oracle."""
import numpy as np
import pytest

from dual_window_attention_amd import inputs as I
from oracle import ttcd_oracle as O
from tests.gpu_helpers import assert_close, assert_correction, say, to_np, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BASE = I.CONFIGS[3]


def eq6_beta(cfg, z_s):
    """Raw keys have |z_S|^2 ~ d_ff: the step size is the workloads' gate
    u ~ U(0,1) over the mean squared key norm, which keeps the correction a
    visible part of y."""
    ms = float(np.mean(np.sum(z_s.astype(np.float64) ** 2, axis=-1)))
    return (I.beta_for(cfg) / np.float32(ms)).astype(np.float32)


def check_eq6(cfg, out_dtype="f32"):
    from dual_window_attention_amd import ttcd
    say(f"eq6 {cfg.dtype} B={cfg.batch} T={cfg.seq} f={cfg.d_ff} d={cfg.d_model} "
        f"C={cfg.chunk} y={out_dtype}")
    z = I.hidden_activations(cfg)
    w = I.layer_weights(cfg)
    beta = eq6_beta(cfg, z["z_s"].f64())
    zt, zs = I.to_torch(z["z_t"]), I.to_torch(z["z_s"])
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    y, st = ttcd.fastweight_scan_eq6(zt, zs, zt, I.to_torch(w["w_down0"]), I.f32_to_torch(beta),
                                     cfg.chunk, out_dtype=odt, want_state=True)
    torch.cuda.synchronize()
    ref = O.fastweight_scan_eq6(z["z_t"].f64(), z["z_s"].f64(), z["z_t"].f64(),
                                w["w_down0"].f64(), beta.astype(np.float64), cfg.chunk)
    tol = tol_for(cfg.dtype)
    assert_close(to_np(y), ref["y"], tol, f"y ({out_dtype} out)")
    assert_close(to_np(st), ref["state_complete"], tol,
                 f"state after the {cfg.seq // cfg.chunk} complete chunks")
    base = z["z_t"].f64() @ w["w_down0"].f64().T
    assert_correction(to_np(y) - base, ref["y"] - base, ref["y"], cfg.chunk, cfg.dtype)


@pytest.mark.parametrize("case", [
    dict(dtype="f32", batch=1, seq=300, d_model=64, d_ff=96, chunk=64, seed=51),
    dict(dtype="bf16", batch=2, seq=517, d_model=128, d_ff=256, chunk=128, seed=52),
    dict(dtype="f32", batch=2, seq=333, d_model=64, d_ff=128, chunk=32, seed=53),
    dict(dtype="bf16", batch=1, seq=100, d_model=64, d_ff=128, chunk=128, seed=54),
], ids=["f32", "bf16-B2-ragged", "f32-chunk32", "bf16-single-chunk"])
def test_eq6_small(case):
    check_eq6(BASE.scaled(**case))


def test_eq6_bf16_output():
    check_eq6(BASE.scaled(batch=1, seq=640, d_model=128, d_ff=256, chunk=128, seed=55),
              out_dtype="bf16")


def test_eq6_qwen3_dims_ragged():
    check_eq6(BASE.scaled(batch=1, seq=4500, d_model=1024, d_ff=3072, chunk=1024, seed=56))


def test_eq6_equal_paths_write_nothing():
    from dual_window_attention_amd import ttcd
    cfg = BASE.scaled(batch=1, seq=256, d_model=64, d_ff=128, chunk=64, seed=57)
    z = I.hidden_activations(cfg)
    w = I.layer_weights(cfg)
    zt = I.to_torch(z["z_t"])
    w0 = I.to_torch(w["w_down0"])
    _, st = ttcd.fastweight_scan_eq6(zt, zt, zt, w0, I.f32_to_torch(I.beta_for(cfg)), cfg.chunk,
                                     want_state=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(st)[0], w["w_down0"].f64())


def test_eq6_qwen3_64k_full():
    """The 64K workload's fast-weight shapes at full length: sampled rows of
    every chunk and the final state against the oracle."""
    from dual_window_attention_amd import ttcd
    cfg = BASE
    say(f"eq6 full {cfg.name} T={cfg.seq} C={cfg.chunk}")
    z = I.hidden_activations(cfg)
    w = I.layer_weights(cfg)
    beta = eq6_beta(cfg, z["z_s"].f64())
    zt, zs = I.to_torch(z["z_t"]), I.to_torch(z["z_s"])
    y, st = ttcd.fastweight_scan_eq6(zt, zs, zt, I.to_torch(w["w_down0"]), I.f32_to_torch(beta),
                                     cfg.chunk, want_state=True)
    torch.cuda.synchronize()
    rows = np.arange(7, cfg.seq, 331)
    y = to_np(y)[0, rows]
    st = to_np(st)[0]
    del zt, zs
    torch.cuda.empty_cache()
    ref = O.fastweight_scan_eq6(z["z_t"].f64(), z["z_s"].f64(), z["z_t"].f64(),
                                w["w_down0"].f64(), beta.astype(np.float64), cfg.chunk)
    assert_close(y, ref["y"][0, rows], tol_for(cfg.dtype), f"y on {len(rows)} sampled rows")
    assert_close(st, ref["state"][0], tol_for(cfg.dtype), "state after all 64 writes")
