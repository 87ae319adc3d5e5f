"""ttcd_fastweight_scan_backward on the GPU against the fp64 oracle's
gradient of the fast-weight scan."""
import numpy as np
import pytest

from dual_window_attention_amd import inputs as I
from oracle import ttcd_oracle as O
from tests.gpu_helpers import U_BF16, assert_close, errors, say, to_np, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BASE = I.CONFIGS[3]


def dbeta_sigma(z_t, z_s, z_main, conv_t, conv_s, w0, wp, dy, C, eps=1e-12):
    """First-order spread of dbeta [B, n] under the bf16 storage of the
    fast-weight stream's outputs.

    dbeta_j = sum_{t in C_j} r_t . (G_j k_t) is an inner product whose terms
    cancel, so its error is not a fraction of its value.  The path stores
    dbar (r_t = M dbar_t) and the unit keys k_t (from bf16 zbar_S) in bf16,
    as the forward does; M and G_j it carries to fp32 accuracy.  Each
    rounding is an independent relative perturbation of RMS at most u/sqrt 3
    per element, so to first order
        var(dbeta_j) <= u^2/3 [ sum_{t,f} (dbar_t[f] (M^T G_j k_t)[f])^2
                              + 2 sum_{t,f} (k_t[f] (G_j^T r_t)[f])^2 ]
    (the key term counts twice: zbar_S and then k are rounded)."""
    B, T, _ = z_t.shape
    bounds = O.chunk_bounds(T, C)
    M = w0 @ wp
    sig = np.zeros((B, len(bounds)))
    for b in range(B):
        dbar = O.causal_depthwise_conv(z_t[b], conv_t) - O.causal_depthwise_conv(z_s[b], conv_s)
        k = O.l2_normalize(O.causal_depthwise_conv(z_s[b], conv_s), eps)
        r = dbar @ M.T
        G = np.zeros_like(w0)
        for j in range(len(bounds) - 1, -1, -1):
            a, e = bounds[j]
            P = k[a:e] @ G.T
            td = np.sum((dbar[a:e] * (P @ M)) ** 2)
            tk = np.sum((k[a:e] * (r[a:e] @ G)) ** 2)
            sig[b, j] = U_BF16 / np.sqrt(3.0) * np.sqrt(td + 2.0 * tk)
            G = G + dy[b, a:e].T @ z_main[b, a:e]
    return sig


def assert_dbeta(got, ref, sig):
    """|err_j| <= 4 sigma_j + 1e-5 max|ref| (the fp32 sums): every entry, so
    the last chunk's (whose write reaches no token: sigma = 0) is exact."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bound = 4.0 * sig + 1e-5 * float(np.abs(ref).max())
    _, rel = errors(got, ref)
    ratio = float(np.max(err / np.where(bound > 0, bound, 1.0)))
    say(f"  dbeta: max|err|/bound={ratio:.3f} max|err|={err.max():.3e} "
        f"relL2={rel:.3e} (bound 4 sigma_j, sigma max {sig.max():.3g})")
    assert np.all(err <= bound), f"dbeta: err {err} bound {bound}"


def check_scan_backward(cfg, main="teacher", out_dtype="f32", chunk_mean=False):
    from dual_window_attention_amd import ttcd
    say(f"scan backward {cfg.dtype} B={cfg.batch} T={cfg.seq} f={cfg.d_ff} d={cfg.d_model} "
        f"C={cfg.chunk} kc={cfg.conv_k} main={main} dz={out_dtype} chunk_mean={chunk_mean}")
    z = I.hidden_activations(cfg)
    w = I.layer_weights(cfg)
    beta = I.beta_for(cfg, chunk_mean=chunk_mean)
    dy = I.normal(cfg.seed, "dy", (cfg.batch, cfg.seq, cfg.d_model), 1.0, cfg.dtype)
    zt, zs = I.to_torch(z["z_t"]), I.to_torch(z["z_s"])
    zm = zt if main == "teacher" else zs
    dev = {n: I.to_torch(w[n]) for n in ("conv_t", "conv_s", "w_down0", "w_proj")}
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    g = ttcd.fastweight_scan_backward(zt, zs, zm, dev["conv_t"], dev["conv_s"], dev["w_down0"],
                                      dev["w_proj"], I.f32_to_torch(beta), I.to_torch(dy),
                                      cfg.chunk, out_dtype=odt)
    torch.cuda.synchronize()
    zm64 = (z["z_t"] if main == "teacher" else z["z_s"]).f64()
    ref = O.fastweight_scan_backward(z["z_t"].f64(), z["z_s"].f64(), zm64, w["conv_t"].f64(),
                                     w["conv_s"].f64(), w["w_down0"].f64(), w["w_proj"].f64(),
                                     beta.astype(np.float64), cfg.chunk, dy.f64())
    tol = tol_for(cfg.dtype)
    for n in ("dz_t", "dz_s", "dz_main", "dconv_t", "dconv_s", "dw_down0", "dw_proj"):
        assert_close(to_np(g[n]), ref[n], tol, n)
    if cfg.dtype == "bf16":
        sig = dbeta_sigma(z["z_t"].f64(), z["z_s"].f64(), zm64, w["conv_t"].f64(),
                          w["conv_s"].f64(), w["w_down0"].f64(), w["w_proj"].f64(), dy.f64(),
                          cfg.chunk)
        assert_dbeta(to_np(g["dbeta"]), ref["dbeta"], sig)
    else:
        assert_close(to_np(g["dbeta"]), ref["dbeta"], tol, "dbeta")
    return g


@pytest.mark.parametrize("case", [
    dict(dtype="f32", batch=1, seq=300, d_model=64, d_ff=96, chunk=64, conv_k=4, seed=81),
    dict(dtype="bf16", batch=2, seq=517, d_model=128, d_ff=256, chunk=128, conv_k=1, seed=82),
    dict(dtype="bf16", batch=1, seq=1024, d_model=256, d_ff=384, chunk=256, conv_k=3, seed=83),
    dict(dtype="bf16", batch=2, seq=700, d_model=96, d_ff=160, chunk=48, conv_k=8, seed=84),
    dict(dtype="f32", batch=2, seq=333, d_model=64, d_ff=128, chunk=32, conv_k=7, seed=85),
], ids=["f32-kc4", "bf16-kc1-B2-ragged", "bf16-kc3", "bf16-kc8-chunk48", "f32-kc7-chunk32"])
def test_scan_backward_small(case):
    check_scan_backward(BASE.scaled(**case))


def test_scan_backward_student_main_bf16_grads_and_chunk_mean():
    cfg = BASE.scaled(batch=1, seq=640, d_model=128, d_ff=256, chunk=128, seed=86)
    check_scan_backward(cfg, main="student", out_dtype="bf16")
    check_scan_backward(cfg, chunk_mean=True)


def test_scan_backward_single_chunk():
    """T <= C: nothing is written; only W_down0 and z_main get gradients."""
    g = check_scan_backward(BASE.scaled(batch=2, seq=100, d_model=64, d_ff=128, chunk=128,
                                        seed=87))
    for n in ("dz_t", "dz_s", "dconv_t", "dconv_s", "dw_proj"):
        assert not g[n].any().item(), n


def test_scan_backward_qwen3_fast_weight_shapes():
    """d_model 1024, d_ff 3072, chunk 1024 over 4.5 chunks (ragged tail)."""
    check_scan_backward(BASE.scaled(batch=1, seq=4608, seed=88))


def test_scan_backward_qwen3_16_chunks():
    """The 64K layer's fast-weight shapes over 16 chunks of 1024 tokens."""
    check_scan_backward(BASE.scaled(batch=1, seq=16384, seed=89))


def test_scan_backward_deterministic_run_to_run():
    """Every reduction of the gradient (chunk suffix, the K-sliced dM, the
    tap partials, dbeta) runs in a fixed order: two calls on the same inputs
    agree bit for bit."""
    from dual_window_attention_amd import ttcd
    cfg = BASE.scaled(batch=2, seq=1100, d_model=128, d_ff=256, chunk=128, conv_k=4, seed=90)
    say(f"scan backward determinism B={cfg.batch} T={cfg.seq}")
    z = I.hidden_activations(cfg)
    w = I.layer_weights(cfg)
    beta = I.f32_to_torch(I.beta_for(cfg))
    dy = I.to_torch(I.normal(cfg.seed, "dy", (cfg.batch, cfg.seq, cfg.d_model), 1.0, cfg.dtype))
    zt, zs = I.to_torch(z["z_t"]), I.to_torch(z["z_s"])
    dev = {n: I.to_torch(w[n]) for n in ("conv_t", "conv_s", "w_down0", "w_proj")}

    def run():
        g = ttcd.fastweight_scan_backward(zt, zs, zt, dev["conv_t"], dev["conv_s"],
                                          dev["w_down0"], dev["w_proj"], beta, dy, cfg.chunk,
                                          out_dtype=torch.float32)
        torch.cuda.synchronize()
        return g

    a, b = run(), run()
    for n in a:
        assert torch.equal(a[n], b[n]), n
