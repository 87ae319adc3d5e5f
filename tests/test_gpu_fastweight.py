"""ttcd_fastweight_scan and ttcd_fastweight_fold on the GPU against the fp64 oracle."""
import numpy as np
import pytest

from dual_window_attention_amd import inputs as I
from oracle import ttcd_oracle as O
from tests.gpu_helpers import assert_close, assert_correction, say, to_np, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def scan_inputs(cfg, chunk_mean=False):
    z = I.hidden_activations(cfg)
    w = I.layer_weights(cfg)
    beta = I.beta_for(cfg, chunk_mean=chunk_mean)
    return z, w, beta


def check_scan(cfg, main="teacher", out_dtype="f32", chunk_mean=False, lists=True):
    from dual_window_attention_amd import ttcd
    say(f"scan {cfg.name} {cfg.dtype} B={cfg.batch} T={cfg.seq} f={cfg.d_ff} d={cfg.d_model} "
        f"C={cfg.chunk} kc={cfg.conv_k} main={main} y={out_dtype} chunk_mean={chunk_mean}")
    z, w, beta = scan_inputs(cfg, chunk_mean)
    zt, zs = I.to_torch(z["z_t"]), I.to_torch(z["z_s"])
    zm = zt if main == "teacher" else zs
    dev = {n: I.to_torch(w[n]) for n in ("conv_t", "conv_s", "w_down0", "w_proj")}
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    B, T, f = zt.shape
    r_out = torch.empty((B, T, cfg.d_model), dtype=zt.dtype, device="cuda") if lists else None
    k_out = torch.empty((B, T, f), dtype=zt.dtype, device="cuda") if lists else None
    y, st = ttcd.fastweight_scan(zt, zs, zm, dev["conv_t"], dev["conv_s"], dev["w_down0"],
                                 dev["w_proj"], I.f32_to_torch(beta), cfg.chunk, out_dtype=odt,
                                 want_state=True, r_out=r_out, k_out=k_out)
    torch.cuda.synchronize()
    ref = O.fastweight_scan(z["z_t"].f64(), z["z_s"].f64(),
                            (z["z_t"] if main == "teacher" else z["z_s"]).f64(),
                            w["conv_t"].f64(), w["conv_s"].f64(), w["w_down0"].f64(),
                            w["w_proj"].f64(), beta.astype(np.float64), cfg.chunk)
    say(f"  oracle magnitudes: max|y|={np.abs(ref['y']).max():.3g} "
        f"max|S_n|={np.abs(ref['state_complete']).max():.3g}")
    tol = tol_for(cfg.dtype)
    assert_close(to_np(y), ref["y"], tol, f"y ({out_dtype} out)")
    assert_close(to_np(st), ref["state_complete"], tol,
                 f"state after the {cfg.seq // cfg.chunk} complete chunks")
    if lists:
        assert_close(to_np(r_out), ref["r"], tol, "r (list residuals)")
        assert_close(to_np(k_out), ref["k"], tol, "k (list unit keys)")
    # the correction alone, y - W0 z
    w0 = w["w_down0"].f64()
    zm64 = (z["z_t"] if main == "teacher" else z["z_s"]).f64()
    assert_correction(to_np(y) - zm64 @ w0.T, ref["y"] - zm64 @ w0.T, ref["y"], cfg.chunk,
                      cfg.dtype)


BASE = I.CONFIGS[3]


@pytest.mark.parametrize("case", [
    dict(dtype="f32", batch=1, seq=300, d_model=64, d_ff=96, chunk=64, conv_k=4, seed=21),
    dict(dtype="bf16", batch=2, seq=517, d_model=128, d_ff=256, chunk=128, conv_k=1, seed=22),
    dict(dtype="bf16", batch=1, seq=1024, d_model=256, d_ff=384, chunk=256, conv_k=3, seed=23),
    dict(dtype="bf16", batch=2, seq=700, d_model=96, d_ff=160, chunk=48, conv_k=8, seed=24),
    dict(dtype="f32", batch=2, seq=333, d_model=64, d_ff=128, chunk=32, conv_k=7, seed=25),
], ids=["f32-kc4", "bf16-kc1-B2-ragged", "bf16-kc3", "bf16-kc8-chunk48", "f32-kc7-chunk32"])
def test_scan_small(case):
    check_scan(BASE.scaled(**case))


def test_scan_student_main_and_bf16_output():
    cfg = BASE.scaled(batch=1, seq=640, d_model=128, d_ff=256, chunk=128, seed=26)
    check_scan(cfg, main="student")
    check_scan(cfg, out_dtype="bf16")


def test_scan_chunk_mean_writes():
    """beta_i = u_i / |C_i|: a small correction, checked on its own."""
    check_scan(BASE.scaled(batch=2, seq=900, d_model=128, d_ff=256, chunk=128, seed=20),
               chunk_mean=True)


def test_scan_without_lists():
    check_scan(BASE.scaled(batch=1, seq=333, d_model=64, d_ff=128, chunk=64, seed=19),
               lists=False)


def test_scan_qwen3_fast_weight_shapes():
    """d_model 1024, d_ff 3072, chunk 1024 over 4.5 chunks (ragged tail)
    at the workload's beta ~ U(0,1)."""
    check_scan(BASE.scaled(batch=1, seq=4608))


def test_scan_ragged_large_tiles():
    """Shapes that take the 256 x 256 GEMM tiles (the residual projection,
    the chunk writes and the apply) with ragged edges: T % 256 != 0, two
    sequences."""
    check_scan(BASE.scaled(batch=2, seq=20000, seed=18))


def test_scan_single_chunk_is_base_mlp():
    """T <= C: no earlier chunk, y = W_down0 z exactly as the base MLP."""
    check_scan(BASE.scaled(batch=2, seq=100, d_model=64, d_ff=128, chunk=128, seed=27))


def test_scan_zero_student_conv_is_base_mlp():
    """conv_S = 0 makes every key zero: no write reaches any chunk."""
    from dual_window_attention_amd import ttcd
    cfg = BASE.scaled(batch=1, seq=512, d_model=64, d_ff=128, chunk=128, seed=28)
    z, w, beta = scan_inputs(cfg)
    zt, zs = I.to_torch(z["z_t"]), I.to_torch(z["z_s"])
    cz = torch.zeros_like(I.to_torch(w["conv_s"]))
    y, st = ttcd.fastweight_scan(zt, zs, zt, I.to_torch(w["conv_t"]), cz,
                                 I.to_torch(w["w_down0"]), I.to_torch(w["w_proj"]),
                                 I.f32_to_torch(beta), cfg.chunk, want_state=True)
    torch.cuda.synchronize()
    ref = z["z_t"].f64() @ w["w_down0"].f64().T
    assert_close(to_np(y), ref, tol_for(cfg.dtype), "y with zero student conv")
    np.testing.assert_array_equal(to_np(st)[0], w["w_down0"].f64())


def test_scan_equal_paths_write_nothing():
    """Teacher and student identical (same activations, same conv): the
    residual dbar is zero, so no chunk is written, y is the base MLP and the
    weight after the complete chunks is W_down0 exactly (notes on "Learning
    What to Remember", key design 3: the write is driven by the gap)."""
    from dual_window_attention_amd import ttcd
    cfg = BASE.scaled(batch=2, seq=700, d_model=128, d_ff=256, chunk=128, seed=29)
    z, w, beta = scan_inputs(cfg)
    zt = I.to_torch(z["z_t"])
    ct = I.to_torch(w["conv_t"])
    y, st = ttcd.fastweight_scan(zt, zt, zt, ct, ct, I.to_torch(w["w_down0"]),
                                 I.to_torch(w["w_proj"]), I.f32_to_torch(beta), cfg.chunk,
                                 want_state=True)
    torch.cuda.synchronize()
    ref = z["z_t"].f64() @ w["w_down0"].f64().T
    assert_close(to_np(y), ref, tol_for(cfg.dtype), "y with equal paths")
    for b in range(cfg.batch):
        np.testing.assert_array_equal(to_np(st)[b], w["w_down0"].f64())


def test_scan_deterministic():
    from dual_window_attention_amd import ttcd
    cfg = BASE.scaled(batch=1, seq=2048, d_model=256, d_ff=512, chunk=256, seed=29)
    z, w, beta = scan_inputs(cfg)
    args = [I.to_torch(z["z_t"]), I.to_torch(z["z_s"])]
    args.append(args[0])
    args += [I.to_torch(w[n]) for n in ("conv_t", "conv_s", "w_down0", "w_proj")]
    args.append(I.f32_to_torch(beta))
    y1, s1 = ttcd.fastweight_scan(*args, cfg.chunk, want_state=True)
    y2, s2 = ttcd.fastweight_scan(*args, cfg.chunk, want_state=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2)


# ----------------------------------------------------------------------- fold
def check_fold(B, n, C, d, f, dtype, seed):
    from dual_window_attention_amd import ttcd
    cfg = I.CONFIGS[5].scaled(batch=B, cache_len=n * C, chunk=C, d_model=d, d_ff=f,
                              dtype=dtype, seed=seed)
    say(f"fold B={B} n={n} C={C} d={d} f={f} {dtype}")
    lists = [I.decode_lists(cfg, b) for b in range(B)]
    r = np.stack([lr.data for lr, _ in lists])
    k = np.stack([lk.data for _, lk in lists])
    rT = I.Tensor(r, dtype)
    kT = I.Tensor(k, dtype)
    beta = I._rng(seed, "fold_beta").random(size=(B, n)).astype(np.float32)
    w0 = I.layer_weights(cfg)["w_down0"]
    got = ttcd.fastweight_fold(I.to_torch(w0), I.to_torch(rT), I.to_torch(kT),
                               I.f32_to_torch(beta), C)
    torch.cuda.synchronize()
    ref = O.fold_lists(w0.f64(), rT.f64(), kT.f64(), beta.astype(np.float64), C)
    assert_close(to_np(got), ref, tol_for(dtype), "folded dense weight")
    return got


def test_fold_small():
    check_fold(2, 5, 64, 96, 160, "bf16", 31)
    check_fold(1, 3, 32, 64, 128, "f32", 32)


def test_fold_no_chunks_is_w0():
    from dual_window_attention_amd import ttcd
    cfg = I.CONFIGS[5].scaled(batch=2, cache_len=64, chunk=64, d_model=64, d_ff=128, seed=33)
    w0 = I.layer_weights(cfg)["w_down0"]
    e = torch.empty((2, 0, 64), dtype=torch.bfloat16, device="cuda")
    ek = torch.empty((2, 0, 128), dtype=torch.bfloat16, device="cuda")
    got = ttcd.fastweight_fold(I.to_torch(w0), e, ek,
                               torch.empty((2, 0), dtype=torch.float32, device="cuda"), 64)
    torch.cuda.synchronize()
    for b in range(2):
        np.testing.assert_array_equal(to_np(got)[b], w0.f64())


# --------------------------------------------------------------------- stream
def check_stream(cfg):
    from dual_window_attention_amd import ttcd
    say(f"stream {cfg.dtype} B={cfg.batch} T={cfg.seq} f={cfg.d_ff} C={cfg.chunk} kc={cfg.conv_k}")
    z, w, beta = scan_inputs(cfg)
    dbar, zbt, ks = ttcd.fastweight_stream(I.to_torch(z["z_t"]), I.to_torch(z["z_s"]),
                                           I.to_torch(w["conv_t"]), I.to_torch(w["conv_s"]),
                                           I.f32_to_torch(beta), cfg.chunk)
    torch.cuda.synchronize()
    T, Tp = cfg.seq, ttcd.stream_pad(cfg.seq)
    tol = tol_for(cfg.dtype)
    dbar_g, zbt_g, ks_g = to_np(dbar), to_np(zbt), to_np(ks)
    assert not dbar_g[:, T:].any() and not zbt_g[:, :, T:].any() and not ks_g[:, T:].any(), \
        "padding rows must be zero"
    c0 = O.chunk_bounds(T, cfg.chunk)
    for b in range(cfg.batch):
        zb_t = O.causal_depthwise_conv(z["z_t"].f64()[b], w["conv_t"].f64())
        zb_s = O.causal_depthwise_conv(z["z_s"].f64()[b], w["conv_s"].f64())
        assert_close(dbar_g[b, :T], zb_t - zb_s, tol, "dbar")
        assert_close(zbt_g[b, :, :T].T, zb_s, tol, "conv_S(Z_S)")
        nrm = np.maximum(np.linalg.norm(zb_s, axis=-1), 1e-12)
        bt = np.concatenate([np.full(e - a, beta[b, i], dtype=np.float64)
                             for i, (a, e) in enumerate(c0)])
        want = bt / nrm
        rel = np.abs(ks_g[b, :T] - want) / want
        say(f"  key scale: max rel err {rel.max():.3e}")
        assert rel.max() <= 1e-4
        # the scaled keys against beta * l2_normalize(conv_S(Z_S))
        kt = ks_g[b, :T, None] * zbt_g[b, :, :T].T
        kref = bt[:, None] * O.l2_normalize(zb_s, 1e-12)
        err = np.linalg.norm(kt - kref, axis=-1) / np.linalg.norm(kref, axis=-1)
        say(f"  scaled keys: max per-token rel L2 {err.max():.3e}")
        assert err.max() <= (1e-2 if cfg.dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("case", [
    dict(dtype="bf16", batch=2, seq=517, d_ff=384, chunk=128, conv_k=4, seed=51),
    dict(dtype="f32", batch=1, seq=200, d_ff=136, chunk=64, conv_k=3, seed=52),
    dict(dtype="bf16", batch=1, seq=64, d_ff=8, chunk=16, conv_k=8, seed=53),
], ids=["bf16-B2-ragged", "f32-f136", "bf16-f8-kc8"])
def test_stream_small(case):
    check_stream(BASE.scaled(**case))


def test_stream_qwen3_64k_full():
    """The stream step at the 64K workload's full size (T 65536, d_ff 3072)."""
    check_stream(BASE.scaled(batch=1))
