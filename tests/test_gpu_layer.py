"""The whole IP-TTCD layer forward on the GPU against the fp64 oracle."""
import numpy as np
import pytest

from dual_window_attention_amd import inputs as I
from oracle import ttcd_oracle as O
from tests.gpu_helpers import assert_close, assert_correction, say, to_np, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def run_layer(cfg, main_path="teacher", aux=True, chunk_mean=False):
    from dual_window_attention_amd import ttcd
    att = I.attention_inputs(cfg)
    w = I.layer_weights(cfg)
    beta = I.beta_for(cfg, chunk_mean=chunk_mean)
    x = I.residual_input(cfg)
    q, k, v = (I.to_torch(att[n]) for n in ("q", "k", "v"))
    wd = {n: I.to_torch(t) for n, t in w.items()}
    wd["beta"] = I.f32_to_torch(beta)
    res = ttcd.layer_forward(q, k, v, I.to_torch(x), wd, cfg.w_teacher, cfg.w_student, cfg.chunk,
                             main_path=main_path, aux=aux)
    torch.cuda.synchronize()
    wo = {n: t.f64() for n, t in w.items()}
    wo["beta"] = beta.astype(np.float64)
    return res, (att, wo, x)


def oracle_layer(cfg, att, wo, x, main_path="teacher"):
    return O.layer_forward(att["q"].f64(), att["k"].f64(), att["v"].f64(), x.f64(), wo,
                           cfg.w_teacher, cfg.w_student, cfg.chunk, main_path=main_path)


def check_layer(cfg, main_path="teacher", chunk_mean=False):
    say(f"layer {cfg.name} T={cfg.seq} main={main_path} chunk_mean={chunk_mean}: GPU")
    (out, aux), (att, wo, x) = run_layer(cfg, main_path, chunk_mean=chunk_mean)
    say("  oracle")
    ref = oracle_layer(cfg, att, wo, x, main_path)
    say(f"  oracle magnitudes: max|out|={np.abs(ref['out']).max():.3g} "
        f"max|y|={np.abs(ref['y']).max():.3g} max|S_n|={np.abs(ref['state_complete']).max():.3g}")
    tol = tol_for(cfg.dtype)
    assert_close(to_np(out), ref["out"], tol, "out")
    assert_close(to_np(aux["o_teacher"]), ref["o_t"], tol, "O_teacher")
    assert_close(to_np(aux["o_student"]), ref["o_s"], tol, "O_student")
    assert_close(to_np(aux["z_teacher"]), ref["z_t"], tol, "Z_teacher")
    assert_close(to_np(aux["z_student"]), ref["z_s"], tol, "Z_student")
    assert_close(to_np(aux["y"]), ref["y"], tol, "y (fast-weight MLP output)")
    # the fast-weight correction alone (y - W0 z)
    zm = ref["z_t"] if main_path == "teacher" else ref["z_s"]
    corr_ref = ref["y"] - zm @ wo["w_down0"].T
    corr = to_np(aux["y"]) - to_np(aux["z_teacher" if main_path == "teacher" else "z_student"]) @ wo["w_down0"].T
    assert_correction(corr, corr_ref, ref["y"], cfg.chunk, cfg.dtype)
    # the low-rank chunk lists and the weight after the complete chunks
    assert_close(to_np(aux["r"]), ref["r"], tol, "r (list residuals)")
    assert_close(to_np(aux["k"]), ref["k"], tol, "k (list unit keys)")
    st = to_np(aux["state_out"])
    assert_close(st, ref["state_complete"], tol, f"state after the {cfg.seq // cfg.chunk} complete chunks")
    # the launch configuration of a plain call: O and Z stay in the
    # workspace and both paths' products run as one launch each
    say("  GPU, O and Z internal")
    (out2, aux2), _ = run_layer(cfg, main_path, chunk_mean=chunk_mean, aux="fw")
    assert_close(to_np(out2), ref["out"], tol, "out (O, Z internal)")
    assert_close(to_np(aux2["y"]), ref["y"], tol, "y (O, Z internal)")
    assert_close(to_np(aux2["r"]), ref["r"], tol, "r (O, Z internal)")
    assert_close(to_np(aux2["k"]), ref["k"], tol, "k (O, Z internal)")
    assert_close(to_np(aux2["state_out"]), ref["state_complete"], tol, "state (O, Z internal)")


def test_tiny_fp32_layer():
    check_layer(I.CONFIGS[1])


def test_small_bf16_layer_ragged_chunks():
    cfg = I.CONFIGS[3].scaled(batch=2, seq=700, n_q_heads=4, n_kv_heads=2, d_model=256,
                              d_ff=384, w_teacher=300, w_student=40, chunk=128, seed=11)
    check_layer(cfg)


def test_small_bf16_layer_chunk_mean_writes():
    """beta_i = u_i / |C_i|: the correction is a small part of y and is
    checked on its own."""
    cfg = I.CONFIGS[3].scaled(batch=1, seq=1100, n_q_heads=4, n_kv_heads=2, d_model=256,
                              d_ff=512, w_teacher=400, w_student=64, chunk=256, seed=14)
    check_layer(cfg, chunk_mean=True)


def test_small_bf16_layer_student_main_path():
    cfg = I.CONFIGS[2].scaled(seq=640, d_model=192, d_ff=256, w_teacher=256, w_student=32,
                              chunk=128, seed=12)
    check_layer(cfg, main_path="student")


def test_small_chunk_uses_generic_apply():
    cfg = I.CONFIGS[3].scaled(seq=300, n_q_heads=2, n_kv_heads=1, d_model=64, d_ff=96,
                              w_teacher=90, w_student=10, chunk=48, seed=13)
    check_layer(cfg)


def test_smollm2_shapes_ragged_sequence():
    """The SmolLM2-shaped layer over 12000 tokens: the SwiGLU and apply
    GEMMs take 256 x 256 tiles with a ragged last row tile."""
    check_layer(I.CONFIGS[2].scaled(seq=12000, seed=15))


def test_qwen3_dims_8k_student_main_path():
    """Qwen3 dims over 8192 tokens with the student as the main path: the
    joint output projection and SwiGLU of both paths take the 256 x 256 tile
    path, and the student half of h feeds the output."""
    cfg = I.CONFIGS[3].scaled(seq=8192, w_teacher=1024, w_student=128, seed=17)
    check_layer(cfg, main_path="student")


def test_smollm2_16k_layer_full():
    check_layer(I.CONFIGS[2])


def test_qwen3_64k_layer_full_against_stored_oracle_rows():
    """The 64K workload at full size, in the launch configuration of the
    benchmark, against oracle rows written by tests/golden/make_layer_golden.py."""
    from dual_window_attention_amd import ttcd
    from tests.golden import make_layer_golden as G
    ref = np.load(G.OUT)
    cfg = I.CONFIGS[3]
    say("layer qwen3 64K: inputs")
    att = I.attention_inputs(cfg)
    w = I.layer_weights(cfg)
    beta = I.beta_for(cfg)
    x = I.residual_input(cfg)
    fp = G.fingerprint({"q": att["q"].f64(),
                        "k": att["k"].f64(), "v": att["v"].f64(), "x": x.f64(),
                        **{n: t.f64() for n, t in w.items()}, "beta": beta.astype(np.float64)})
    for n, a in fp.items():
        np.testing.assert_allclose(a, ref[n], rtol=1e-12, err_msg=f"stored rows are stale ({n})")
    q, k, v = (I.to_torch(att[n]) for n in ("q", "k", "v"))
    del att
    wd = {n: I.to_torch(t) for n, t in w.items()}
    wd["beta"] = I.f32_to_torch(beta)
    xd = I.to_torch(x)
    rows = torch.from_numpy(ref["rows"]).cuda()
    tol = tol_for(cfg.dtype)
    say(f"  stored magnitudes: max|out|={np.abs(ref['out']).max():.3g} "
        f"max|y|={np.abs(ref['y']).max():.3g} max|S| (sampled)={np.abs(ref['state']).max():.3g}")
    say("  GPU, benchmark launch configuration (no intermediates)")
    out = ttcd.layer_forward(q, k, v, xd, wd, cfg.w_teacher, cfg.w_student, cfg.chunk)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    assert_close(to_np(out[0, rows]), ref["out"], tol, "out (sampled rows)")
    del out
    say("  GPU, with intermediates")
    out, aux = ttcd.layer_forward(q, k, v, xd, wd, cfg.w_teacher, cfg.w_student, cfg.chunk,
                                  aux=True)
    torch.cuda.synchronize()
    assert_close(to_np(out[0, rows]), ref["out"], tol, "out (sampled rows)")
    assert_close(to_np(aux["y"][0, rows]), ref["y"], tol, "y (sampled rows)")
    assert_close(to_np(aux["o_teacher"][0, rows]).reshape(len(rows), -1),
                 ref["o_t"].reshape(len(rows), -1), tol, "O_teacher")
    assert_close(to_np(aux["o_student"][0, rows]).reshape(len(rows), -1),
                 ref["o_s"].reshape(len(rows), -1), tol, "O_student")
    assert_close(to_np(aux["lse_teacher"][0][:, rows]), ref["lse_t"], (1e-3, 1e-5), "LSE_T")
    assert_close(to_np(aux["lse_student"][0][:, rows]), ref["lse_s"], (1e-3, 1e-5), "LSE_S")
    assert_close(to_np(aux["z_teacher"][0, rows]), ref["z_t"], tol, "Z_teacher")
    assert_close(to_np(aux["z_student"][0, rows]), ref["z_s"], tol, "Z_student")
    assert_close(to_np(aux["r"][0, rows]), ref["r"], tol, "r (sampled rows)")
    assert_close(to_np(aux["k"][0, rows]), ref["k"], tol, "k (sampled rows)")
    si = torch.from_numpy(ref["state_i"]).cuda()
    sj = torch.from_numpy(ref["state_j"]).cuda()
    assert_close(to_np(aux["state_out"][0, si, sj]), ref["state"], tol, "final state (sampled)")


def test_layer_deterministic_run_to_run():
    """The whole layer (both paths through the joint GEMMs, the stream, the
    K-sliced M = W_down0 W_proj, the prefix) gives the same bits twice, at
    Qwen3 widths over a ragged 2.5 chunks."""
    from dual_window_attention_amd import ttcd
    cfg = I.CONFIGS[3].scaled(seq=2560, w_teacher=1024, w_student=128, seed=93)
    say(f"layer determinism T={cfg.seq} d={cfg.d_model} f={cfg.d_ff}")
    att = I.attention_inputs(cfg)
    w = I.layer_weights(cfg)
    q, k, v = (I.to_torch(att[n]) for n in ("q", "k", "v"))
    wd = {n: I.to_torch(t) for n, t in w.items()}
    wd["beta"] = I.f32_to_torch(I.beta_for(cfg))
    x = I.to_torch(I.residual_input(cfg))

    def run():
        out = ttcd.layer_forward(q, k, v, x, wd, cfg.w_teacher, cfg.w_student, cfg.chunk)
        torch.cuda.synchronize()
        return out.clone()

    assert torch.equal(run(), run())
