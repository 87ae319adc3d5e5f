"""The decode-time fast-weight stream on the GPU: the per-token append
(conv over a history, residual r, unit key k) against the oracle, and a
multi-step generation that grows the chunk lists across chunk boundaries
and reproduces the prefill oracle's rows."""
import numpy as np
import pytest

from dual_window_attention_amd import inputs as I
from oracle import ttcd_oracle as O
from tests.gpu_helpers import assert_close, say, to_np, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()


@pytest.mark.parametrize("kc", [1, 3, 4])
def test_decode_append_matches_oracle(kc):
    """r and k land in row 2 of chunk-list-like buffers (row stride > width);
    the histories advance by exactly one row."""
    from dual_window_attention_amd import ttcd
    say(f"decode append kc={kc}")
    rng = np.random.default_rng(40 + kc)
    B, d, f = 3, 128, 256
    z_t, z_s = rng.standard_normal((B, f)), rng.standard_normal((B, f))
    h_t, h_s = rng.standard_normal((B, kc - 1, f)), rng.standard_normal((B, kc - 1, f))
    c_t, c_s = rng.standard_normal((f, kc)) / np.sqrt(kc), rng.standard_normal((f, kc)) / np.sqrt(kc)
    w0 = rng.standard_normal((d, f)) / np.sqrt(f)
    wp = rng.standard_normal((f, f)) / np.sqrt(f)
    dz_t, dz_s, dh_t, dh_s = _bf16(z_t), _bf16(z_s), _bf16(h_t), _bf16(h_s)
    dc_t, dc_s, dw0, dwp = _bf16(c_t), _bf16(c_s), _bf16(w0), _bf16(wp)
    f64 = lambda t: to_np(t)
    m = ttcd.fastweight_residual_proj(dw0, dwp)
    r_buf = torch.zeros((B, 5, d), dtype=torch.bfloat16, device="cuda")
    k_buf = torch.zeros((B, 5, f), dtype=torch.bfloat16, device="cuda")
    h_t0, h_s0 = dh_t.clone(), dh_s.clone()
    ttcd.fastweight_decode_append(dz_t, dz_s, dh_t, dh_s, dc_t, dc_s, m, r_buf[:, 2], k_buf[:, 2])
    torch.cuda.synchronize()
    r, k, dbar, nh_t, nh_s = O.decode_append(f64(dz_t), f64(dz_s), f64(h_t0), f64(h_s0),
                                             f64(dc_t), f64(dc_s), f64(dw0), f64(dwp))
    assert_close(to_np(r_buf[:, 2]), r, tol_for("bf16"), "r")
    assert_close(to_np(k_buf[:, 2]), k, tol_for("bf16"), "k")
    assert np.abs(to_np(k_buf[:, 2])).max() < 1.0
    for row in (0, 1, 3, 4):
        assert not r_buf[:, row].any() and not k_buf[:, row].any()
    if kc > 1:
        assert torch.equal(dh_t[:, :-1], h_t0[:, 1:]) and torch.equal(dh_t[:, -1], dz_t)
        assert torch.equal(dh_s[:, :-1], h_s0[:, 1:]) and torch.equal(dh_s[:, -1], dz_s)


def test_hip_prefill_then_generation_across_chunk_boundaries():
    """A ragged HIP prefill (L0 % C != 0) hands over to HIP decode steps:
    the prefill's list outputs (r, k), its Z rows (conv histories) and its
    weight after the complete chunks are the decode's starting state, with
    nothing taken from the oracle.  Each generated token's output and its
    appended (r, k) must equal the rows of one oracle prefill over the whole
    sequence, in both state forms (the lists, and a dense weight refolded
    whenever a chunk completes)."""
    from dual_window_attention_amd import ttcd
    cfg = I.CONFIGS[3].scaled(batch=2, seq=106, n_q_heads=4, n_kv_heads=2, d_model=128,
                              d_ff=256, w_teacher=48, w_student=12, chunk=32, seed=46)
    T, C, kc = cfg.seq, cfg.chunk, cfg.conv_k
    L0 = 2 * C - 6                                   # the prefill ends inside chunk 1
    att = I.attention_inputs(cfg)
    w = I.layer_weights(cfg)
    beta = I.beta_for(cfg)
    x = I.residual_input(cfg)
    wo = {k_: t.f64() for k_, t in w.items()}
    wo["beta"] = beta.astype(np.float64)
    say("  oracle prefill over the whole sequence")
    ref = O.layer_forward(att["q"].f64(), att["k"].f64(), att["v"].f64(), x.f64(), wo,
                          cfg.w_teacher, cfg.w_student, C)
    q, k, v = (I.to_torch(att[n_]) for n_ in ("q", "k", "v"))
    xd = I.to_torch(x)
    wd = {n_: I.to_torch(t) for n_, t in w.items()}
    beta_dev = I.f32_to_torch(beta)
    tol = tol_for(cfg.dtype)
    B, d, f = cfg.batch, cfg.d_model, cfg.d_ff

    say(f"  HIP prefill of {L0} tokens (chunk {C})")
    wp = dict(wd)
    wp["beta"] = beta_dev[:, :-(-L0 // C)].contiguous()
    out0, aux0 = ttcd.layer_forward(q[:, :L0].contiguous(), k[:, :L0].contiguous(),
                                    v[:, :L0].contiguous(), xd[:, :L0].contiguous(), wp,
                                    cfg.w_teacher, cfg.w_student, C, aux=True)
    torch.cuda.synchronize()
    assert_close(to_np(out0), ref["out"][:, :L0], tol, "prefill out")
    assert_close(to_np(aux0["r"]), ref["r"][:, :L0], tol, "prefill r")
    assert_close(to_np(aux0["k"]), ref["k"][:, :L0], tol, "prefill k")
    n0 = L0 // C
    want0 = O.fold_lists(wo["w_down0"], ref["r"][:, :n0 * C], ref["k"][:, :n0 * C],
                         beta[:, :n0].astype(np.float64), C)
    assert_close(to_np(aux0["state_out"]), want0, tol, f"prefill weight after {n0} chunk(s)")

    nmax = (T + C - 1) // C
    r_buf = torch.zeros((B, nmax * C, d), dtype=torch.bfloat16, device="cuda")
    k_buf = torch.zeros((B, nmax * C, f), dtype=torch.bfloat16, device="cuda")
    r_buf[:, :L0] = aux0["r"]
    k_buf[:, :L0] = aux0["k"]
    h_t = aux0["z_teacher"][:, L0 - (kc - 1):L0].contiguous()
    h_s = aux0["z_student"][:, L0 - (kc - 1):L0].contiguous()
    dense = aux0["state_out"].clone()
    dense_n = n0
    m = ttcd.fastweight_residual_proj(wd["w_down0"], wd["w_proj"])
    for t in range(L0, T):
        n = t // C                                   # chunks complete before t
        if n > dense_n:                              # a chunk completed: refold
            dense = ttcd.fastweight_fold(wd["w_down0"], r_buf[:, :n * C].contiguous(),
                                         k_buf[:, :n * C].contiguous(),
                                         beta_dev[:, :n].contiguous(), C)
            dense_n = n
        dec = {"pos": t, "beta_list": beta_dev[:, :n].contiguous()}
        if n > 0:
            dec["r_list"] = r_buf[:, :n * C].contiguous()
            dec["k_list"] = k_buf[:, :n * C].contiguous()
        qt, xt = q[:, t:t + 1].contiguous(), xd[:, t:t + 1].contiguous()
        out_d = ttcd.layer_forward(qt, k, v, xt, wd, cfg.w_teacher, cfg.w_student, C,
                                   decode={"pos": t, "state_dense": dense,
                                           "beta_list": beta_dev[:, :n].contiguous()})
        out, aux = ttcd.layer_forward(qt, k, v, xt, wd, cfg.w_teacher, cfg.w_student, C,
                                      aux=True, decode=dec)
        ttcd.fastweight_decode_append(aux["z_teacher"][:, 0], aux["z_student"][:, 0], h_t, h_s,
                                      wd["conv_t"], wd["conv_s"], m, r_buf[:, t], k_buf[:, t])
        torch.cuda.synchronize()
        assert_close(to_np(out)[:, 0], ref["out"][:, t], tol, f"step {t}: out (lists)")
        assert_close(to_np(out_d)[:, 0], ref["out"][:, t], tol, f"step {t}: out (dense)")
        assert_close(to_np(r_buf[:, t]), ref["r"][:, t], tol, f"step {t}: r")
        assert_close(to_np(k_buf[:, t]), ref["k"][:, t], tol, f"step {t}: k")
    # the lists folded once give the oracle's weight after the complete chunks
    n = T // C
    folded = ttcd.fastweight_fold(wd["w_down0"], r_buf[:, :n * C].contiguous(),
                                  k_buf[:, :n * C].contiguous(), beta_dev[:, :n].contiguous(), C)
    torch.cuda.synchronize()
    assert_close(to_np(folded), ref["state_complete"], tol, "folded state")
