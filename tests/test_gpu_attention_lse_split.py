"""The LSE-combination path of the dual-window attention (student call,
shifted far-band call, exact merge; README "Fused inference kernels") on
the GPU, against the fp64 oracle and against the fused kernel."""
import numpy as np
import pytest

from dual_window_attention_amd import inputs as I
from oracle import ttcd_oracle as O
from tests.gpu_helpers import assert_close, attn_tensors, say, to_np, tol_for
from tests.test_gpu_attention import CASES, _sample_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _split(att, wT, wS, out_dtype=None):
    from dual_window_attention_amd import ttcd
    q, k, v = (I.to_torch(att[n]) for n in ("q", "k", "v"))
    res = ttcd.dual_window_attn_lse_split(q, k, v, wT, wS, out_dtype=out_dtype or torch.float32)
    torch.cuda.synchronize()
    return res


def _fused(att, wT, wS, out_dtype=None):
    from dual_window_attention_amd import ttcd
    q, k, v = (I.to_torch(att[n]) for n in ("q", "k", "v"))
    res = ttcd.dual_window_attn(q, k, v, wT, wS, out_dtype=out_dtype or torch.float32)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_T{}_H{}/{}_D{}_w{}/{}_{}".format(*c))
def test_lse_split_matches_oracle(case):
    B, T, Hq, Hkv, D, wT, wS, dt = case
    say(f"lse-split case {case}")
    att = attn_tensors(B, T, Hq, Hkv, D, dt, seed=T + Hq)
    o_t, o_s, l_t, l_s = _split(att, wT, wS)
    r_t, r_s, rl_t, rl_s = O.dual_window_attention(att["q"].f64(), att["k"].f64(),
                                                   att["v"].f64(), wT, wS)
    tol = tol_for(dt)
    assert_close(to_np(o_t), r_t, tol, "O_teacher")
    assert_close(to_np(o_s), r_s, tol, "O_student")
    ltol = (1e-3, 1e-4) if dt == "bf16" else (1e-4, 1e-6)
    assert_close(to_np(l_t), rl_t, ltol, "LSE_teacher")
    assert_close(to_np(l_s), rl_s, ltol, "LSE_student")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_lse_split_agrees_with_fused(dt):
    """Both paths compute the same function.  The student outputs come from
    the same kernel walk and are bitwise equal; the teacher outputs differ
    by the rounding of P (bf16 P is formed against a different running max
    in each band) and of the merge, so they are held to the bound each path
    meets against the oracle."""
    say(f"lse-split vs fused {dt}")
    D = 128 if dt == "bf16" else 64
    att = attn_tensors(2, 900, 4, 2, D, dt, seed=11)
    a = _split(att, 300, 40)
    b = _fused(att, 300, 40)
    assert torch.equal(a[1], b[1]) and torch.equal(a[3], b[3])
    assert_close(to_np(a[0]), to_np(b[0]), tol_for(dt), "O_teacher split vs fused")
    ltol = (1e-3, 1e-4) if dt == "bf16" else (1e-4, 1e-6)
    assert_close(to_np(a[2]), to_np(b[2]), ltol, "LSE_teacher split vs fused")


def test_lse_split_without_far_band_copies_the_student():
    say("lse-split, w_T == w_S")
    att = attn_tensors(1, 400, 4, 2, 128, "bf16", seed=5)
    o_t, o_s, l_t, l_s = _split(att, 64, 64, torch.bfloat16)
    assert torch.equal(o_t, o_s) and torch.equal(l_t, l_s)


@pytest.mark.parametrize("D", [64, 128])
def test_lse_split_extreme_score_range(D):
    """Queries scaled x40: the two partial LSEs differ by hundreds of nats
    for some rows, so one side's weight underflows; the merge stays exact."""
    say(f"lse-split extreme score range D={D}")
    att = attn_tensors(1, 300, 4, 2, D, "bf16", seed=77)
    q32 = I.bf16_bits_to_f32(att["q"].data) * np.float32(40.0)
    att["q"] = I.Tensor(I.f32_to_bf16_bits(q32), "bf16")
    o_t, o_s, l_t, l_s = _split(att, 200, 40)
    r_t, r_s, rl_t, rl_s = O.dual_window_attention(att["q"].f64(), att["k"].f64(),
                                                   att["v"].f64(), 200, 40)
    tol = tol_for("bf16")
    assert_close(to_np(o_t), r_t, tol, "O_teacher")
    assert_close(to_np(o_s), r_s, tol, "O_student")
    assert_close(to_np(l_t), rl_t, (2e-3, 1e-5), "LSE_teacher")
    assert_close(to_np(l_s), rl_s, (2e-3, 1e-5), "LSE_student")


def test_lse_split_qwen3_64k_sampled_rows():
    """The 64K Qwen3 workload in the configuration the benchmark times (bf16
    outputs), checked on sampled rows against the oracle."""
    from dual_window_attention_amd import ttcd
    cfg = I.CONFIGS[3]
    say(f"lse-split full size {cfg.name}: generating inputs")
    att = I.attention_inputs(cfg)
    q, k, v = (I.to_torch(att[n]) for n in ("q", "k", "v"))
    wT, wS = cfg.w_teacher, cfg.w_student
    say("  GPU run")
    o_t, o_s, l_t, l_s = ttcd.dual_window_attn_lse_split(q, k, v, wT, wS, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.isfinite(o_t.float()).all() and torch.isfinite(l_t).all()
    rows = _sample_rows(cfg.seq, wT, wS, 30, seed=wT + 1)
    qf, kf, vf = (att[n].f64() for n in ("q", "k", "v"))
    r_t, r_s, rl_t, rl_s = O.dual_window_attention(qf, kf, vf, wT, wS, rows=rows)
    sel = np.asarray(rows)
    assert_close(to_np(o_t[0, sel]), r_t[0, sel], tol_for("bf16"), "O_teacher rows")
    assert_close(to_np(o_s[0, sel]), r_s[0, sel], tol_for("bf16"), "O_student rows")
    assert_close(to_np(l_t[0][:, sel]), rl_t[0][:, sel], (1e-3, 1e-4), "LSE_T rows")
    assert_close(to_np(l_s[0][:, sel]), rl_s[0][:, sel], (1e-3, 1e-4), "LSE_S rows")
