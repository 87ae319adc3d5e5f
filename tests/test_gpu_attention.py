"""Dual-window attention on the GPU against the fp64 oracle (C-ABI path)."""
import numpy as np
import pytest

from dual_window_attention_amd import inputs as I
from oracle import ttcd_oracle as O
from tests.gpu_helpers import assert_close, attn_tensors, say, to_np, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _gpu(att, wT, wS, out_dtype=None):
    from dual_window_attention_amd import ttcd
    q, k, v = (I.to_torch(att[n]) for n in ("q", "k", "v"))
    o_t, o_s, l_t, l_s = ttcd.dual_window_attn(q, k, v, wT, wS,
                                               out_dtype=out_dtype or torch.float32)
    torch.cuda.synchronize()
    return o_t, o_s, l_t, l_s


CASES = [
    # B, T, Hq, Hkv, D, wT, wS, dtype
    (2, 1, 2, 1, 128, 16, 4, "bf16"),
    (2, 37, 2, 1, 128, 42, 1, "bf16"),
    (1, 300, 4, 2, 128, 64, 16, "bf16"),
    (2, 513, 6, 2, 64, 200, 33, "bf16"),
    (1, 700, 15, 5, 64, 256, 64, "bf16"),
    (1, 520, 16, 8, 128, 100, 100, "bf16"),
    (1, 333, 3, 3, 128, 1000, 50, "bf16"),
    (1, 257, 2, 1, 64, 64, 16, "f32"),
    (2, 130, 4, 2, 128, 50, 7, "f32"),
    (1, 1024, 2, 1, 64, 256, 64, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_T{}_H{}/{}_D{}_w{}/{}_{}".format(*c))
def test_attention_matches_oracle(case):
    B, T, Hq, Hkv, D, wT, wS, dt = case
    say(f"attention case {case}")
    att = attn_tensors(B, T, Hq, Hkv, D, dt, seed=T + Hq)
    o_t, o_s, l_t, l_s = _gpu(att, wT, wS)
    r_t, r_s, rl_t, rl_s = O.dual_window_attention(att["q"].f64(), att["k"].f64(),
                                                   att["v"].f64(), wT, wS)
    tol = tol_for(dt)
    assert_close(to_np(o_t), r_t, tol, "O_teacher")
    assert_close(to_np(o_s), r_s, tol, "O_student")
    ltol = (1e-3, 1e-4) if dt == "bf16" else (1e-4, 1e-6)
    assert_close(to_np(l_t), rl_t, ltol, "LSE_teacher")
    assert_close(to_np(l_s), rl_s, ltol, "LSE_student")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_teacher_equals_student_bitwise(dt):
    """No far band -> the teacher result IS the student result, bit for bit."""
    say(f"bitwise teacher==student {dt}")
    att = attn_tensors(1, 400, 4, 2, 128 if dt == "bf16" else 64, dt, seed=5)
    o_t, o_s, l_t, l_s = _gpu(att, 64, 64)
    assert torch.equal(o_t, o_s) and torch.equal(l_t, l_s)
    o_t, o_s, l_t, l_s = _gpu(att, 300, 77)
    assert torch.equal(o_t[:, :77], o_s[:, :77])
    assert torch.equal(l_t[:, :, :77], l_s[:, :, :77])
    assert not torch.equal(o_t[:, 77:], o_s[:, 77:])


def test_deterministic_run_to_run():
    say("determinism")
    att = attn_tensors(2, 777, 4, 2, 128, "bf16", seed=6)
    a = _gpu(att, 300, 40, torch.bfloat16)
    b = _gpu(att, 300, 40, torch.bfloat16)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bf16_outputs_are_rounded_fp32_outputs():
    say("bf16 output == rounded fp32 output")
    att = attn_tensors(1, 300, 4, 2, 128, "bf16", seed=7)
    a = _gpu(att, 128, 32, torch.float32)
    b = _gpu(att, 128, 32, torch.bfloat16)
    assert torch.equal(a[0].to(torch.bfloat16), b[0])
    assert torch.equal(a[1].to(torch.bfloat16), b[1])


def _sample_rows(T, wT, wS, n, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, wS - 1, wS, wS + 1, wT - 1, wT, wT + 1, T // 2, T - 2, T - 1]
    rows = set(r for r in fixed if 0 <= r < T)
    rows.update(int(x) for x in rng.integers(0, T, n))
    return sorted(rows)


def _full_size_sampled(cfg, windows, nrows):
    from dual_window_attention_amd import ttcd
    say(f"full-size attention {cfg.name}: generating inputs")
    att = I.attention_inputs(cfg)
    q, k, v = (I.to_torch(att[n]) for n in ("q", "k", "v"))
    qf, kf, vf = (att[n].f64() for n in ("q", "k", "v"))
    for wT, wS in windows:
        say(f"  windows ({wT}, {wS}): GPU run")
        o_t, o_s, l_t, l_s = ttcd.dual_window_attn(q, k, v, wT, wS, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.isfinite(o_t).all() and torch.isfinite(o_s).all()
        rows = _sample_rows(cfg.seq, wT, wS, nrows, seed=wT)
        for b in range(cfg.batch):
            r_t, r_s, rl_t, rl_s = O.dual_window_attention(qf[b:b + 1], kf[b:b + 1], vf[b:b + 1],
                                                           wT, wS, rows=rows)
            sel = np.asarray(rows)
            assert_close(to_np(o_t[b, sel]), r_t[0, sel], tol_for("bf16"), f"b{b} O_teacher rows")
            assert_close(to_np(o_s[b, sel]), r_s[0, sel], tol_for("bf16"), f"b{b} O_student rows")
            assert_close(to_np(l_t[b][:, sel]), rl_t[0][:, sel], (1e-3, 1e-4), f"b{b} LSE_T rows")
            assert_close(to_np(l_s[b][:, sel]), rl_s[0][:, sel], (1e-3, 1e-4), f"b{b} LSE_S rows")


def test_smollm2_16k_sampled_rows():
    cfg = I.CONFIGS[2]
    _full_size_sampled(cfg, [(cfg.w_teacher, cfg.w_student)], 40)


def test_qwen3_64k_sampled_rows():
    cfg = I.CONFIGS[3]
    _full_size_sampled(cfg, [(cfg.w_teacher, cfg.w_student)], 40)


def test_b8_32k_window_sweep_with_outlier_keys_sampled_rows():
    cfg = I.CONFIGS[4]
    _full_size_sampled(cfg, list(cfg.windows), 12)


@pytest.mark.parametrize("D", [64, 128])
def test_extreme_score_range(D):
    """Queries scaled x40: within a row the scores span hundreds of nats, so
    the running max moves many times and the accumulators are rescaled
    again and again; the result still matches the oracle."""
    say(f"extreme score range D={D}")
    att = attn_tensors(1, 300, 4, 2, D, "bf16", seed=77)
    q32 = I.bf16_bits_to_f32(att["q"].data) * np.float32(40.0)
    att["q"] = I.Tensor(I.f32_to_bf16_bits(q32), "bf16")
    o_t, o_s, l_t, l_s = _gpu(att, 200, 40)
    r_t, r_s, rl_t, rl_s = O.dual_window_attention(att["q"].f64(), att["k"].f64(),
                                                   att["v"].f64(), 200, 40)
    tol = tol_for("bf16")
    assert_close(to_np(o_t), r_t, tol, "O_teacher")
    assert_close(to_np(o_s), r_s, tol, "O_student")
    assert_close(to_np(l_t), rl_t, (2e-3, 1e-5), "LSE_teacher")
    assert_close(to_np(l_s), rl_s, (2e-3, 1e-5), "LSE_student")
