"""ttcd_dual_window_attn_backward on the GPU against the fp64 oracle's
gradient of the dual-window attention (C-ABI path).

The GPU backward consumes the GPU forward's outputs and LSEs (stored in the
input dtype, as a training step would); the oracle differentiates its own
exact forward.  Tolerances are those of every other output (relative 1e-2 in
the L2 and max norms for bf16, 1e-5 for fp32)."""
import numpy as np
import pytest

from dual_window_attention_amd import inputs as I
from oracle import ttcd_oracle as O
from tests.gpu_helpers import assert_close, attn_tensors, say, to_np, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def gpu_backward(att, wT, wS, do_t, do_s):
    from dual_window_attention_amd import ttcd
    q, k, v = (I.to_torch(att[n]) for n in ("q", "k", "v"))
    o_t, o_s, l_t, l_s = ttcd.dual_window_attn(q, k, v, wT, wS, out_dtype=q.dtype)
    g = ttcd.dual_window_attn_backward(q, k, v, o_t, o_s, l_t, l_s, I.to_torch(do_t),
                                       I.to_torch(do_s), wT, wS, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return g


def grads_case(B, T, Hq, Hkv, D, wT, wS, dt, seed):
    att = attn_tensors(B, T, Hq, Hkv, D, dt, seed=seed)
    do_t = I.normal(seed, "do_t", (B, T, Hq, D), 1.0, dt)
    do_s = I.normal(seed, "do_s", (B, T, Hq, D), 1.0, dt)
    return att, do_t, do_s


CASES = [
    # B, T, Hq, Hkv, D, wT, wS, dtype
    (1, 77, 2, 1, 64, 32, 8, "f32"),
    (2, 50, 3, 3, 128, 64, 1, "f32"),
    (1, 300, 4, 2, 128, 96, 16, "bf16"),
    (2, 333, 3, 1, 64, 200, 37, "bf16"),
    (1, 257, 4, 2, 128, 64, 64, "bf16"),
    (1, 200, 2, 1, 128, 256, 32, "bf16"),
    (1, 190, 4, 4, 128, 70, 1, "bf16"),
    (2, 130, 6, 2, 64, 33, 5, "bf16"),
    (1, 2048, 16, 8, 128, 512, 64, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_T{}_H{}/{}_D{}_w{}/{}_{}".format(*c))
def test_attention_backward_matches_oracle(case):
    B, T, Hq, Hkv, D, wT, wS, dt = case
    say(f"attention backward {case}")
    att, do_t, do_s = grads_case(B, T, Hq, Hkv, D, wT, wS, dt, seed=T + Hq + 7)
    dq, dk, dv = gpu_backward(att, wT, wS, do_t, do_s)
    rq, rk, rv = O.dual_window_attention_backward(att["q"].f64(), att["k"].f64(), att["v"].f64(),
                                                  wT, wS, do_t.f64(), do_s.f64())
    tol = tol_for(dt)
    assert_close(to_np(dq), rq, tol, "dq")
    assert_close(to_np(dk), rk, tol, "dk")
    assert_close(to_np(dv), rv, tol, "dv")


def test_attention_backward_qwen3_heads_4k():
    """16/8 heads x 128 over 4096 tokens, w_T 1024, w_S 128: many key and
    query workgroups per head, the far band and the student band both long."""
    say("attention backward qwen3 heads T=4096 w=1024/128")
    att, do_t, do_s = grads_case(1, 4096, 16, 8, 128, 1024, 128, "bf16", seed=41)
    dq, dk, dv = gpu_backward(att, 1024, 128, do_t, do_s)
    rq, rk, rv = O.dual_window_attention_backward(att["q"].f64(), att["k"].f64(), att["v"].f64(),
                                                  1024, 128, do_t.f64(), do_s.f64())
    tol = tol_for("bf16")
    assert_close(to_np(dq), rq, tol, "dq")
    assert_close(to_np(dk), rk, tol, "dk")
    assert_close(to_np(dv), rv, tol, "dv")


def test_attention_backward_64k_prefix_rows_and_dv_sums():
    """The 64K Qwen3 attention (16/8 heads x 128, w_T 8192, w_S 512).
    * dq of the first 1024 positions against the oracle run on that prefix:
      a query sees no later key, so the prefix's dq is exact there;
    * for every kv head and dim, sum_j dv_j = sum over its q heads and all
      positions of dO_T + dO_S (each softmax row sums to one): a property
      of the whole gradient, in fp64 over the GPU's output;
    * every gradient finite."""
    from dual_window_attention_amd import ttcd
    cfg = I.CONFIGS[3]
    T, wT, wS = cfg.seq, cfg.w_teacher, cfg.w_student
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    say(f"attention backward 64K: T={T} w={wT}/{wS}")
    att = I.attention_inputs(cfg)
    do_t = I.normal(51, "do_t", (1, T, Hq, D), 1.0, "bf16")
    do_s = I.normal(51, "do_s", (1, T, Hq, D), 1.0, "bf16")
    q, k, v = (I.to_torch(att[n]) for n in ("q", "k", "v"))
    o_t, o_s, l_t, l_s = ttcd.dual_window_attn(q, k, v, wT, wS, out_dtype=torch.bfloat16)
    dtt, dst = I.to_torch(do_t), I.to_torch(do_s)
    dq, dk, dv = ttcd.dual_window_attn_backward(q, k, v, o_t, o_s, l_t, l_s, dtt, dst, wT, wS,
                                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isfinite(t).all().item(), n
    P = 1024
    rq, _, _ = O.dual_window_attention_backward(att["q"].f64()[:, :P], att["k"].f64()[:, :P],
                                                att["v"].f64()[:, :P], wT, wS,
                                                do_t.f64()[:, :P], do_s.f64()[:, :P])
    assert_close(to_np(dq[:, :P]), rq, tol_for("bf16"), "dq[:1024]")
    G = Hq // Hkv
    got = dv.double().sum(dim=1).cpu().numpy()                          # [1, Hkv, D]
    want = (dtt.double() + dst.double()).reshape(1, T, Hkv, G, D).sum(dim=(1, 3)).cpu().numpy()
    assert_close(got, want, tol_for("bf16"), "sum_j dv_j")


def test_attention_backward_deterministic_run_to_run():
    """No atomics: every gradient is a fixed-order sum, so two calls agree
    bit for bit (GQA 2:1, both windows, a ragged tail)."""
    say("attention backward determinism")
    att, do_t, do_s = grads_case(2, 777, 4, 2, 128, 300, 40, "bf16", seed=9)
    a = gpu_backward(att, 300, 40, do_t, do_s)
    b = gpu_backward(att, 300, 40, do_t, do_s)
    for n, x, y in zip(("dq", "dk", "dv"), a, b):
        assert torch.equal(x, y), n
