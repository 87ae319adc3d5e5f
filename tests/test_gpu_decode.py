"""One decode step (seq_q = 1) of the IP-TTCD layer on the GPU against the oracle.

The cache holds NaN in every row outside the teacher window of the new
token, so a kernel that reads an out-of-window key poisons its output."""
import numpy as np
import pytest

from dual_window_attention_amd import inputs as I
from oracle import ttcd_oracle as O
from tests.gpu_helpers import assert_close, say, to_np, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def nan_cache(win, L, start):
    """[B, L+1, Hkv, D] device cache: NaN everywhere but rows start..L."""
    t = I.to_torch(win)
    B, W, H, D = t.shape
    cache = torch.full((B, L + 1, H, D), float("nan"), dtype=t.dtype, device=t.device)
    cache[:, start:start + W] = t
    return cache


def run_decode(cfg, dec, w, r_dev, k_dev, state=None):
    from dual_window_attention_amd import ttcd
    L = cfg.cache_len
    kc = nan_cache(dec["k_win"], L, dec["window_start"])
    vc = nan_cache(dec["v_win"], L, dec["window_start"])
    wd = {n: I.to_torch(t) for n, t in w.items()}
    d = {"pos": L, "beta_list": I.f32_to_torch(dec["beta_list"])}
    if state is not None:
        d["state_dense"] = state
    else:
        d["r_list"], d["k_list"] = r_dev, k_dev
    out, aux = ttcd.layer_forward(I.to_torch(dec["q"]), kc, vc, I.to_torch(dec["x"]), wd,
                                  cfg.w_teacher, cfg.w_student, cfg.chunk, aux=True, decode=d)
    torch.cuda.synchronize()
    return out, aux


def oracle_decode(cfg, dec, w, r_lists, k_lists):
    wo = {n: t.f64() for n, t in w.items()}
    return O.decode_step(dec["q"].f64(), dec["k_win"].f64(), dec["v_win"].f64(), dec["x"].f64(),
                         wo, cfg.cache_len, cfg.w_teacher, cfg.w_student, r_lists, k_lists,
                         dec["beta_list"].astype(np.float64), cfg.chunk,
                         key_offset=dec["window_start"])


def check_outputs(cfg, out, aux, ref, what):
    tol = tol_for(cfg.dtype)
    say(f"  [{what}]")
    assert_close(to_np(out)[:, 0], ref["out"][:, 0], tol, "out")
    assert_close(to_np(aux["y"])[:, 0], ref["y"][:, 0], tol, "y")
    assert_close(to_np(aux["o_teacher"]), ref["o_t"], tol, "O_teacher")
    assert_close(to_np(aux["o_student"]), ref["o_s"], tol, "O_student")
    assert_close(to_np(aux["lse_teacher"]), ref["lse_t"], (1e-3, 1e-5), "LSE_teacher")
    assert_close(to_np(aux["lse_student"]), ref["lse_s"], (1e-3, 1e-5), "LSE_student")


def check_decode(cfg, list_sets=None):
    """Both state forms against the oracle's low-rank decode.

    With ``list_sets`` = m < batch, sequence b takes the lists and the write
    coefficients of sequence b % m, which keeps the host-side generation and
    the oracle's dense fold bounded at large batch."""
    B, L, C = cfg.batch, cfg.cache_len, cfg.chunk
    m = B if list_sets is None else list_sets
    say(f"decode {cfg.name} B={B} L={L} wT={cfg.w_teacher} wS={cfg.w_student} C={C} "
        f"d={cfg.d_model} f={cfg.d_ff} list sets={m}")
    dec = I.decode_inputs(cfg)
    dec["beta_list"] = np.ascontiguousarray(dec["beta_list"][np.arange(B) % m])
    w = I.layer_weights(cfg)
    sets = [I.decode_lists(cfg, s) for s in range(m)]
    on_dev = [(I.to_torch(r), I.to_torch(k)) for r, k in sets]
    r_dev = torch.stack([on_dev[b % m][0] for b in range(B)])
    k_dev = torch.stack([on_dev[b % m][1] for b in range(B)])
    del on_dev
    # each distinct list widened once; sequences of one set share the array
    wide = [(r.f64(), k.f64()) for r, k in sets]
    say("  oracle (low-rank lists)")
    ref = oracle_decode(cfg, dec, w, [wide[b % m][0] for b in range(B)],
                        [wide[b % m][1] for b in range(B)])
    say("  GPU, low-rank lists")
    out, aux = run_decode(cfg, dec, w, r_dev, k_dev)
    check_outputs(cfg, out, aux, ref, "lists")
    del r_dev, k_dev
    say("  oracle fold -> GPU, dense fp32 state")
    wd0 = w["w_down0"].f64()
    folded = [O.fold_lists(wd0, wide[s][0][None], wide[s][1][None],
                           dec["beta_list"][s:s + 1].astype(np.float64), C)[0].astype(np.float32)
              for s in range(m)]
    states = torch.stack([torch.from_numpy(folded[b % m]) for b in range(B)]).cuda()
    out2, aux2 = run_decode(cfg, dec, w, None, None, state=states)
    check_outputs(cfg, out2, aux2, ref, "dense")


SMALL = I.CONFIGS[5].scaled(batch=3, cache_len=640, n_q_heads=4, n_kv_heads=2, head_dim=64,
                            d_model=128, d_ff=256, chunk=128, w_teacher=300, w_student=40,
                            seed=41)


def test_decode_small():
    check_decode(SMALL)


def test_decode_window_covers_whole_cache():
    """w_T > L: every cached key is visible (no NaN row at all)."""
    check_decode(SMALL.scaled(cache_len=256, w_teacher=1000, w_student=100, seed=42))


def test_decode_gqa3_head64():
    check_decode(I.CONFIGS[2].scaled(batch=2, cache_len=1024, d_model=192, d_ff=256, chunk=256,
                                     w_teacher=700, w_student=64, seed=43))


def test_decode_no_completed_chunk():
    """L < C: no chunk is complete and y is the base MLP output."""
    check_decode(SMALL.scaled(cache_len=100, seed=44))


def test_decode_equals_prefill_row():
    """The decode step at position L with lists from a prefill of tokens
    0..L-1 gives the prefill oracle's row L (same weights, same q/k/v)."""
    from dual_window_attention_amd import ttcd
    cfg = I.CONFIGS[3].scaled(batch=2, seq=385, n_q_heads=4, n_kv_heads=2, d_model=128,
                              d_ff=256, w_teacher=200, w_student=32, chunk=128, seed=45)
    L, C = cfg.seq - 1, cfg.chunk
    n = L // C
    att = I.attention_inputs(cfg)
    w = I.layer_weights(cfg)
    beta = I.beta_for(cfg)
    x = I.residual_input(cfg)
    wo = {k_: t.f64() for k_, t in w.items()}
    wo["beta"] = beta.astype(np.float64)
    say("  oracle prefill")
    ref = O.layer_forward(att["q"].f64(), att["k"].f64(), att["v"].f64(), x.f64(), wo,
                          cfg.w_teacher, cfg.w_student, C)
    # lists of the n completed chunks in the layer's storage type; the beta
    # of chunk j multiplies R_j^T K_j with unit keys
    r_list = torch.from_numpy(ref["r"][:, :n * C].astype(np.float32)).to(torch.bfloat16).cuda()
    k_list = torch.from_numpy(ref["k"][:, :n * C].astype(np.float32)).to(torch.bfloat16).cuda()
    q, k, v = (I.to_torch(att[n_]) for n_ in ("q", "k", "v"))
    wd = {n_: I.to_torch(t) for n_, t in w.items()}
    out = ttcd.layer_forward(q[:, L:L + 1].contiguous(), k, v,
                             I.to_torch(x)[:, L:L + 1].contiguous(), wd, cfg.w_teacher,
                             cfg.w_student, C,
                             decode={"pos": L, "r_list": r_list, "k_list": k_list,
                                     "beta_list": I.f32_to_torch(beta[:, :n])})
    torch.cuda.synchronize()
    assert_close(to_np(out)[:, 0], ref["out"][:, L], tol_for(cfg.dtype), "decode vs prefill row L")


def test_decode_config5_full():
    """Full size: batch 32, 64K cache (NaN outside the window), 64 chunk lists."""
    check_decode(I.CONFIGS[5], list_sets=2)
