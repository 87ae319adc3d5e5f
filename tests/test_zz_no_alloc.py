"""ttcd_layer_forward_noalloc (the library's own scratch, no workspace)
against ttcd_layer_forward (caller's workspace) on the GPU: the same kernels
on the same inputs, so the outputs must agree bit for bit.  Two decode steps
in a row, the second with a smaller batch, cache and list set, then a short
prefill; the array keeps each call's contents for the next."""
import numpy as np
import pytest

from dual_window_attention_amd import inputs as I
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def decode_case(cfg):
    """Device inputs of one decode step in list form (NaN outside the
    teacher window of the cache)."""
    B, L = cfg.batch, cfg.cache_len
    dec = I.decode_inputs(cfg)
    lists = [I.decode_lists(cfg, b) for b in range(B)]
    r = torch.stack([I.to_torch(lr) for lr, _ in lists])
    k = torch.stack([I.to_torch(lk) for _, lk in lists])
    start = dec["window_start"]

    def cache(win):
        t = I.to_torch(win)
        c = torch.full((B, L + 1) + tuple(t.shape[2:]), float("nan"), dtype=t.dtype,
                       device="cuda")
        c[:, start:start + t.shape[1]] = t
        return c

    w = {n: I.to_torch(t) for n, t in I.layer_weights(cfg).items()}
    d = {"pos": L, "r_list": r, "k_list": k, "beta_list": I.f32_to_torch(dec["beta_list"])}
    return (I.to_torch(dec["q"]), cache(dec["k_win"]), cache(dec["v_win"]),
            I.to_torch(dec["x"]), w, d)


def both(q, k, v, x, w, cfg, decode=None):
    from dual_window_attention_amd import ttcd
    args = (q, k, v, x, w, cfg.w_teacher, cfg.w_student, cfg.chunk)
    out_a, aux_a = ttcd.layer_forward(*args, aux=True, decode=decode)
    out_b, aux_b = ttcd.layer_forward(*args, aux=True, decode=decode, no_alloc=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out_a).all().item()
    assert torch.equal(out_a, out_b), "out differs"
    for n in aux_a:
        assert torch.equal(aux_a[n], aux_b[n]), f"aux {n} differs"
    say(f"  equal: out and {len(aux_a)} aux outputs, max|out|={out_a.abs().max().item():.3g}")


def test_noalloc_layer_equals_workspace_layer_twice_then_smaller():
    big = I.CONFIGS[5].scaled(batch=4, cache_len=1280, n_q_heads=4, n_kv_heads=2, head_dim=128,
                              d_model=256, d_ff=512, chunk=256, w_teacher=600, w_student=64,
                              seed=61)
    small = big.scaled(batch=2, cache_len=300, seed=62)
    for cfg in (big, small):
        say(f"decode B={cfg.batch} L={cfg.cache_len} chunks={cfg.cache_len // cfg.chunk}")
        q, k, v, x, w, d = decode_case(cfg)
        both(q, k, v, x, w, cfg, decode=d)
    cfg = I.CONFIGS[3].scaled(seq=384, n_q_heads=4, n_kv_heads=2, d_model=256, d_ff=384,
                              w_teacher=160, w_student=40, chunk=128, seed=63)
    say(f"prefill T={cfg.seq}")
    att = I.attention_inputs(cfg)
    w = {n: I.to_torch(t) for n, t in I.layer_weights(cfg).items()}
    w["beta"] = I.f32_to_torch(I.beta_for(cfg))
    both(*(I.to_torch(att[n]) for n in ("q", "k", "v")), I.to_torch(I.residual_input(cfg)), w,
         cfg)
