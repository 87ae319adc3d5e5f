"""Library calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library allocates nothing and issues no memset or copy: every call is
kernel launches on the caller's stream, so a caller can capture a decode
step or a prefill once and replay it.  Each case runs the call eagerly,
captures the same call, then replays the graph three times with eager work
between the replays (the output cleared by a fill kernel, another call of
the library into a second output with the same workspace, a torch product)
and device synchronisations; every replay must reproduce the eager result
bit for bit (all kernels are deterministic)."""
import pytest

from dual_window_attention_amd import inputs as I
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEC = I.CONFIGS[5].scaled(batch=3, cache_len=640, n_q_heads=4, n_kv_heads=2, head_dim=128,
                          d_model=256, d_ff=512, chunk=128, w_teacher=300, w_student=40, seed=71)


def decode_case(cfg, dense):
    """Device inputs of one decode step (NaN outside the teacher window of
    the cache); the fast weight as chunk lists or folded dense."""
    from dual_window_attention_amd import ttcd
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
    bl = I.f32_to_torch(dec["beta_list"])
    d = {"pos": L, "beta_list": bl}
    if dense:
        d["state_dense"] = ttcd.fastweight_fold(w["w_down0"], r, k, bl, cfg.chunk)
    else:
        d["r_list"], d["k_list"] = r, k
    return (I.to_torch(dec["q"]), cache(dec["k_win"]), cache(dec["v_win"]),
            I.to_torch(dec["x"]), w, d)


def replay_matches(call, out, out2):
    """Eager call, capture, three replays against the eager result."""
    call(out)
    torch.cuda.synchronize()
    ref = out.clone()
    assert torch.isfinite(ref).all().item()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    torch.cuda.synchronize()
    a = torch.randn(512, 512, device="cuda")
    for i in range(3):
        out.zero_()
        call(out2)                       # eager use of the same workspace between replays
        a = a @ a.T / 512.0
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager call"
        assert torch.equal(out2, ref), f"eager call {i} differs"
    say(f"  3 replays equal to the eager call, max|out|={ref.abs().max().item():.3g}")


@pytest.mark.parametrize("form", ["lists", "dense"])
def test_decode_step_graph_replays(form):
    from dual_window_attention_amd import ttcd
    cfg = DEC
    say(f"decode graph {form} B={cfg.batch} L={cfg.cache_len}")
    q, k, v, x, w, d = decode_case(cfg, dense=form == "dense")
    need = ttcd.layer_workspace_bytes(q, k, cfg.d_model, cfg.d_ff, cfg.w_teacher, cfg.w_student,
                                      cfg.chunk, decode_chunks=cfg.cache_len // cfg.chunk,
                                      pos=cfg.cache_len)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.batch, 1, cfg.d_model), dtype=torch.float32, device="cuda")

    def call(o):
        ttcd.layer_forward(q, k, v, x, w, cfg.w_teacher, cfg.w_student, cfg.chunk, decode=d,
                           out=o, workspace=ws)

    replay_matches(call, out, torch.empty_like(out))


def test_decode_step_noalloc_graph_replays():
    """The entry point for callers that cannot allocate, captured."""
    from dual_window_attention_amd import ttcd
    cfg = DEC.scaled(seed=72)
    say(f"decode graph no-alloc B={cfg.batch} L={cfg.cache_len}")
    q, k, v, x, w, d = decode_case(cfg, dense=False)
    out = torch.empty((cfg.batch, 1, cfg.d_model), dtype=torch.float32, device="cuda")

    def call(o):
        ttcd.layer_forward(q, k, v, x, w, cfg.w_teacher, cfg.w_student, cfg.chunk, decode=d,
                           out=o, no_alloc=True)

    replay_matches(call, out, torch.empty_like(out))


def test_prefill_graph_replays():
    from dual_window_attention_amd import ttcd
    cfg = I.CONFIGS[3].scaled(seq=700, n_q_heads=4, n_kv_heads=2, d_model=256, d_ff=384,
                              w_teacher=200, w_student=40, chunk=128, seed=73)
    say(f"prefill graph T={cfg.seq} (ragged last chunk)")
    att = I.attention_inputs(cfg)
    q, k, v = (I.to_torch(att[n]) for n in ("q", "k", "v"))
    x = I.to_torch(I.residual_input(cfg))
    w = {n: I.to_torch(t) for n, t in I.layer_weights(cfg).items()}
    w["beta"] = I.f32_to_torch(I.beta_for(cfg))
    need = ttcd.layer_workspace_bytes(q, k, cfg.d_model, cfg.d_ff, cfg.w_teacher, cfg.w_student,
                                      cfg.chunk)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.batch, cfg.seq, cfg.d_model), dtype=torch.float32, device="cuda")

    def call(o):
        ttcd.layer_forward(q, k, v, x, w, cfg.w_teacher, cfg.w_student, cfg.chunk, out=o,
                           workspace=ws)

    replay_matches(call, out, torch.empty_like(out))
