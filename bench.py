"""Benchmark: IP-TTCD layer forward on one MI355X.

Default workload: the Qwen3-0.6B-shaped layer at 64K context (batch 1,
65536 tokens, 16 q heads / 8 kv heads, head_dim 128, d_model 1024, d_ff
3072, w_T 8192, w_S 512, chunk 1024, conv 4), bf16 inputs, synthetic data.

Prints ONE JSON line: whole-layer tokens/s, the roofline of the dominant
kernel (the dual-window attention, bf16 MFMA) measured with HIP events on
the stream it runs on, and the fp64 CPU oracle timed on a bounded sample of
the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6       # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_qwen3_64k.txt")
# the sources whose kernels each traffic figure was measured on
TRAFFIC_SOURCES = {
    "attention": ["dual_window_attention_amd/csrc/attn.hip", "dual_window_attention_amd/csrc/common.hpp"],
    "scan": ["dual_window_attention_amd/csrc/stream.hip", "dual_window_attention_amd/csrc/common.hpp"],
}


def source_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(part):
    """HBM bytes per launch of ``part`` from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of known size), or
    None when the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    sec, vals = None, {}
    for ln in lines:
        ln = ln.strip()
        if ln.startswith("[") and ln.endswith("]"):
            sec = ln[1:-1]
        elif sec == part and ":" in ln and not ln.startswith("#"):
            k_, v_ = ln.split(":", 1)
            vals[k_.strip()] = v_.strip()
    if vals.get("sources_sha256") != source_digest(TRAFFIC_SOURCES[part]):
        return None
    try:
        return float(vals["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attention_flops(cfg, wT):
    """Algorithmic flops: 4*D per (query, key) pair inside the teacher
    window (2D for QK^T, 2D for PV); the student band is a subset of it."""
    T, Hq, D, B = cfg.seq, cfg.n_q_heads, cfg.head_dim, cfg.batch
    full = max(0, T - wT) * wT
    ramp = sum(min(t + 1, wT) for t in range(min(T, wT)))
    return 4.0 * D * Hq * B * (full + ramp)


def scan_bytes(cfg):
    """Algorithmic bytes of the fast-weight stream: read Z_T, Z_S, write
    the residual difference and the keys (bf16): 8 B T f."""
    return 8.0 * cfg.batch * cfg.seq * cfg.d_ff


def time_events(fn, n, stream, warmup=5):
    """Mean device time of ``fn`` over ``n`` back-to-back calls: one HIP event
    recorded on ``stream`` (the stream the library launches on) before the
    first call and one after the last, so the average covers the kernels
    and the gaps between launches but not an event per call.  The warmup
    calls bring the clocks back up after host-side set-up left the GPU
    idle."""
    import torch
    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return float(e0.elapsed_time(e1)) / n


def scan_roofline(cfg, dev, n):
    """The fast-weight stream (HBM-bound) at the workload's size, timed alone."""
    import torch
    from dual_window_attention_amd import inputs as I
    from dual_window_attention_amd import ttcd

    z = I.hidden_activations(cfg)
    w = I.layer_weights(cfg)
    zt, zs = I.to_torch(z["z_t"], dev), I.to_torch(z["z_s"], dev)
    del z
    ct, cs = I.to_torch(w["conv_t"], dev), I.to_torch(w["conv_s"], dev)
    beta = I.f32_to_torch(I.beta_for(cfg), dev)
    out = ttcd.fastweight_stream(zt, zs, ct, cs, beta, cfg.chunk)
    ws = torch.empty(max(256, ttcd.lib().ttcd_fastweight_stream_workspace_size(
        ttcd.fw_desc(zt, 8, cfg.chunk, cfg.conv_k))), dtype=torch.uint8, device=dev)

    def run():
        ttcd.fastweight_stream(zt, zs, ct, cs, beta, cfg.chunk, out=out, workspace=ws)

    ms = time_events(run, n, torch.cuda.current_stream(), warmup=20)
    gb = scan_bytes(cfg) / 1e9
    return {"bound": "hbm", "kernel": "fast-weight stream (ttcd_fastweight_stream)",
            "achieved": gb / (ms * 1e-3), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": gb / (ms * 1e-3) / PEAK_HBM_GBS, "traffic": measured_traffic("scan"),
            "ms_per_launch": ms, "algorithmic_gb": gb}


def update_rules_bench(cfg, dev, n):
    """The fast-weight path (stream, residual projection, writes, prefix,
    apply) under the off-policy rule (all residuals at W_down^(0), parallel
    over chunks), under the on-policy recurrence (chunk after chunk), and
    the unprojected write (no convs, no W_proj, raw keys), same inputs,
    output y in fp32."""
    import torch
    from dual_window_attention_amd import inputs as I
    from dual_window_attention_amd import ttcd

    z = I.hidden_activations(cfg)
    w = I.layer_weights(cfg)
    zt, zs = I.to_torch(z["z_t"], dev), I.to_torch(z["z_s"], dev)
    del z
    a = [zt, zs, zt] + [I.to_torch(w[k], dev) for k in ("conv_t", "conv_s", "w_down0", "w_proj")]
    a.append(I.f32_to_torch(I.beta_for(cfg), dev))
    d = ttcd.fw_desc(zt, cfg.d_model, cfg.chunk, cfg.conv_k, 0.0, torch.float32)
    lib = ttcd.lib()
    ws = torch.empty(max(lib.ttcd_fastweight_scan_workspace_size(d),
                         lib.ttcd_fastweight_scan_on_policy_workspace_size(d),
                         lib.ttcd_fastweight_scan_eq6_workspace_size(d)),
                     dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream()
    off_ms = time_events(lambda: ttcd.fastweight_scan(*a, cfg.chunk, workspace=ws), n, st, 3)
    on_ms = time_events(lambda: ttcd.fastweight_scan_on_policy(*a, cfg.chunk, workspace=ws),
                        n, st, 3)
    e6 = [a[0], a[1], a[2], a[5], a[7]]
    eq6_ms = time_events(lambda: ttcd.fastweight_scan_eq6(*e6, cfg.chunk, workspace=ws), n, st, 3)
    # how far the off-policy approximation moves y: the gap between the two
    # rules' outputs, against the on-policy correction y - W_down0 z
    y_off, _ = ttcd.fastweight_scan(*a, cfg.chunk, workspace=ws)
    y_on, _ = ttcd.fastweight_scan_on_policy(*a, cfg.chunk, workspace=ws)
    base = torch.matmul(zt[0].float(), a[5].float().t())
    gap = float(torch.linalg.vector_norm(y_off[0] - y_on[0]))
    corr = float(torch.linalg.vector_norm(y_on[0] - base))
    yn = float(torch.linalg.vector_norm(y_on[0]))
    del a, e6, ws, y_off, y_on, base
    return {"kernel": "fast-weight path: off-policy (ttcd_fastweight_scan), on-policy "
                      "recurrence (ttcd_fastweight_scan_on_policy), unprojected write "
                      "(ttcd_fastweight_scan_eq6)",
            "off_policy_ms": off_ms, "on_policy_ms": on_ms, "on_over_off": on_ms / off_ms,
            "eq6_unprojected_ms": eq6_ms,
            "off_vs_on_gap_rel_correction": gap / corr, "off_vs_on_gap_rel_y": gap / yn,
            "tokens": cfg.batch * cfg.seq, "chunks": cfg.n_chunks}


def decode_bench(dev, n):
    """One decode token per sequence at the batch-32, 64K-cache workload:
    low-rank lists and folded dense state; the fold itself timed once."""
    import torch
    from dual_window_attention_amd import inputs as I
    from dual_window_attention_amd import ttcd

    cfg = I.CONFIGS[5]
    B, L = cfg.batch, cfg.cache_len
    dec = I.decode_inputs(cfg)
    m = 2      # sequence b takes the lists and write coefficients of sequence b % 2
    dec["beta_list"] = np.ascontiguousarray(dec["beta_list"][np.arange(B) % m])
    sets = [I.decode_lists(cfg, s) for s in range(m)]
    on = [(I.to_torch(r, dev), I.to_torch(k, dev)) for r, k in sets]
    del sets
    r_l = torch.stack([on[b % m][0] for b in range(B)])
    k_l = torch.stack([on[b % m][1] for b in range(B)])
    del on
    w = I.layer_weights(cfg)
    wd = {k_: I.to_torch(t, dev) for k_, t in w.items()}
    start = dec["window_start"]

    def cache(win):
        t = I.to_torch(win, dev)
        c = torch.full((B, L + 1) + tuple(t.shape[2:]), float("nan"), dtype=t.dtype, device=dev)
        c[:, start:start + t.shape[1]] = t
        return c

    kc, vc = cache(dec["k_win"]), cache(dec["v_win"])
    q, x = I.to_torch(dec["q"], dev), I.to_torch(dec["x"], dev)
    bl = I.f32_to_torch(dec["beta_list"], dev)
    stream = torch.cuda.current_stream()
    fold_ws = torch.empty(max(256, ttcd.lib().ttcd_fastweight_fold_workspace_size(
        ttcd.FwDesc(B, L, cfg.d_model, cfg.d_ff, cfg.chunk, 1, 0.0, 1, 0), L // cfg.chunk)),
        dtype=torch.uint8, device=dev)
    dense = ttcd.fastweight_fold(wd["w_down0"], r_l, k_l, bl, cfg.chunk, workspace=fold_ws)
    fold_ms = time_events(lambda: ttcd.fastweight_fold(wd["w_down0"], r_l, k_l, bl, cfg.chunk,
                                                       workspace=fold_ws), 2, stream, warmup=1)
    out = torch.empty((B, 1, cfg.d_model), dtype=torch.float32, device=dev)
    res = {}
    win_bytes = 2.0 * B * min(cfg.w_teacher, L + 1) * cfg.n_kv_heads * cfg.head_dim * 2
    w_bytes = sum(int(wd[n_].numel()) * 2 for n_ in ("w_o", "w_gate", "w_up", "w_down0"))
    for form, d in (("dense", {"pos": L, "state_dense": dense, "beta_list": bl}),
                    ("lists", {"pos": L, "r_list": r_l, "k_list": k_l, "beta_list": bl})):
        need = ttcd.layer_workspace_bytes(q, kc, cfg.d_model, cfg.d_ff, cfg.w_teacher,
                                          cfg.w_student, cfg.chunk,
                                          decode_chunks=L // cfg.chunk, pos=L)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

        def step(d=d, ws=ws):
            ttcd.layer_forward(q, kc, vc, x, wd, cfg.w_teacher, cfg.w_student, cfg.chunk,
                               decode=d, out=out, workspace=ws)

        ms = time_events(step, n, stream, warmup=10)
        st_bytes = (B * cfg.d_model * cfg.d_ff * 4.0 if form == "dense"
                    else float(r_l.numel() + k_l.numel()) * 2)
        gb = (win_bytes + w_bytes + st_bytes) / 1e9
        res[form] = {"ms_per_step": ms, "tokens_per_s": B / (ms * 1e-3),
                     "algorithmic_gb": gb, "achieved_gbs": gb / (ms * 1e-3),
                     "hbm_frac": gb / (ms * 1e-3) / PEAK_HBM_GBS}
        assert torch.isfinite(out).all().item()
    # a generation step that also extends the fast weight: the dense-state
    # decode step returning both paths' Z, then the token's (r, k) appended
    # to the pending chunk (conv over a history of kc-1 rows per path)
    f, C = cfg.d_ff, cfg.chunk
    ntap = int(wd["conv_t"].shape[1])
    m_res = ttcd.fastweight_residual_proj(wd["w_down0"], wd["w_proj"])
    hist_t = torch.zeros((B, ntap - 1, f), dtype=torch.bfloat16, device=dev)
    hist_s = torch.zeros_like(hist_t)
    r_pend = torch.zeros((B, C, cfg.d_model), dtype=torch.bfloat16, device=dev)
    k_pend = torch.zeros((B, C, f), dtype=torch.bfloat16, device=dev)
    dense_d = {"pos": L, "state_dense": dense, "beta_list": bl}
    need = ttcd.layer_workspace_bytes(q, kc, cfg.d_model, cfg.d_ff, cfg.w_teacher, cfg.w_student,
                                      cfg.chunk, decode_chunks=L // cfg.chunk, pos=L)
    gws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    zpair = {}

    def append():
        ttcd.fastweight_decode_append(zpair["t"], zpair["s"], hist_t, hist_s, wd["conv_t"],
                                      wd["conv_s"], m_res, r_pend[:, 0], k_pend[:, 0])

    def gen_step():
        _, a = ttcd.layer_forward(q, kc, vc, x, wd, cfg.w_teacher, cfg.w_student, cfg.chunk,
                                  decode=dense_d, out=out, workspace=gws, aux=True)
        zpair["t"], zpair["s"] = a["z_teacher"][:, 0], a["z_student"][:, 0]
        append()

    gen_ms = time_events(gen_step, n, stream, warmup=10)
    app_ms = time_events(append, n, stream, warmup=5)
    res["generate_dense"] = {"ms_per_step": gen_ms, "tokens_per_s": B / (gen_ms * 1e-3),
                             "append_ms": app_ms,
                             "what": "dense-state decode step with both paths' Z, then the "
                                     "token's (r, k) appended to the pending chunk"}
    res["fold_ms"] = fold_ms
    res["fold_tflops"] = 2.0 * B * L * cfg.d_model * cfg.d_ff / (fold_ms * 1e-3) / 1e12
    res["workload"] = (f"{cfg.name}: decode step, batch {B}, 64K cache (NaN outside the "
                       f"w_T={cfg.w_teacher} window), {L // cfg.chunk} chunk lists")
    return res


def cpu_baseline(cfg, sample_tokens):
    """The fp64 oracle, as it stands, on the first ``sample_tokens`` tokens
    of the same inputs (same shapes, weights and windows)."""
    from dual_window_attention_amd import inputs as I
    from oracle import ttcd_oracle as O

    sc = cfg.scaled(seq=sample_tokens)
    att = I.attention_inputs(sc)
    w = {n: t.f64() for n, t in I.layer_weights(sc).items()}
    w["beta"] = I.beta_for(sc).astype(np.float64)
    x = I.residual_input(sc).f64()
    q, k, v = att["q"].f64(), att["k"].f64(), att["v"].f64()
    t0 = time.perf_counter()
    O.layer_forward(q, k, v, x, w, sc.w_teacher, sc.w_student, sc.chunk)
    wall = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": sample_tokens * sc.batch / wall, "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"fp64 NumPy oracle, full layer forward over the first {sample_tokens} "
                      f"tokens of the same config (windows fill up over the first "
                      f"{sc.w_teacher} tokens), wall {wall:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--cpu-sample", type=int, default=20480,
                    help="tokens of the oracle CPU baseline sample (0 = skip)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step section")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the LSE-combination and update-rule sections (the counter passes "
                         "then see only the fused attention call)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (a reference "
                         "kernel of known traffic for scaling memory counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only (no collectives); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from dual_window_attention_amd import inputs as I
    from dual_window_attention_amd import ttcd

    cfg = I.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    att = I.attention_inputs(cfg)
    q, k, v = (I.to_torch(att[n], dev) for n in ("q", "k", "v"))
    del att
    w = I.layer_weights(cfg)
    wd = {n: I.to_torch(t, dev) for n, t in w.items()}
    wd["beta"] = I.f32_to_torch(I.beta_for(cfg), dev)
    x = I.to_torch(I.residual_input(cfg), dev)
    B, T = cfg.batch, cfg.seq
    ws_bytes = ttcd.layer_workspace_bytes(q, k, cfg.d_model, cfg.d_ff, cfg.w_teacher,
                                          cfg.w_student, cfg.chunk, cfg.conv_k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, cfg.d_model), dtype=torch.float32, device=dev)

    def step():
        ttcd.layer_forward(q, k, v, x, wd, cfg.w_teacher, cfg.w_student, cfg.chunk, out=out,
                           workspace=ws)

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    tokens_per_s = B * T / dt
    assert torch.isfinite(out).all().item()

    # dominant kernel: dual-window attention, timed with events on its stream
    stream = torch.cuda.current_stream()
    o_t = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    o_s = torch.empty_like(o_t)
    aws = torch.empty(max(256, ttcd.lib().ttcd_dual_window_attn_workspace_size(
        ttcd.attn_desc(q, k, cfg.w_teacher, cfg.w_student))), dtype=torch.uint8, device=dev)
    n_att = max(10, args.steps)
    att_ms = time_events(lambda: ttcd.dual_window_attn(q, k, v, cfg.w_teacher, cfg.w_student,
                                                       with_lse=False, out=(o_t, o_s),
                                                       workspace=aws), n_att, stream)
    flops = attention_flops(cfg, cfg.w_teacher)
    achieved = flops / (att_ms * 1e-3) / 1e12
    # the same outputs through the LSE-combination path (student call,
    # shifted far-band call, exact merge), for the fused-versus-split figure
    sws = torch.empty(max(256, ttcd.lib().ttcd_dual_window_attn_lse_split_workspace_size(
        ttcd.attn_desc(q, k, cfg.w_teacher, cfg.w_student))), dtype=torch.uint8, device=dev)
    split_ms = None if args.no_variants else time_events(
        lambda: ttcd.dual_window_attn_lse_split(q, k, v, cfg.w_teacher, cfg.w_student,
                                                with_lse=False, out=(o_t, o_s), workspace=sws),
        n_att, stream)

    res = {
        "metric": "IP-TTCD layer fwd tokens/s at 64K ctx; % bf16 MFMA peak (attn), % HBM BW (scan)",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian inputs, fan-in scaled random weights)",
        "config": {"workload": f"{cfg.name}: IP-TTCD layer forward, batch {B}, seq {T}, "
                               f"{cfg.n_q_heads}/{cfg.n_kv_heads} heads x {cfg.head_dim}, "
                               f"d_model {cfg.d_model}, d_ff {cfg.d_ff}, w_T {cfg.w_teacher}, "
                               f"w_S {cfg.w_student}, chunk {cfg.chunk}",
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "dual-window attention (ttcd_dual_window_attn)",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic("attention"),
                     "ms_per_launch": att_ms, "algorithmic_tflop": flops / 1e12},
    }
    if split_ms is not None:
        res["lse_split"] = {"kernel": "LSE-combination path (ttcd_dual_window_attn_lse_split)",
                            "ms_per_launch": split_ms,
                            "achieved": flops / (split_ms * 1e-3) / 1e12, "unit": "TFLOP/s",
                            "fused_ms_per_launch": att_ms, "fused_saving": 1.0 - att_ms / split_ms}
    del q, k, v, wd, x, out, ws, o_t, o_s, aws, sws
    torch.cuda.empty_cache()
    res["scan"] = scan_roofline(cfg, dev, n_att)
    torch.cuda.empty_cache()
    if not args.no_variants:
        res["update_rules"] = update_rules_bench(cfg, dev, 5)
        torch.cuda.empty_cache()
    if not args.no_decode:
        res["decode"] = decode_bench(dev, n_att)
        torch.cuda.empty_cache()
    if args.cpu_sample > 0:
        res["cpu_baseline"] = cpu_baseline(cfg, min(args.cpu_sample, cfg.seq))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
