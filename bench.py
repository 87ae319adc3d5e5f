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


TRAFFIC_HEADER = """\
# HBM traffic per launch on the 64K Qwen3 layer workload (rocprofv3 --pmc)
#
# Two counter passes, each its own run, from /tmp with TMPDIR=/tmp (R = repository root):
#   rocprofv3 --pmc FETCH_SIZE --kernel-include-regex "ttcd|copyBuffer" --output-format csv -d <dir> -o FETCH_SIZE -- python3 R/bench.py --steps 1 --warmup 0 --no-decode --no-variants --no-extra --no-backward --cpu-sample 0 --calib-copy
#   rocprofv3 --pmc WRITE_SIZE --kernel-include-regex "ttcd|copyBuffer" --output-format csv -d <dir> -o WRITE_SIZE -- python3 R/bench.py --steps 1 --warmup 0 --no-decode --no-variants --no-extra --no-backward --cpu-sample 0 --calib-copy
# then: python3 R/bench.py --write-traffic <dir>/FETCH_SIZE_counter_collection.csv <dir>/WRITE_SIZE_counter_collection.csv
#
# Scaling: the same counters on the plain 1 GiB device-to-device copy that --calib-copy runs
# (__amd_rocclr_copyBuffer, the largest copy of the run): FETCH_SIZE {cf:.0f} KiB, WRITE_SIZE {cw:.0f} KiB for
# 1048576 KiB read and written, so bytes = FETCH_SIZE KiB x 1024 x {ff:.5f} and WRITE_SIZE KiB x 1024 x {fw:.5f}.
# FETCH_SIZE counts what L2 requests from the memory side, so Infinity Cache hits are included.
# bench.py reports bytes_per_launch as roofline.traffic while sources_sha256 matches the sources.
"""

# (section, comment, [(short name, kernel-name substring, grid)], algorithmic bytes)
TRAFFIC_PARTS = [
    ("attention",
     "ttcd_dual_window_attn: V^T prologue + dual-window kernel (bf16 O, no LSE); "
     "algorithmic = Q,K,V read + O_T,O_S written",
     [("vt", "v_transpose_kernel", "4194304"), ("attn", "dual_window_attn_mfma", "2097152")],
     2 * 65536 * (16 + 8 + 8 + 16 + 16) * 128),
    ("scan",
     "fw_stream2_kernel (the key-scale reduction adds 6 MB); algorithmic = 8 B T f",
     [("stream", "fw_stream2_kernel", "6291456")],
     8 * 65536 * 3072),
]


def write_traffic(fetch_csv, write_csv, out_path=TRAFFIC_FILE):
    """Write the per-launch HBM traffic summary from the two counter passes
    (FETCH_SIZE and WRITE_SIZE, KiB per dispatch), each scaled by what the
    same counter reads for the 1 GiB copy of the calibration run."""
    import csv

    def per_dispatch(path, counter):
        rows = []
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                grid = row["Grid_Size"] if "Grid_Size" in row else "x".join(
                    row.get(f"Grid_Size_{a}", "?") for a in "XYZ")
                rows.append((row["Kernel_Name"], grid, float(row["Counter_Value"])))
        return rows

    fetch = per_dispatch(fetch_csv, "FETCH_SIZE")
    write = per_dispatch(write_csv, "WRITE_SIZE")

    def calib(rows):
        # the 1 GiB calibration copy is the largest copy of the run (the
        # stream's copy ceiling runs smaller copies at the same grid)
        copies = [v for n, g, v in rows if "copyBuffer" in n]
        if not copies:
            raise SystemExit("no copyBuffer dispatch in the counter file (run with --calib-copy)")
        return float(max(copies))

    cf, cw = calib(fetch), calib(write)
    ff, fw = 1048576.0 / cf, 1048576.0 / cw
    out = [TRAFFIC_HEADER.format(cf=cf, cw=cw, ff=ff, fw=fw)]
    for sec, comment, kernels, alg in TRAFFIC_PARTS:
        lines = [f"[{sec}]", f"# {comment}", "kernels: " + ", ".join(k for k, _, _ in kernels)]
        rd = wr = 0.0
        counts = []
        body = []
        for short, sub, grid in kernels:
            fv = [v for n, g, v in fetch if sub in n and g == grid]
            wv = [v for n, g, v in write if sub in n and g == grid]
            if not fv or not wv:
                raise SystemExit(f"no {sub} dispatch at grid {grid} in the counter files")
            counts.append(min(len(fv), len(wv)))
            body.append(f"fetch_kib_per_dispatch_{short}: {np.mean(fv):.0f}")
            body.append(f"write_kib_per_dispatch_{short}: {np.mean(wv):.0f}")
            rd += np.mean(fv) * 1024 * ff
            wr += np.mean(wv) * 1024 * fw
        lines.append(f"dispatches: {min(counts)}")
        lines += body
        lines += [f"read_bytes_per_launch: {rd:.4e}", f"write_bytes_per_launch: {wr:.4e}",
                  f"bytes_per_launch: {rd + wr:.4e}", f"algorithmic_bytes_per_launch: {alg:.4e}",
                  f"traffic_over_algorithmic: {(rd + wr) / alg:.2f}",
                  f"sources_sha256: {source_digest(TRAFFIC_SOURCES[sec])}", ""]
        out.append("\n".join(lines))
    with open(out_path, "w") as f:
        f.write("\n".join(out))
    print(f"wrote {out_path}")


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


def scan_roofline(cfg, dev, n, counters=True):
    """The fast-weight stream (HBM-bound) at the workload's size, timed alone.
    ``counters``: attach the committed counter traffic, which was taken at
    the 64K workload (None for other sizes)."""
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
    # the practical ceiling for this traffic: a plain device-to-device copy
    # of the same bytes (half of them read, half written), timed the same way
    src = torch.ones(int(scan_bytes(cfg) // 2), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_ms = time_events(lambda: dst.copy_(src), n, torch.cuda.current_stream(), warmup=5)
    copy_gbs = 2 * src.numel() / (copy_ms * 1e-3) / 1e9
    del src, dst
    return {"bound": "hbm", "kernel": "fast-weight stream (ttcd_fastweight_stream)",
            "achieved": gb / (ms * 1e-3), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": gb / (ms * 1e-3) / PEAK_HBM_GBS,
            "traffic": measured_traffic("scan") if counters else None,
            "ms_per_launch": ms, "algorithmic_gb": gb,
            "copy_ceiling": {"gbs": copy_gbs, "ms": copy_ms,
                             "what": "device-to-device copy of the same byte count (read + written)"},
            "of_copy": gb / (ms * 1e-3) / copy_gbs}


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
    # chunk-mean write coefficients: under beta ~ U(0,1) the on-policy
    # recurrence grows the weight geometrically and the gap below is moot
    a.append(I.f32_to_torch(I.beta_for(cfg, chunk_mean=True), dev))
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
            "eq6_unprojected_ms": eq6_ms, "beta": "u_i / |C_i|, u_i ~ U(0,1)",
            "off_vs_on_gap_rel_correction": gap / corr, "off_vs_on_gap_rel_y": gap / yn,
            "tokens": cfg.batch * cfg.seq, "chunks": cfg.n_chunks}


def backward_bench(cfg, dev, n):
    """The fast-weight path's gradient (ttcd_fastweight_scan_backward) at the
    workload's size, beside its forward (ttcd_fastweight_scan) on the same
    inputs; gradients of the activations in bf16, of the weights in fp32."""
    import torch
    from dual_window_attention_amd import inputs as I
    from dual_window_attention_amd import ttcd

    z = I.hidden_activations(cfg)
    w = I.layer_weights(cfg)
    zt, zs = I.to_torch(z["z_t"], dev), I.to_torch(z["z_s"], dev)
    del z
    wt = [I.to_torch(w[k], dev) for k in ("conv_t", "conv_s", "w_down0", "w_proj")]
    beta = I.f32_to_torch(I.beta_for(cfg), dev)
    dy = torch.randn((cfg.batch, cfg.seq, cfg.d_model), generator=torch.Generator().manual_seed(5),
                     dtype=torch.float32).to(dev, torch.bfloat16)
    d = ttcd.fw_desc(zt, cfg.d_model, cfg.chunk, cfg.conv_k, 0.0, torch.bfloat16)
    lib = ttcd.lib()
    ws = torch.empty(max(lib.ttcd_fastweight_scan_backward_workspace_size(d),
                         lib.ttcd_fastweight_scan_workspace_size(d)),
                     dtype=torch.uint8, device=dev)
    g = ttcd.fastweight_scan_backward(zt, zs, zt, *wt, beta, dy, cfg.chunk,
                                      out_dtype=torch.bfloat16, workspace=ws)
    st = torch.cuda.current_stream()
    bwd_ms = time_events(lambda: ttcd.fastweight_scan_backward(
        zt, zs, zt, *wt, beta, dy, cfg.chunk, out_dtype=torch.bfloat16, out=g, workspace=ws),
        n, st, 3)
    fwd_ms = time_events(lambda: ttcd.fastweight_scan(zt, zs, zt, *wt, beta, cfg.chunk,
                                                      workspace=ws), n, st, 3)
    finite = all(torch.isfinite(t).all().item() for t in g.values())
    ws_gb = ws.numel() / 1e9
    del zt, zs, wt, beta, dy, g, ws
    return {"kernel": "fast-weight path backward (ttcd_fastweight_scan_backward): gradients of "
                      "z_T, z_S, z_main, both convs, W_down0, W_proj and beta",
            "ms_per_call": bwd_ms, "forward_ms_per_call": fwd_ms, "bwd_over_fwd": bwd_ms / fwd_ms,
            "workspace_gb": ws_gb, "finite": finite, "tokens": cfg.batch * cfg.seq}


def attn_backward_bench(cfg, dev, n):
    """The dual-window attention's gradient (ttcd_dual_window_attn_backward)
    at the workload's size.  Algorithmic flops: five products over the
    teacher window's (query, key) pairs (S recomputed, dP, dV, dQ, dK:
    2.5 x the forward's) plus two over the student window's (its dP and dV)."""
    import torch
    from dual_window_attention_amd import inputs as I
    from dual_window_attention_amd import ttcd

    att = I.attention_inputs(cfg)
    q, k, v = (I.to_torch(att[n], dev) for n in ("q", "k", "v"))
    del att
    wT, wS = cfg.w_teacher, cfg.w_student
    o_t, o_s, l_t, l_s = ttcd.dual_window_attn(q, k, v, wT, wS, out_dtype=torch.bfloat16)
    gen = torch.Generator().manual_seed(6)
    do_t = torch.randn(q.shape, generator=gen).to(dev, torch.bfloat16)
    do_s = torch.randn(q.shape, generator=gen).to(dev, torch.bfloat16)
    lib = ttcd.lib()
    ws = torch.empty(lib.ttcd_dual_window_attn_backward_workspace_size(
        ttcd.attn_desc(q, k, wT, wS)), dtype=torch.uint8, device=dev)
    g = ttcd.dual_window_attn_backward(q, k, v, o_t, o_s, l_t, l_s, do_t, do_s, wT, wS,
                                       workspace=ws)
    st = torch.cuda.current_stream()
    ms = time_events(lambda: ttcd.dual_window_attn_backward(
        q, k, v, o_t, o_s, l_t, l_s, do_t, do_s, wT, wS, out=g, workspace=ws), n, st, 2)
    flops = 2.5 * attention_flops(cfg, wT) + attention_flops(cfg, wS)
    finite = all(torch.isfinite(t).all().item() for t in g)
    del q, k, v, o_t, o_s, l_t, l_s, do_t, do_s, ws, g
    achieved = flops / (ms * 1e-3) / 1e12
    return {"kernel": "dual-window attention backward (ttcd_dual_window_attn_backward): dq, dk, "
                      "dv in bf16",
            "ms_per_call": ms, "algorithmic_tflop": flops / 1e12, "achieved": achieved,
            "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "finite": finite}


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
        # the same step captured once in a HIP graph and replayed (the
        # library's calls are kernel launches only, so they capture whole)
        try:
            ref = out.clone()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            gms = time_events(graph.replay, n, stream, warmup=3)
            torch.cuda.synchronize()
            res[form].update({"graph_ms_per_step": gms, "graph_tokens_per_s": B / (gms * 1e-3),
                              "graph_hbm_frac": gb / (gms * 1e-3) / PEAK_HBM_GBS,
                              "graph_equals_eager": bool(torch.equal(out, ref))})
            del graph
        except RuntimeError as e:       # report, keep the rest of the run
            res[form]["graph_error"] = str(e)[:200]
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
    """The fp64 oracle, as it stands, on two prefixes of the same inputs
    (same shapes, weights and windows): the first ``sample_tokens`` tokens
    and the first ``sample_tokens - w_T`` tokens.  Both prefixes are past the
    window ramp by then, so the difference of their wall times is the
    oracle's steady-state cost of ``w_T`` tokens with full windows; that
    rate is the value, the whole-sample rate is reported beside it."""
    from dual_window_attention_amd import inputs as I
    from oracle import ttcd_oracle as O

    def run(tokens):
        sc = cfg.scaled(seq=tokens)
        att = I.attention_inputs(sc)
        w = {n: t.f64() for n, t in I.layer_weights(sc).items()}
        w["beta"] = I.beta_for(sc).astype(np.float64)
        x = I.residual_input(sc).f64()
        q, k, v = att["q"].f64(), att["k"].f64(), att["v"].f64()
        t0 = time.perf_counter()
        O.layer_forward(q, k, v, x, w, sc.w_teacher, sc.w_student, sc.chunk)
        return time.perf_counter() - t0

    short = sample_tokens - cfg.w_teacher
    if short < cfg.w_teacher:
        raise ValueError("the CPU sample must cover at least two teacher windows")
    wall_long = run(sample_tokens)
    wall_short = run(short)
    steady = cfg.w_teacher * cfg.batch / max(wall_long - wall_short, 1e-9)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": steady, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "whole_sample_tokens_per_s": sample_tokens * cfg.batch / wall_long,
            "sample": f"fp64 NumPy oracle, full layer forward over the first {sample_tokens} "
                      f"and the first {short} tokens of the same config (wall {wall_long:.1f} s "
                      f"and {wall_short:.1f} s); value = the {cfg.w_teacher} tokens between "
                      f"them, all with full {cfg.w_teacher}-key windows, over the wall-time "
                      f"difference"}


def layer_inputs(cfg, dev):
    """Device inputs, weights, workspace and output of one layer step of ``cfg``."""
    import torch
    from dual_window_attention_amd import inputs as I
    from dual_window_attention_amd import ttcd

    att = I.attention_inputs(cfg)
    q, k, v = (I.to_torch(att[n], dev) for n in ("q", "k", "v"))
    del att
    wd = {n: I.to_torch(t, dev) for n, t in I.layer_weights(cfg).items()}
    wd["beta"] = I.f32_to_torch(I.beta_for(cfg), dev)
    x = I.to_torch(I.residual_input(cfg), dev)
    ws = torch.empty(ttcd.layer_workspace_bytes(q, k, cfg.d_model, cfg.d_ff, cfg.w_teacher,
                                                cfg.w_student, cfg.chunk, cfg.conv_k),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.batch, cfg.seq, cfg.d_model), dtype=torch.float32, device=dev)
    return q, k, v, x, wd, ws, out


def attention_call(cfg, dev, q, k, v, w_t, w_s, n):
    """Mean time of the fused dual-window attention call (V^T prologue and
    kernel, bf16 outputs, no LSE) and its fraction of the bf16 MFMA peak."""
    import torch
    from dual_window_attention_amd import ttcd

    o_t = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    o_s = torch.empty_like(o_t)
    aws = torch.empty(max(256, ttcd.lib().ttcd_dual_window_attn_workspace_size(
        ttcd.attn_desc(q, k, w_t, w_s))), dtype=torch.uint8, device=dev)
    ms = time_events(lambda: ttcd.dual_window_attn(q, k, v, w_t, w_s, with_lse=False,
                                                   out=(o_t, o_s), workspace=aws),
                     n, torch.cuda.current_stream())
    flops = attention_flops(cfg, w_t)
    achieved = flops / (ms * 1e-3) / 1e12
    return {"w_teacher": w_t, "w_student": w_s, "ms_per_launch": ms,
            "algorithmic_tflop": flops / 1e12, "achieved_tflops": achieved,
            "mfma_frac": achieved / PEAK_BF16_TFLOPS}


def smollm2_bench(dev, steps, n):
    """The SmolLM2-360M-shaped layer at 16K (batch 1, 15/5 heads x 64, d_model
    960, d_ff 2560, w_T 4096, w_S 256, chunk 512): layer tokens/s, the
    attention call's fraction of the MFMA peak and the stream's of HBM."""
    import torch
    from dual_window_attention_amd import inputs as I
    from dual_window_attention_amd import ttcd

    cfg = I.CONFIGS[2]
    q, k, v, x, wd, ws, out = layer_inputs(cfg, dev)

    def step():
        ttcd.layer_forward(q, k, v, x, wd, cfg.w_teacher, cfg.w_student, cfg.chunk, out=out,
                           workspace=ws)

    ms = time_events(step, steps, torch.cuda.current_stream(), warmup=3)
    assert torch.isfinite(out).all().item()
    res = {"workload": f"{cfg.name}: IP-TTCD layer forward, batch {cfg.batch}, seq {cfg.seq}, "
                       f"{cfg.n_q_heads}/{cfg.n_kv_heads} heads x {cfg.head_dim}, d_model "
                       f"{cfg.d_model}, d_ff {cfg.d_ff}, w_T {cfg.w_teacher}, w_S "
                       f"{cfg.w_student}, chunk {cfg.chunk}",
           "ms_per_step": ms, "tokens_per_s": cfg.batch * cfg.seq / (ms * 1e-3)}
    res["attention"] = attention_call(cfg, dev, q, k, v, cfg.w_teacher, cfg.w_student, n)
    del q, k, v, x, wd, ws, out
    torch.cuda.empty_cache()
    res["scan"] = scan_roofline(cfg, dev, n, counters=False)
    return res


def attention_sweep_bench(dev, n):
    """The attention-only workload (batch 8, 32K, 16/8 heads x 128, 5 % of
    key rows x8) at its three (w_T, w_S) pairs: fraction of the MFMA peak."""
    import torch
    from dual_window_attention_amd import inputs as I

    cfg = I.CONFIGS[4]
    att = I.attention_inputs(cfg)
    q, k, v = (I.to_torch(att[nm], dev) for nm in ("q", "k", "v"))
    del att
    pairs = [attention_call(cfg, dev, q, k, v, w_t, w_s, n) for w_t, w_s in cfg.windows]
    del q, k, v
    torch.cuda.empty_cache()
    return {"workload": f"{cfg.name}: dual-window attention, batch {cfg.batch}, seq {cfg.seq}, "
                        f"{cfg.n_q_heads}/{cfg.n_kv_heads} heads x {cfg.head_dim}, 5% of key "
                        f"rows x8", "pairs": pairs}


def summarize_trace(path, dispatch_regex=None):
    """Per-shape table of a rocprofv3 CSV: a kernel trace (duration of each
    dispatch) or a counter collection (value of each counter per dispatch),
    grouped by kernel name and grid size, so that launches of one kernel at
    different shapes are not averaged together.

    For a counter collection holding SQ_VALU_MFMA_BUSY_CYCLES and
    GRBM_GUI_ACTIVE it adds, per group, the matrix-core busy fraction
    BUSY / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8 XCDs) and the shader clock
    GRBM_GUI_ACTIVE / 8 / duration.  With ``dispatch_regex`` it lists every
    matching dispatch in issue order instead (index among the matches, grid,
    duration or counter values), so that calls of one kernel at one grid but
    different windows can be told apart by their place in the run."""
    import csv
    import re
    from collections import OrderedDict

    groups = OrderedDict()
    per_dispatch = OrderedDict()
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name", "?")
            if "Grid_Size" in row:
                grid = row["Grid_Size"]
            else:
                grid = "x".join(row.get(f"Grid_Size_{a}", "?") for a in "XYZ")
            dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            if "Counter_Name" in row:
                key = (name, grid, row["Counter_Name"])
                val = float(row["Counter_Value"])
                d = per_dispatch.setdefault(row["Dispatch_Id"], {"name": name, "grid": grid,
                                                                "duration_us": dur})
                d[row["Counter_Name"]] = val
            else:
                key = (name, grid, "duration_us")
                val = dur
                per_dispatch[row.get("Dispatch_Id", str(len(per_dispatch)))] = {
                    "name": name, "grid": grid, "duration_us": dur}
            groups.setdefault(key, []).append(val)
    if dispatch_regex:
        rx = re.compile(dispatch_regex)
        qty = None
        print(f"{'#':>4} {'dispatch':>9} {'grid':>22}  values")
        i = 0
        for did, d in per_dispatch.items():
            if not rx.search(d["name"]):
                continue
            vals = {k: v for k, v in d.items() if k not in ("name", "grid")}
            if qty is None:
                qty = sorted(vals)
            print(f"{i:>4} {did:>9} {d['grid']:>22}  " +
                  "  ".join(f"{k}={vals[k]:.6g}" for k in qty if k in vals))
            i += 1
        return
    print(f"{'kernel':<58} {'grid':>22} {'quantity':>26} {'n':>5} {'mean':>12} {'min':>12} "
          f"{'max':>12}")
    for (name, grid, qty), vals in groups.items():
        short = name if len(name) <= 58 else name[:55] + "..."
        print(f"{short:<58} {grid:>22} {qty:>26} {len(vals):>5} {np.mean(vals):>12.4g} "
              f"{np.min(vals):>12.4g} {np.max(vals):>12.4g}")
    # derived: matrix-core busy fraction and clock per (kernel, grid)
    derived = OrderedDict()
    for d in per_dispatch.values():
        if "SQ_VALU_MFMA_BUSY_CYCLES" in d and "GRBM_GUI_ACTIVE" in d:
            derived.setdefault((d["name"], d["grid"]), []).append(d)
    if derived:
        print()
        print(f"{'kernel':<58} {'grid':>22} {'n':>5} {'mfma_busy_frac':>15} {'clock_GHz':>10}")
        for (name, grid), ds in derived.items():
            busy = np.mean([x["SQ_VALU_MFMA_BUSY_CYCLES"] for x in ds])
            act = np.mean([x["GRBM_GUI_ACTIVE"] for x in ds]) / 8.0
            dur = np.mean([x["duration_us"] for x in ds])
            short = name if len(name) <= 58 else name[:55] + "..."
            print(f"{short:<58} {grid:>22} {len(ds):>5} {busy / 1024.0 / act:>15.3f} "
                  f"{act / dur / 1e3:>10.2f}")


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
    ap.add_argument("--no-backward", action="store_true", help="skip the gradient section")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 16K SmolLM2-shaped layer and the batch-8 attention sweep")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="print a per-shape table of a rocprofv3 kernel-trace or counter CSV "
                         "and exit (no GPU work)")
    ap.add_argument("--dispatches", metavar="REGEX",
                    help="with --summarize-trace: list the dispatches of the kernels matching "
                         "REGEX in issue order")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic summary under profiles/ from the FETCH_SIZE and "
                         "WRITE_SIZE counter collections of the calibration run, and exit")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (a reference "
                         "kernel of known traffic for scaling memory counters)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.dispatches)
        return
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
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
    if not args.no_backward:
        res["backward"] = backward_bench(cfg, dev, 5)
        torch.cuda.empty_cache()
        res["attention_backward"] = attn_backward_bench(cfg, dev, 3)
        torch.cuda.empty_cache()
    if not args.no_decode:
        res["decode"] = decode_bench(dev, n_att)
        torch.cuda.empty_cache()
    if not args.no_extra:
        res["config2"] = smollm2_bench(dev, max(5, args.steps), n_att)
        torch.cuda.empty_cache()
        res["config4"] = attention_sweep_bench(dev, 5)
        torch.cuda.empty_cache()
    if args.cpu_sample > 0:
        res["cpu_baseline"] = cpu_baseline(cfg, min(args.cpu_sample, cfg.seq))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
