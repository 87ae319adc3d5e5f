"""fp64 CPU oracle for the IP-TTCD layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call
this module; only the tests, the package's ``smoke()`` check and the CPU
baseline leg of the benchmark do.  It shares no code with the HIP library.

It is a plain, slow, obviously-correct restatement of what the method
computes, in float64 NumPy (BLAS matmul is the only library primitive).
Sources are the pages on "Learning What to Remember: Test-Time Training via
Context Distillation":

  [README]   the GitHub README "TTCD: Test-Time Training via Context
             Distillation" (sections "Model configuration", "Fused
             inference kernels")
  [NOTES]    the papernotes.org notes on the NeurIPS 2026 paper (method
             section: overall framework, key designs 1-4)
  [PODCAST]  the podcast transcript of the paper (cues on sliding windows,
             Eq. 4 / Eq. 6 / Eq. 12 and Proposition 1)

Readings taken where the pages leave a step open (all shared with the HIP
path and listed in the design notes):
  * window w holds w keys including the query's own position:
    key j is visible to query t iff 0 <= t - j < w;
  * the student window is a token window (not chunk aligned);
  * the teacher path is the layer's main path (its MLP output receives the
    fast weight);
  * a chunk's write acts on strictly later chunks;
  * the short conv is a full-sequence causal depthwise conv with zero left
    padding, tap kc-1 on the current token, no bias;  <- parity unpinned
    (orientation; the pages do not fix it)
  * l2 normalisation is per token over d_ff with x / max(||x||, eps);
  * beta is one scalar per (batch, chunk) and is the exact coefficient of
    R_i K_i^T;
  * layer glue: h = x + O W_o^T, RMSNorm(eps=1e-6, gain gamma), SwiGLU;
    Q/K already carry any positional encoding.  <- parity unpinned (the
    pages do not describe the glue; it is a declared standard block)

Layouts (row-major, token-major): q [B,T,Hq,D], k/v [B,Tk,Hkv,D],
x [B,T,d], w_o [d, Hq*D], w_gate/w_up [f, d], w_down0 [d, f],
w_proj [f, f], conv taps [f, kc], beta [B, n_chunks].
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


# ==========================================================================
# O1  dual-window causal sliding-window attention
#     [PODCAST] cue on sliding windows: a token attends only to the most
#     recent w tokens; [README] "Fused inference kernels": one pass yields
#     the teacher (long window) and student (short window) outputs over the
#     same Q/K/V; [NOTES] overall framework: w_S < w_T over one backbone.
# ==========================================================================


def window_attention(q, k, v, window: int, scale: Optional[float] = None,
                     q_pos0: int = 0, rows: Optional[Sequence[int]] = None,
                     block: int = 256):
    """Causal sliding-window softmax attention, one window.

    q [B,Tq,Hq,D], k/v [B,Tk,Hkv,D].  Query i sits at position q_pos0 + i;
    key j at position j.  Query head h reads kv head h // (Hq/Hkv).
    Visible set of query t: J(t) = {j : max(0, t-window+1) <= j <= t}.

    Returns o [B,Tq,Hq,D] and lse [B,Hq,Tq] (natural log), both float64:
        o[t]   = sum_{j in J} exp(s_j - m) v_j / sum_{j in J} exp(s_j - m)
        lse[t] = m + log sum_{j in J} exp(s_j - m),   s_j = scale <q_t, k_j>
    If ``rows`` is given, only those query indices are computed (others
    stay zero).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, Tq, Hq, D = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = np.zeros((B, Tq, Hq, D), F64)
    lse = np.zeros((B, Hq, Tq), F64)
    idx = np.arange(Tq) if rows is None else np.asarray(sorted(set(int(r) for r in rows)))
    if idx.size == 0:
        return o, lse
    for b in range(B):
        for s0 in range(0, idx.size, block):
            sel = idx[s0:s0 + block]
            t = q_pos0 + sel  # absolute positions
            j_lo = max(0, int(t.min()) - window + 1)
            j_hi = min(Tk - 1, int(t.max()))
            j = np.arange(j_lo, j_hi + 1)
            diff = t[:, None] - j[None, :]
            mask = (diff >= 0) & (diff < window)
            for h in range(Hq):
                g = h // G
                qs = q[b, sel, h, :]                      # [n, D]
                ks = k[b, j_lo:j_hi + 1, g, :]            # [m, D]
                vs = v[b, j_lo:j_hi + 1, g, :]
                s = (qs @ ks.T) * scale
                s = np.where(mask, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                l = p.sum(axis=1, keepdims=True)
                o[b, sel, h, :] = (p @ vs) / l
                lse[b, h, sel] = (m + np.log(l))[:, 0]
    return o, lse


def dual_window_attention(q, k, v, w_teacher: int, w_student: int,
                          scale: Optional[float] = None, q_pos0: int = 0,
                          rows: Optional[Sequence[int]] = None):
    """Teacher (w_T) and student (w_S) outputs of one shared Q/K/V.

    Returns (o_t, o_s, lse_t, lse_s).  This is the definition applied once
    per window; the single-pass fusion the pages describe is an exact
    rewrite of it ([README] "Fused inference kernels").
    """
    o_t, lse_t = window_attention(q, k, v, w_teacher, scale, q_pos0, rows)
    o_s, lse_s = window_attention(q, k, v, w_student, scale, q_pos0, rows)
    return o_t, o_s, lse_t, lse_s


def window_attention_bruteforce(q, k, v, window: int, scale: Optional[float] = None,
                                q_pos0: int = 0, band: Optional[Tuple[int, int]] = None):
    """Pure-loop version of ``window_attention`` for tiny shapes.

    ``band=(a, b)`` makes the visible keys of query t the set
    {j : a <= t - j < b}; (0, window) is the plain window.  Used to pin the
    vectorised oracle and the far-band identity.
    """
    B, Tq, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Tk, Hkv = len(k[0]), len(k[0][0])
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    a, bnd = (0, window) if band is None else band
    o = [[[[0.0] * D for _ in range(Hq)] for _ in range(Tq)] for _ in range(B)]
    lse = [[[float("-inf")] * Tq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for i in range(Tq):
            t = q_pos0 + i
            for h in range(Hq):
                g = h // G
                keys = [jj for jj in range(Tk) if a <= t - jj < bnd]
                if not keys:
                    continue
                sc = []
                for jj in keys:
                    acc = 0.0
                    for e in range(D):
                        acc += float(q[b][i][h][e]) * float(k[b][jj][g][e])
                    sc.append(acc * scale)
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                tot = sum(w)
                for e in range(D):
                    acc = 0.0
                    for wi, jj in zip(w, keys):
                        acc += wi * float(v[b][jj][g][e])
                    o[b][i][h][e] = acc / tot
                lse[b][h][i] = mx + math.log(tot)
    return np.array(o, F64), np.array(lse, F64)


# ==========================================================================
# O2-O3  half-layer glue and the SwiGLU MLP activations of both paths
#     [NOTES] key design 2: both paths' MLP activations are computed with
#     the base weights (off-policy); the glue itself is a declared standard
#     pre-norm block (parity unpinned by the pages).
# ==========================================================================


def attn_out_residual(x, o, w_o):
    """h = x + concat_heads(o) W_o^T.   x [B,T,d], o [B,T,Hq,D], w_o [d,Hq*D]."""
    o = _f64(o)
    B, T, Hq, D = o.shape
    return _f64(x) + o.reshape(B, T, Hq * D) @ _f64(w_o).T


def rmsnorm(h, gamma=None, eps: float = 1e-6):
    """u = h / sqrt(mean(h^2) + eps) * gamma, over the last axis."""
    h = _f64(h)
    u = h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    if gamma is not None:
        u = u * _f64(gamma)
    return u


def silu(a):
    a = _f64(a)
    return a / (1.0 + np.exp(-a))


def swiglu_hidden(u, w_gate, w_up):
    """Z = silu(u W_gate^T) * (u W_up^T): the input of W_down.  [.., f]"""
    u = _f64(u)
    return silu(u @ _f64(w_gate).T) * (u @ _f64(w_up).T)


# ==========================================================================
# O4-O8  fast-weight update of W_down (IP-TTCD)
#     [NOTES] key design 3 (the practical update, Eq. 12 in [PODCAST]):
#       R_i = W_down^(0) W_proj (conv_T(Z_i^T) - conv_S(Z_i^S)),
#       K_i = l2norm(conv_S(Z_i^S)),  dW_i = beta_i R_i K_i^T;
#     [NOTES] key design 2: off-policy activations at W_down^(0), causal
#     prefix sum over chunks; [README] "Fused inference kernels": the conv
#     is a chunked depthwise causal conv equal to a plain full-sequence one.
# ==========================================================================


def causal_depthwise_conv(z, taps):
    """zbar[t, c] = sum_{i=0}^{kc-1} taps[c, i] * z[t - (kc-1) + i, c],
    with z[tau < 0] = 0.  z [..., T, f], taps [f, kc]."""
    z = _f64(z)
    taps = _f64(taps)
    kc = taps.shape[1]
    T = z.shape[-2]
    out = np.zeros_like(z)
    for i in range(kc):
        shift = kc - 1 - i          # how far back tap i looks
        if shift >= T:
            continue
        if shift == 0:
            out += z * taps[:, i]
        else:
            out[..., shift:, :] += z[..., :T - shift, :] * taps[:, i]
    return out


def l2_normalize(x, eps: float = 1e-12):
    """x / max(||x||_2, eps) over the last axis (a zero row stays zero)."""
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def fastweight_terms(z_t, z_s, conv_t, conv_s, w_down0, w_proj, eps: float = 1e-12):
    """Per-token write terms of one sequence.

    Returns (r [T, d], k [T, f], dbar [T, f], zbar_s [T, f]):
        dbar_t = conv_T(Z^T)_t - conv_S(Z^S)_t
        r_t    = W_down^(0) (W_proj dbar_t)
        k_t    = conv_S(Z^S)_t / max(||conv_S(Z^S)_t||, eps)
    """
    zb_t = causal_depthwise_conv(z_t, conv_t)
    zb_s = causal_depthwise_conv(z_s, conv_s)
    dbar = zb_t - zb_s
    r = (dbar @ _f64(w_proj).T) @ _f64(w_down0).T
    k = l2_normalize(zb_s, eps)
    return r, k, dbar, zb_s


def chunk_bounds(T: int, C: int) -> List[Tuple[int, int]]:
    return [(i, min(i + C, T)) for i in range(0, T, C)]


def fastweight_apply_prefix(r, k, beta, z_main, w_down0, C: int,
                            return_states: bool = False):
    """Running causal prefix over chunks (one sequence).

        S_0 = W_down^(0),   S_{i+1} = S_i + beta_i R_i^T K_i
        y_t = S_{floor(t/C)} z_main[t]

    r [T,d], k [T,f], beta [n], z_main [T,f]  ->  y [T,d] (and S_N).
    """
    r, k, z = _f64(r), _f64(k), _f64(z_main)
    T = z.shape[0]
    S = _f64(w_down0).copy()
    y = np.zeros((T, S.shape[0]), F64)
    states = []
    for i, (a, b) in enumerate(chunk_bounds(T, C)):
        if return_states:
            states.append(S.copy())
        y[a:b] = z[a:b] @ S.T
        S = S + float(beta[i]) * (r[a:b].T @ k[a:b])
    if return_states:
        return y, S, states
    return y, S


def fastweight_apply_explicit(r, k, beta, z_main, w_down0, C: int):
    """Same result, each chunk's weight summed afresh from the explicit
    per-chunk updates: S_i = W_down^(0) + sum_{j<i} dW_j."""
    r, k, z = _f64(r), _f64(k), _f64(z_main)
    T = z.shape[0]
    bounds = chunk_bounds(T, C)
    dWs = [float(beta[j]) * (r[a:b].T @ k[a:b]) for j, (a, b) in enumerate(bounds)]
    y = np.zeros((T, w_down0.shape[0]), F64)
    for i, (a, b) in enumerate(bounds):
        S = _f64(w_down0).copy()
        for j in range(i):
            S = S + dWs[j]
        y[a:b] = z[a:b] @ S.T
    return y


def fastweight_apply_lowrank(r, k, beta, z_main, w_down0, C: int):
    """Same result in low-rank form, never forming a d x f update:
        y_t = W_down^(0) z_t + sum_{j < i} beta_j R_j^T (K_j z_t)."""
    r, k, z = _f64(r), _f64(k), _f64(z_main)
    T = z.shape[0]
    bounds = chunk_bounds(T, C)
    y = z @ _f64(w_down0).T
    for i, (a, b) in enumerate(bounds):
        for j in range(i):
            ja, jb = bounds[j]
            y[a:b] += float(beta[j]) * ((z[a:b] @ k[ja:jb].T) @ r[ja:jb])
    return y


def fastweight_scan(z_t, z_s, z_main, conv_t, conv_s, w_down0, w_proj, beta,
                    C: int, eps: float = 1e-12, form: str = "prefix"):
    """Fast-weight stream + prefix + apply for a batch.

    z_* [B,T,f], beta [B, n_chunks].  Returns dict with y [B,T,d],
    state [B,d,f] (= S_N, the weight after every chunk's write),
    state_complete [B,d,f] (= S_n, n = T // C: the weight after the writes
    of the chunks that hold all C tokens -- a short last chunk is still
    pending, its writes take effect once it completes, the decode position
    convention), r [B,T,d], k [B,T,f] (unit keys), dbar [B,T,f].
    """
    z_t, z_s, z_main = _f64(z_t), _f64(z_s), _f64(z_main)
    B, T, f = z_t.shape
    d = w_down0.shape[0]
    y = np.zeros((B, T, d), F64)
    st = np.zeros((B, d, f), F64)
    st_done = np.zeros((B, d, f), F64)
    rr = np.zeros((B, T, d), F64)
    kk = np.zeros((B, T, f), F64)
    dd = np.zeros((B, T, f), F64)
    n_done = T // C
    for b in range(B):
        r, k, dbar, _ = fastweight_terms(z_t[b], z_s[b], conv_t, conv_s, w_down0, w_proj, eps)
        if form == "prefix":
            yb, S, states = fastweight_apply_prefix(r, k, beta[b], z_main[b], w_down0, C,
                                                    return_states=True)
            st_done[b] = S if n_done == len(states) else states[n_done]
        elif form == "explicit":
            yb = fastweight_apply_explicit(r, k, beta[b], z_main[b], w_down0, C)
            S = None
        elif form == "lowrank":
            yb = fastweight_apply_lowrank(r, k, beta[b], z_main[b], w_down0, C)
            S = None
        else:
            raise ValueError(form)
        y[b] = yb
        if S is not None:
            st[b] = S
        rr[b], kk[b], dd[b] = r, k, dbar
    return {"y": y, "state": st, "state_complete": st_done, "r": rr, "k": kk, "dbar": dd}


def fastweight_scan_on_policy(z_t, z_s, z_main, conv_t, conv_s, w_down0, w_proj, beta,
                              C: int, eps: float = 1e-12):
    """The sequential recurrence that the off-policy scan approximates
    ([NOTES] key design 2: chunk i should see the weight left by chunk i-1;
    [PODCAST] Eq. 12 cue: the parallel scan instead evaluates everything at
    the base weight).  Chunk by chunk, one sequence at a time:

        y_t     = S_i z_main[t]                      for t in chunk i
        r_t     = S_i (W_proj dbar_t)                (residual at S_i)
        S_{i+1} = S_i + beta_i R_i^T K_i,            S_0 = W_down^(0)

    dbar and the unit keys are those of ``fastweight_terms`` (they do not
    depend on the weight).  Returns dict with y [B,T,d], state [B,d,f]
    (= S_N) and state_complete (the weight after the complete chunks, as in
    ``fastweight_scan``)."""
    z_t, z_s, z_main = _f64(z_t), _f64(z_s), _f64(z_main)
    B, T, f = z_t.shape
    d = w_down0.shape[0]
    wp = _f64(w_proj)
    y = np.zeros((B, T, d), F64)
    st = np.zeros((B, d, f), F64)
    st_done = np.zeros((B, d, f), F64)
    for b in range(B):
        _, k, dbar, _ = fastweight_terms(z_t[b], z_s[b], conv_t, conv_s, w_down0, w_proj, eps)
        S = _f64(w_down0).copy()
        st_done[b] = S
        for i, (a, e) in enumerate(chunk_bounds(T, C)):
            y[b, a:e] = z_main[b, a:e] @ S.T
            r = (dbar[a:e] @ wp.T) @ S.T
            S = S + float(beta[b, i]) * (r.T @ k[a:e])
            if e - a == C:
                st_done[b] = S
        st[b] = S
    return {"y": y, "state": st, "state_complete": st_done}


def fastweight_scan_eq6(z_t, z_s, z_main, w_down0, beta, C: int):
    """The unprojected write of the distillation gradient ([PODCAST] Eq. 4
    and Eq. 6 cues), off-policy at W_down^(0), with no convs, no W_proj and
    no key normalisation.  Chunk i's loss is half the squared gap between the
    student's MLP output W z_S and the detached teacher's W0 z_T; its
    gradient in W at W0 is  sum_t (W0 z_S,t - W0 z_T,t) z_S,t^T, and the
    write is beta_i times its negative:

        dW_i    = beta_i sum_{t in chunk i} W0 (z_T,t - z_S,t) z_S,t^T
        S_{i+1} = S_i + dW_i,   S_0 = W0,   y_t = S_{floor(t/C)} z_main[t]

    Returns dict with y [B,T,d], state [B,d,f] (= S_N), state_complete
    (the weight after the complete chunks) and dw [B,N,d,f]."""
    z_t, z_s, z_main = _f64(z_t), _f64(z_s), _f64(z_main)
    w0 = _f64(w_down0)
    B, T, f = z_t.shape
    bounds = chunk_bounds(T, C)
    y = np.zeros((B, T, w0.shape[0]), F64)
    st = np.zeros((B,) + w0.shape, F64)
    st_done = np.zeros((B,) + w0.shape, F64)
    dws = np.zeros((B, len(bounds)) + w0.shape, F64)
    for b in range(B):
        S = w0.copy()
        st_done[b] = S
        for i, (a, e) in enumerate(bounds):
            y[b, a:e] = z_main[b, a:e] @ S.T
            gap = (z_t[b, a:e] - z_s[b, a:e]) @ w0.T         # teacher - student outputs
            dws[b, i] = float(beta[b, i]) * (gap.T @ z_s[b, a:e])
            S = S + dws[b, i]
            if e - a == C:
                st_done[b] = S
        st[b] = S
    return {"y": y, "state": st, "state_complete": st_done, "dw": dws}


# ==========================================================================
# full layer (prefill) and one decode step
# ==========================================================================


def layer_forward(q, k, v, x, w, w_teacher: int, w_student: int, C: int,
                  rms_eps: float = 1e-6, l2_eps: float = 1e-12,
                  main_path: str = "teacher", scale: Optional[float] = None):
    """IP-TTCD layer forward from Q/K/V onward (prefill).

    w: dict with w_o, gamma, w_gate, w_up, w_down0, w_proj, conv_t, conv_s,
    beta [B, n].  Returns dict with out [B,T,d] and the intermediates.
    """
    o_t, o_s, lse_t, lse_s = dual_window_attention(q, k, v, w_teacher, w_student, scale)
    h_t = attn_out_residual(x, o_t, w["w_o"])
    h_s = attn_out_residual(x, o_s, w["w_o"])
    z_t = swiglu_hidden(rmsnorm(h_t, w.get("gamma"), rms_eps), w["w_gate"], w["w_up"])
    z_s = swiglu_hidden(rmsnorm(h_s, w.get("gamma"), rms_eps), w["w_gate"], w["w_up"])
    z_main, h_main = (z_t, h_t) if main_path == "teacher" else (z_s, h_s)
    fw = fastweight_scan(z_t, z_s, z_main, w["conv_t"], w["conv_s"], w["w_down0"],
                         w["w_proj"], w["beta"], C, l2_eps)
    out = h_main + fw["y"]
    return {"out": out, "o_t": o_t, "o_s": o_s, "lse_t": lse_t, "lse_s": lse_s,
            "h_t": h_t, "h_s": h_s, "z_t": z_t, "z_s": z_s, "y": fw["y"],
            "r": fw["r"], "k": fw["k"], "dbar": fw["dbar"], "state": fw["state"],
            "state_complete": fw["state_complete"]}


def decode_step(q, k_cache, v_cache, x, w, pos: int, w_teacher: int, w_student: int,
                r_list, k_list, beta_list, C: int, rms_eps: float = 1e-6,
                scale: Optional[float] = None, key_offset: int = 0):
    """One generated token per sequence at absolute position ``pos``.

    q [B,1,Hq,D]; k_cache/v_cache [B, M, Hkv, D] hold keys at positions
    key_offset .. key_offset+M-1 (the new token's key included, at ``pos``).
    The fast weight is taken straight from the chunk lists (low-rank form):
        y = W_down^(0) z + sum_j beta_j R_j^T (K_j z)
    r_list [B, n*C, d], k_list [B, n*C, f] (unit keys), beta_list [B, n];
    the lists may be sequences of per-batch arrays (converted slice by slice).
    """
    B = q.shape[0]
    # positions relative to the slice held in the cache arrays
    qpos = pos - key_offset
    o_t, o_s, lse_t, lse_s = dual_window_attention(q, k_cache, v_cache, w_teacher,
                                                   w_student, scale, q_pos0=qpos)
    h = attn_out_residual(x, o_t, w["w_o"])
    z = swiglu_hidden(rmsnorm(h, w.get("gamma"), rms_eps), w["w_gate"], w["w_up"])
    y = z @ _f64(w["w_down0"]).T
    n = beta_list.shape[1]
    for b in range(B):
        rb, kb = r_list[b], k_list[b]
        for j in range(n):
            a, e = j * C, (j + 1) * C
            y[b] += float(beta_list[b, j]) * ((z[b] @ _f64(kb[a:e]).T) @ _f64(rb[a:e]))
    return {"out": h + y, "o_t": o_t, "o_s": o_s, "lse_t": lse_t, "lse_s": lse_s,
            "h": h, "z": z, "y": y}


def fold_lists(w_down0, r_list, k_list, beta_list, C: int):
    """Dense weight from chunk lists: W_down^(0) + sum_j beta_j R_j^T K_j."""
    r_list, k_list = _f64(r_list), _f64(k_list)
    B = r_list.shape[0]
    out = np.repeat(_f64(w_down0)[None], B, axis=0)
    for b in range(B):
        for j in range(beta_list.shape[1]):
            a, e = j * C, (j + 1) * C
            out[b] += float(beta_list[b, j]) * (r_list[b, a:e].T @ k_list[b, a:e])
    return out


def decode_append(z_t, z_s, hist_t, hist_s, conv_t, conv_s, w_down0, w_proj,
                  eps: float = 1e-12):
    """The per-token write terms of one generated token ([NOTES] key design
    3; [PODCAST] Eq. 12), from the new token's SwiGLU outputs of both paths
    and each path's last kc-1 inputs (the history, oldest first).

    z_t, z_s [B, f]; hist_t, hist_s [B, kc-1, f]; taps [f, kc] with tap kc-1
    on the new token (the reading of the conv above).  Returns
    (r [B, d], k [B, f], dbar [B, f], new hist_t, new hist_s):
        zbar_p = sum_i taps_p[:, i] * window_p[i],  window_p = [hist_p; z_p]
        dbar   = zbar_T - zbar_S,  r = W_down^(0) (W_proj dbar),
        k      = zbar_S / max(||zbar_S||, eps)
    and each history with its oldest row dropped and the token appended.
    """
    z_t, z_s = _f64(z_t), _f64(z_s)
    hist_t, hist_s = _f64(hist_t), _f64(hist_s)
    taps_t, taps_s = _f64(conv_t), _f64(conv_s)
    win_t = np.concatenate([hist_t, z_t[:, None, :]], axis=1)      # [B, kc, f]
    win_s = np.concatenate([hist_s, z_s[:, None, :]], axis=1)
    zb_t = np.einsum("bif,fi->bf", win_t, taps_t)
    zb_s = np.einsum("bif,fi->bf", win_s, taps_s)
    dbar = zb_t - zb_s
    r = (dbar @ _f64(w_proj).T) @ _f64(w_down0).T
    k = l2_normalize(zb_s, eps)
    return r, k, dbar, win_t[:, 1:, :], win_s[:, 1:, :]


# ==========================================================================
# Backward pass (the gradient of the forward above; the pages give only its
# cost, 1.1-1.2x of a standard layer in training: [NOTES] 局限与展望,
# [PODCAST] the cue on training overhead).  Each function is the vector-
# Jacobian product of the matching forward, written step by step with the
# chain rule in the forward's own notation.
# ==========================================================================


def causal_depthwise_conv_backward(z, taps, dzbar):
    """Gradients of zbar = causal_depthwise_conv(z, taps) given dzbar.

    zbar[t, c] = sum_i taps[c, i] z[t - (kc-1) + i, c]  gives
        dz[tau, c]    = sum_i taps[c, i] dzbar[tau + (kc-1) - i, c]   (t < T)
        dtaps[c, i]   = sum_t dzbar[t, c] z[t - (kc-1) + i, c]        (tau >= 0)
    z, dzbar [T, f]; taps [f, kc].  Returns (dz [T, f], dtaps [f, kc])."""
    z, taps, dzbar = _f64(z), _f64(taps), _f64(dzbar)
    T = z.shape[0]
    kc = taps.shape[1]
    dz = np.zeros_like(z)
    dtaps = np.zeros_like(taps)
    for i in range(kc):
        shift = kc - 1 - i
        if shift >= T:
            continue
        # zbar[t] takes z[t - shift] through tap i, for t >= shift
        dz[:T - shift] += dzbar[shift:] * taps[:, i]
        dtaps[:, i] = np.sum(dzbar[shift:] * z[:T - shift], axis=0)
    return dz, dtaps


def l2_normalize_backward(x, dk, eps: float = 1e-12):
    """Gradient of k = x / max(||x||, eps) (per row) given dk:
    (dk - k (k . dk)) / ||x|| where ||x|| > eps, else dk / eps."""
    x, dk = _f64(x), _f64(dk)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    big = n > eps
    k = x / np.maximum(n, eps)
    proj = dk - k * np.sum(k * dk, axis=-1, keepdims=True)
    return np.where(big, proj / np.maximum(n, eps), dk / eps)


def fastweight_scan_backward(z_t, z_s, z_main, conv_t, conv_s, w_down0, w_proj, beta,
                             C: int, dy, eps: float = 1e-12):
    """Gradients of y = fastweight_scan(...)["y"] (off-policy rule) given dy.

    With S_i the weight in force for chunk i (S_0 = W_down^(0)), the forward
    is y_t = S_{c(t)} z_main[t], S_{i+1} = S_i + beta_i R_i^T K_i,
    r_t = W_down^(0) q_t, q_t = W_proj dbar_t, dbar = zbar_T - zbar_S,
    k_t = zbar_S[t] / max(||zbar_S[t]||, eps).  Backward, per sequence:
        dS_i       = sum_{t in C_i} dy_t z_main[t]^T        (the apply)
        dz_main[t] = S_{c(t)}^T dy_t
        G_j        = sum_{i > j} dS_i                        (chunk j's write
                                                              reaches every
                                                              later chunk)
        dbeta_j    = sum_{t in C_j} r_t . (G_j k_t)
        dr_t       = beta_j G_j k_t,   dk_t = beta_j G_j^T r_t
        dW_down0   = sum_i dS_i + sum_t dr_t q_t^T,   dq_t = W_down0^T dr_t
        dW_proj    = sum_t dq_t dbar_t^T,             ddbar_t = W_proj^T dq_t
        dzbar_S    = l2 backward of dk - ddbar,   dzbar_T = ddbar
    and the conv backward of each path.  Returns dz_t, dz_s, dz_main [B,T,f],
    dconv_t, dconv_s [f,kc], dw_down0 [d,f], dw_proj [f,f], dbeta [B,n]
    (weights are shared by the batch: their gradients are summed over it)."""
    z_t, z_s, z_main, dy = _f64(z_t), _f64(z_s), _f64(z_main), _f64(dy)
    w0, wp = _f64(w_down0), _f64(w_proj)
    B, T, f = z_t.shape
    d = w0.shape[0]
    bounds = chunk_bounds(T, C)
    out = {"dz_t": np.zeros_like(z_t), "dz_s": np.zeros_like(z_s),
           "dz_main": np.zeros_like(z_main), "dconv_t": np.zeros_like(_f64(conv_t)),
           "dconv_s": np.zeros_like(_f64(conv_s)), "dw_down0": np.zeros_like(w0),
           "dw_proj": np.zeros_like(wp), "dbeta": np.zeros((B, len(bounds)), F64)}
    for b in range(B):
        zb_t = causal_depthwise_conv(z_t[b], conv_t)
        zb_s = causal_depthwise_conv(z_s[b], conv_s)
        dbar = zb_t - zb_s
        q = dbar @ wp.T
        r = q @ w0.T
        k = l2_normalize(zb_s, eps)
        # forward states and the apply's backward
        S = w0.copy()
        dS = []
        for i, (a, e) in enumerate(bounds):
            out["dz_main"][b, a:e] = dy[b, a:e] @ S
            dS.append(dy[b, a:e].T @ z_main[b, a:e])
            S = S + float(beta[b, i]) * (r[a:e].T @ k[a:e])
        # exclusive suffix sums of the chunk gradients
        G = [None] * len(bounds)
        acc = np.zeros((d, f), F64)
        for j in range(len(bounds) - 1, -1, -1):
            G[j] = acc.copy()
            acc = acc + dS[j]
        out["dw_down0"] += acc                       # sum_i dS_i
        dr = np.zeros_like(r)
        dk = np.zeros_like(k)
        for j, (a, e) in enumerate(bounds):
            gk = k[a:e] @ G[j].T                     # rows: G_j k_t
            out["dbeta"][b, j] = float(np.sum(r[a:e] * gk))
            dr[a:e] = float(beta[b, j]) * gk
            dk[a:e] = float(beta[b, j]) * (r[a:e] @ G[j])
        out["dw_down0"] += dr.T @ q
        dq = dr @ w0
        out["dw_proj"] += dq.T @ dbar
        ddbar = dq @ wp
        dzb_s = l2_normalize_backward(zb_s, dk, eps) - ddbar
        dzb_t = ddbar
        dz, dtap = causal_depthwise_conv_backward(z_t[b], conv_t, dzb_t)
        out["dz_t"][b] = dz
        out["dconv_t"] += dtap
        dz, dtap = causal_depthwise_conv_backward(z_s[b], conv_s, dzb_s)
        out["dz_s"][b] = dz
        out["dconv_s"] += dtap
    return out


def window_attention_backward(q, k, v, o, lse, do, window: int, scale: Optional[float] = None):
    """Gradients of o = window_attention(q, k, v, window)[0] given do, from
    the forward's o and lse (the softmax weights are P = exp(s - lse) on the
    visible keys):
        dV_j  = sum_t P_tj dO_t
        dP_tj = dO_t . v_j,   D_t = dO_t . o_t,   dS_tj = P_tj (dP_tj - D_t)
        dQ_t  = scale sum_j dS_tj k_j,   dK_j = scale sum_t dS_tj q_t
    q [B,T,Hq,D], k/v [B,T,Hkv,D]; a kv head's gradient sums its q heads.
    Returns (dq, dk, dv)."""
    q, k, v, o, do = _f64(q), _f64(k), _f64(v), _f64(o), _f64(do)
    lse = _f64(lse)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    t = np.arange(T)
    diff = t[:, None] - t[None, :]
    mask = (diff >= 0) & (diff < window)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = (q[b, :, h] @ k[b, :, g].T) * scale
            p = np.where(mask, np.exp(s - lse[b, h][:, None]), 0.0)
            dp = do[b, :, h] @ v[b, :, g].T
            dd = np.sum(do[b, :, h] * o[b, :, h], axis=-1, keepdims=True)
            ds = p * (dp - dd)
            dv[b, :, g] += p.T @ do[b, :, h]
            dq[b, :, h] = scale * (ds @ k[b, :, g])
            dk[b, :, g] += scale * (ds.T @ q[b, :, h])
    return dq, dk, dv


def dual_window_attention_backward(q, k, v, w_teacher: int, w_student: int, do_t, do_s,
                                   scale: Optional[float] = None):
    """Gradients of the teacher and student outputs of one shared Q/K/V given
    dO_T and dO_S: the two windows' gradients add, since both read the same
    q, k and v."""
    o_t, o_s, lse_t, lse_s = dual_window_attention(q, k, v, w_teacher, w_student, scale)
    gq_t, gk_t, gv_t = window_attention_backward(q, k, v, o_t, lse_t, do_t, w_teacher, scale)
    gq_s, gk_s, gv_s = window_attention_backward(q, k, v, o_s, lse_s, do_s, w_student, scale)
    return gq_t + gq_s, gk_t + gk_s, gv_t + gv_s
