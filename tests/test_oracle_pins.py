"""Pins of the fp64 oracle against facts fixed outside the oracle itself:
brute force on tiny inputs, library routines, closed forms, invariants and
special cases of the method.  CPU only.

Each test names what a plausible slip in the oracle would break.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ttcd_oracle as O

torch.set_default_dtype(torch.float64)


def rnd(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def small_layer_weights(rng, d, f, HD, kc=4):
    return {
        "w_o": rnd(rng, d, HD, scale=1 / math.sqrt(HD)),
        "gamma": 1.0 + 0.1 * rnd(rng, d),
        "w_gate": rnd(rng, f, d, scale=1 / math.sqrt(d)),
        "w_up": rnd(rng, f, d, scale=1 / math.sqrt(d)),
        "w_down0": rnd(rng, d, f, scale=1 / math.sqrt(f)),
        "w_proj": rnd(rng, f, f, scale=1 / math.sqrt(f)),
        "conv_t": rnd(rng, f, kc, scale=0.5),
        "conv_s": rnd(rng, f, kc, scale=0.5),
    }


# --------------------------------------------------------------------------
# O1 attention
# --------------------------------------------------------------------------

ATTN_SHAPES = [
    # B, T, Hq, Hkv, D
    (1, 1, 2, 1, 4),
    (1, 17, 2, 1, 8),
    (2, 13, 3, 1, 4),
    (1, 33, 4, 2, 6),
]


@pytest.mark.parametrize("shape", ATTN_SHAPES)
def test_attention_matches_pure_loop_bruteforce(shape):
    """Vectorised windowed softmax == pure-Python loops (masking, GQA map,
    scale, max-shift, LSE) for windows 1, 2, 3, 7, T and T+5."""
    B, T, Hq, Hkv, D = shape
    rng = np.random.default_rng(11 + T)
    q, k, v = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, Hkv, D)
    for w in sorted({1, 2, 3, 7, T, T + 5}):
        o, lse = O.window_attention(q, k, v, w, block=5)
        ob, lseb = O.window_attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), w)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lseb, rtol=0, atol=1e-12)


def test_attention_rows_subset_and_query_offset():
    """Computing selected rows, or queries placed at an offset (decode),
    gives the same rows as the full computation."""
    rng = np.random.default_rng(3)
    B, T, Hq, Hkv, D = 1, 40, 2, 1, 8
    q, k, v = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, Hkv, D)
    o, lse = O.window_attention(q, k, v, 9)
    rows = [0, 5, 39, 17]
    o2, lse2 = O.window_attention(q, k, v, 9, rows=rows)
    np.testing.assert_array_equal(o2[:, rows], o[:, rows])
    o3, lse3 = O.window_attention(q[:, 30:], k, v, 9, q_pos0=30)
    np.testing.assert_allclose(o3, o[:, 30:], atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse3, lse[:, :, 30:], atol=1e-13, rtol=0)


@pytest.mark.parametrize("hq,hkv", [(2, 1), (6, 3), (4, 4)])
def test_full_window_equals_torch_causal_sdpa(hq, hkv):
    """w >= T reduces to plain causal attention: torch SDPA in fp64 on CPU."""
    rng = np.random.default_rng(5)
    B, T, D = 2, 37, 16
    q, k, v = rnd(rng, B, T, hq, D), rnd(rng, B, T, hkv, D), rnd(rng, B, T, hkv, D)
    G = hq // hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.repeat(k, G, axis=2)).permute(0, 2, 1, 3).contiguous()
    tv = torch.from_numpy(np.repeat(v, G, axis=2)).permute(0, 2, 1, 3).contiguous()
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True).permute(0, 2, 1, 3).numpy()
    for w in (T, T + 100):
        o, _ = O.window_attention(q, k, v, w)
        np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


def test_window_one_returns_own_value_and_score():
    """w = 1: each query sees only itself: o_t = v_t and LSE = s_tt."""
    rng = np.random.default_rng(6)
    B, T, Hq, Hkv, D = 1, 12, 4, 2, 8
    q, k, v = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, Hkv, D)
    o, lse = O.window_attention(q, k, v, 1)
    for h in range(Hq):
        g = h // 2
        np.testing.assert_array_equal(o[0, :, h], v[0, :, g])
        s_tt = np.einsum("td,td->t", q[0, :, h], k[0, :, g]) / math.sqrt(D)
        np.testing.assert_allclose(lse[0, h], s_tt, atol=1e-14, rtol=0)


def test_teacher_equals_student_inside_short_window():
    """For t < w_S the far band is empty, so O_T = O_S; with w_S = w_T the
    two outputs are the same computation."""
    rng = np.random.default_rng(7)
    B, T, Hq, Hkv, D = 1, 50, 2, 1, 8
    q, k, v = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, Hkv, D)
    o_t, o_s, l_t, l_s = O.dual_window_attention(q, k, v, 30, 11)
    np.testing.assert_allclose(o_t[:, :11], o_s[:, :11], atol=1e-13, rtol=0)
    np.testing.assert_allclose(l_t[:, :, :11], l_s[:, :, :11], atol=1e-13, rtol=0)
    assert np.abs(o_t[:, 11:] - o_s[:, 11:]).max() > 1e-3
    o_t, o_s, l_t, l_s = O.dual_window_attention(q, k, v, 13, 13)
    np.testing.assert_array_equal(o_t, o_s)
    np.testing.assert_array_equal(l_t, l_s)


def test_teacher_is_exact_lse_merge_of_student_and_far_band():
    """The LSE-combination identity: the teacher output is the
    log-sum-exp weighted merge of the student window and the far band
    [t-w_T+1, t-w_S] (far band computed by the independent brute force)."""
    rng = np.random.default_rng(8)
    B, T, Hq, Hkv, D = 1, 26, 3, 1, 4
    wT, wS = 15, 4
    q, k, v = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, Hkv, D)
    o_t, o_s, l_t, l_s = O.dual_window_attention(q, k, v, wT, wS)
    o_f, l_f = O.window_attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), wT,
                                             band=(wS, wT))
    for t in range(wS, T):
        for h in range(Hq):
            a, b = l_s[0, h, t], l_f[0, h, t]
            m = max(a, b)
            ea, eb = math.exp(a - m), math.exp(b - m)
            merged = (ea * o_s[0, t, h] + eb * o_f[0, t, h]) / (ea + eb)
            np.testing.assert_allclose(o_t[0, t, h], merged, atol=1e-12, rtol=0)
            np.testing.assert_allclose(l_t[0, h, t], m + math.log(ea + eb), atol=1e-12, rtol=0)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(9)
    B, T, Hq, Hkv, D = 2, 21, 6, 2, 8
    q, k, v = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, Hkv, D)
    o, lse = O.window_attention(q, k, v, 7)
    o2, lse2 = O.window_attention(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), 7)
    np.testing.assert_allclose(o, o2, atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse, lse2, atol=1e-14, rtol=0)


def test_causality_and_window_locality():
    """Rows before tau ignore keys at or after tau; row t ignores keys older
    than t - w + 1 (bit-identical results after perturbing them)."""
    rng = np.random.default_rng(10)
    B, T, Hq, Hkv, D = 1, 40, 2, 1, 8
    w = 6
    q, k, v = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, Hkv, D)
    o, lse = O.window_attention(q, k, v, w, block=64)
    k2, v2 = k.copy(), v.copy()
    k2[:, 25:] += 5.0
    v2[:, 25:] -= 3.0
    o2, lse2 = O.window_attention(q, k2, v2, w, block=64)
    np.testing.assert_allclose(o2[:, :25], o[:, :25], atol=1e-14, rtol=0)
    assert np.abs(o2[:, 25:] - o[:, 25:]).max() > 1e-2
    t = 33
    k3, v3 = k.copy(), v.copy()
    k3[:, : t - w + 1] = 100.0
    v3[:, : t - w + 1] = -100.0
    o3, _ = O.window_attention(q, k3, v3, w, rows=[t])
    np.testing.assert_allclose(o3[:, t], o[:, t], atol=1e-13, rtol=0)


# --------------------------------------------------------------------------
# O2-O3 glue
# --------------------------------------------------------------------------


def test_glue_matches_torch_library_routines():
    rng = np.random.default_rng(12)
    B, T, Hq, D, d, f = 2, 9, 3, 4, 10, 14
    x, o = rnd(rng, B, T, d), rnd(rng, B, T, Hq, D)
    w_o = rnd(rng, d, Hq * D)
    h = O.attn_out_residual(x, o, w_o)
    ref = torch.from_numpy(x) + F.linear(torch.from_numpy(o.reshape(B, T, Hq * D)),
                                         torch.from_numpy(w_o))
    np.testing.assert_allclose(h, ref.numpy(), atol=1e-13, rtol=0)
    gamma = 1 + 0.2 * rnd(rng, d)
    u = O.rmsnorm(h, gamma, 1e-6)
    uref = F.rms_norm(torch.from_numpy(h), (d,), torch.from_numpy(gamma), eps=1e-6)
    np.testing.assert_allclose(u, uref.numpy(), atol=1e-13, rtol=0)
    wg, wu = rnd(rng, f, d), rnd(rng, f, d)
    z = O.swiglu_hidden(u, wg, wu)
    tu = torch.from_numpy(u)
    zref = F.silu(F.linear(tu, torch.from_numpy(wg))) * F.linear(tu, torch.from_numpy(wu))
    np.testing.assert_allclose(z, zref.numpy(), atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# O4-O5 conv, keys, residual
# --------------------------------------------------------------------------


def test_conv_identity_taps_and_torch_conv1d():
    rng = np.random.default_rng(13)
    B, T, f, kc = 2, 11, 5, 4
    z = rnd(rng, B, T, f)
    ident = np.zeros((f, kc))
    ident[:, kc - 1] = 1.0
    np.testing.assert_array_equal(O.causal_depthwise_conv(z, ident), z)
    taps = rnd(rng, f, kc)
    out = O.causal_depthwise_conv(z, taps)
    tz = torch.from_numpy(z).transpose(1, 2)                      # [B, f, T]
    ref = F.conv1d(tz, torch.from_numpy(taps)[:, None, :], padding=kc - 1, groups=f)
    ref = ref[..., :T].transpose(1, 2).numpy()
    np.testing.assert_allclose(out, ref, atol=1e-13, rtol=0)


def test_conv_impulse_response_orientation():
    """An impulse at token tau shows tap kc-1 at tau and tap kc-1-s at
    tau+s; nothing before tau (causal, crosses any chunk boundary)."""
    T, f, kc, tau = 10, 3, 4, 5
    z = np.zeros((T, f))
    z[tau] = 1.0
    taps = np.arange(1, f * kc + 1, dtype=float).reshape(f, kc)
    out = O.causal_depthwise_conv(z, taps)
    assert np.all(out[:tau] == 0)
    for s in range(kc):
        np.testing.assert_array_equal(out[tau + s], taps[:, kc - 1 - s])
    assert np.all(out[tau + kc:] == 0)


def test_l2_keys_unit_norm_zero_row_and_torch_normalize():
    rng = np.random.default_rng(14)
    x = rnd(rng, 7, 9)
    x[3] = 0.0
    kx = O.l2_normalize(x)
    n = np.linalg.norm(kx, axis=-1)
    np.testing.assert_allclose(np.delete(n, 3), 1.0, atol=1e-14)
    assert np.all(kx[3] == 0)
    ref = F.normalize(torch.from_numpy(x), dim=-1, eps=1e-12).numpy()
    np.testing.assert_allclose(kx, ref, atol=1e-15, rtol=0)


def test_residual_projection_orientation_with_permutation():
    """W_proj acts on the column vector dbar: a permutation matrix P gives
    W_proj dbar = dbar[perm] (a transposed W_proj would give the inverse)."""
    rng = np.random.default_rng(15)
    T, d, f = 6, 3, 5
    perm = np.array([2, 4, 0, 1, 3])
    P = np.zeros((f, f))
    P[np.arange(f), perm] = 1.0          # (P x)_i = x[perm[i]]
    z_t, z_s = rnd(rng, T, f), rnd(rng, T, f)
    ident = np.zeros((f, 4))
    ident[:, 3] = 1.0
    w0 = rnd(rng, d, f)
    r, k, dbar, _ = O.fastweight_terms(z_t, z_s, ident, ident, w0, P)
    np.testing.assert_allclose(dbar, z_t - z_s, atol=0, rtol=0)
    np.testing.assert_allclose(r, (z_t - z_s)[:, perm] @ w0.T, atol=1e-14, rtol=0)


# --------------------------------------------------------------------------
# O5-O8 fast weights
# --------------------------------------------------------------------------


def _scan_inputs(rng, T=37, f=6, d=4, C=8):
    z_t, z_s = rnd(rng, T, f), rnd(rng, T, f)
    n = -(-T // C)
    return dict(z_t=z_t, z_s=z_s, conv_t=rnd(rng, f, 4), conv_s=rnd(rng, f, 4),
                w0=rnd(rng, d, f), wp=rnd(rng, f, f), beta=rng.random(n), C=C)


def test_three_forms_of_the_prefix_agree():
    """Running prefix == explicit sum of per-chunk dW == low-rank form."""
    rng = np.random.default_rng(16)
    s = _scan_inputs(rng)
    r, k, _, _ = O.fastweight_terms(s["z_t"], s["z_s"], s["conv_t"], s["conv_s"], s["w0"], s["wp"])
    y1, S = O.fastweight_apply_prefix(r, k, s["beta"], s["z_t"], s["w0"], s["C"])
    y2 = O.fastweight_apply_explicit(r, k, s["beta"], s["z_t"], s["w0"], s["C"])
    y3 = O.fastweight_apply_lowrank(r, k, s["beta"], s["z_t"], s["w0"], s["C"])
    scale = np.abs(y1).max()
    np.testing.assert_allclose(y2, y1, atol=1e-12 * scale, rtol=0)
    np.testing.assert_allclose(y3, y1, atol=1e-12 * scale, rtol=0)
    # final state = W0 + every chunk's write (the partial last chunk included)
    full = s["w0"] + sum(s["beta"][i] * (r[a:b].T @ k[a:b])
                         for i, (a, b) in enumerate(O.chunk_bounds(len(r), s["C"])))
    np.testing.assert_allclose(S, full, atol=1e-12, rtol=0)


def test_first_chunk_and_short_sequence_use_base_weight():
    """Chunk 0 (and any T <= C) has no earlier chunk: y = W0 z."""
    rng = np.random.default_rng(17)
    s = _scan_inputs(rng, T=8, C=8)
    out = O.fastweight_scan(s["z_t"][None], s["z_s"][None], s["z_t"][None], s["conv_t"],
                            s["conv_s"], s["w0"], s["wp"], s["beta"][None], s["C"])
    np.testing.assert_allclose(out["y"][0], s["z_t"] @ s["w0"].T, atol=1e-13, rtol=0)
    s = _scan_inputs(rng, T=30, C=8)
    out = O.fastweight_scan(s["z_t"][None], s["z_s"][None], s["z_t"][None], s["conv_t"],
                            s["conv_s"], s["w0"], s["wp"], s["beta"][None], s["C"])
    np.testing.assert_allclose(out["y"][0, :8], s["z_t"][:8] @ s["w0"].T, atol=1e-13, rtol=0)
    assert np.abs(out["y"][0, 8:] - s["z_t"][8:] @ s["w0"].T).max() > 1e-3


def test_writes_act_only_on_strictly_later_chunks():
    """Perturbing the student activations of chunk c (and so its write)
    leaves y of chunks <= c unchanged and changes later chunks."""
    rng = np.random.default_rng(18)
    s = _scan_inputs(rng, T=40, C=8)
    args = lambda zs: (s["z_t"][None], zs[None], s["z_t"][None], s["conv_t"], s["conv_s"],
                       s["w0"], s["wp"], s["beta"][None], s["C"])
    y0 = O.fastweight_scan(*args(s["z_s"]))["y"][0]
    zs2 = s["z_s"].copy()
    zs2[16:21] += 1.0            # chunk 2 only (the conv tail stays inside it)
    y1 = O.fastweight_scan(*args(zs2))["y"][0]
    np.testing.assert_array_equal(y1[:24], y0[:24])
    assert np.abs(y1[24:] - y0[24:]).max() > 1e-3


def test_state_after_complete_chunks_is_the_state_of_the_truncated_sequence():
    """The weight after the complete chunks of a ragged sequence is the final
    weight of the same sequence cut after its last complete chunk (the
    writes are causal: later tokens cannot change them); when T % C == 0 it
    is the final weight, and T < C leaves W0.  Holds for all three update
    rules.  A short chunk's write counted in, or one chunk too few, breaks
    this."""
    rng = np.random.default_rng(23)
    s = _scan_inputs(rng, T=30, C=8)
    fns = [
        lambda zt, zs, b: O.fastweight_scan(zt[None], zs[None], zt[None], s["conv_t"],
                                            s["conv_s"], s["w0"], s["wp"], b[None], s["C"]),
        lambda zt, zs, b: O.fastweight_scan_on_policy(zt[None], zs[None], zt[None], s["conv_t"],
                                                      s["conv_s"], s["w0"], s["wp"], b[None],
                                                      s["C"]),
        lambda zt, zs, b: O.fastweight_scan_eq6(zt[None], zs[None], zt[None], s["w0"], b[None],
                                                s["C"]),
    ]
    for fn in fns:
        ragged = fn(s["z_t"], s["z_s"], s["beta"])
        cut = fn(s["z_t"][:24], s["z_s"][:24], s["beta"][:3])
        np.testing.assert_allclose(ragged["state_complete"], cut["state"],
                                   atol=1e-12 * np.abs(cut["state"]).max(), rtol=0)
        np.testing.assert_array_equal(cut["state_complete"], cut["state"])
        assert np.abs(ragged["state"] - ragged["state_complete"]).max() > 1e-6
        short = fn(s["z_t"][:5], s["z_s"][:5], s["beta"][:1])
        np.testing.assert_array_equal(short["state_complete"][0], s["w0"])


def test_equal_paths_give_no_update():
    """Equal convs and equal activations: dbar = 0, R = 0, y = W0 z."""
    rng = np.random.default_rng(19)
    s = _scan_inputs(rng)
    out = O.fastweight_scan(s["z_t"][None], s["z_t"][None], s["z_t"][None], s["conv_t"],
                            s["conv_t"], s["w0"], s["wp"], s["beta"][None], s["C"])
    assert np.all(out["r"] == 0)
    np.testing.assert_allclose(out["y"][0], s["z_t"] @ s["w0"].T, atol=1e-13, rtol=0)


def test_layer_with_equal_windows_and_convs_is_plain_layer():
    """w_S = w_T and conv_T = conv_S: teacher and student coincide, so the
    layer is attention + plain SwiGLU MLP with W_down^(0)."""
    rng = np.random.default_rng(20)
    B, T, Hq, Hkv, D, d, f, C = 1, 24, 2, 1, 4, 6, 10, 8
    q, k, v, x = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, d)
    w = small_layer_weights(rng, d, f, Hq * D)
    w["conv_s"] = w["conv_t"].copy()
    w["beta"] = rng.random((B, 3))
    res = O.layer_forward(q, k, v, x, w, 9, 9, C)
    z = res["z_t"]
    np.testing.assert_allclose(res["out"], res["h_t"] + z @ w["w_down0"].T, atol=1e-13, rtol=0)


def test_zero_student_conv_leaves_layer_unperturbed():
    """conv_S = 0 gives zero keys, no write, and the plain layer
    (the continued-training initialisation property)."""
    rng = np.random.default_rng(21)
    B, T, Hq, Hkv, D, d, f, C = 1, 24, 2, 1, 4, 6, 10, 8
    q, k, v, x = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, d)
    w = small_layer_weights(rng, d, f, Hq * D)
    w["conv_s"] = np.zeros_like(w["conv_s"])
    w["beta"] = rng.random((B, 3))
    res = O.layer_forward(q, k, v, x, w, 9, 3, C)
    assert np.all(res["k"] == 0)
    np.testing.assert_allclose(res["out"], res["h_t"] + res["z_t"] @ w["w_down0"].T,
                               atol=1e-13, rtol=0)


def test_single_write_closed_form_proposition_one():
    """Identity convs and W_proj = I reduce the residual to the teacher-
    student output gap, r = W0 z^T - W0 z^S (the raw gradient direction).
    One write token q1 in chunk 0 then moves a query q2 in chunk 1 by
    dy = beta r (k.z_q2), so y_q1^T . dy = beta (y_q1^T . r)(k . z_q2)."""
    rng = np.random.default_rng(22)
    T, f, d, C = 16, 7, 5, 8
    z_t = rnd(rng, T, f)
    z_s = z_t.copy()
    q1, q2 = 3, 12
    z_s[q1] += rnd(rng, f)               # only q1 differs between the paths
    ident = np.zeros((f, 4))
    ident[:, 3] = 1.0
    w0 = rnd(rng, d, f)
    beta = np.array([0.7, 0.3])
    out = O.fastweight_scan(z_t[None], z_s[None], z_t[None], ident, ident, w0, np.eye(f),
                            beta[None], C)
    r = out["r"][0]
    np.testing.assert_allclose(r[q1], w0 @ z_t[q1] - w0 @ z_s[q1], atol=1e-13, rtol=0)
    assert np.all(np.delete(r, q1, axis=0) == 0)
    kq1 = z_s[q1] / np.linalg.norm(z_s[q1])
    dy = out["y"][0, q2] - w0 @ z_t[q2]
    np.testing.assert_allclose(dy, beta[0] * r[q1] * (kq1 @ z_t[q2]), atol=1e-13, rtol=0)
    yT = w0 @ z_t[q1]
    lhs = yT @ dy
    rhs = beta[0] * (yT @ r[q1]) * (kq1 @ z_t[q2])
    np.testing.assert_allclose(lhs, rhs, atol=1e-12, rtol=0)
    # positive gap and alignment -> the later output moves toward the teacher
    if (yT @ r[q1]) > 0 and (kq1 @ z_t[q2]) > 0:
        assert lhs > 0


# --------------------------------------------------------------------------
# O9 decode
# --------------------------------------------------------------------------


def test_decode_equals_prefill_row_and_fold_equals_prefix_state():
    """A decode step at position L = n*C, with the lists taken from a
    prefill of the same sequence, equals that prefill's row L; folding the
    lists gives the prefill's weight after n chunks."""
    rng = np.random.default_rng(23)
    B, Hq, Hkv, D, d, f, C = 2, 4, 2, 4, 6, 10, 8
    n = 3
    L = n * C
    T = L + 1
    q, k, v, x = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, d)
    w = small_layer_weights(rng, d, f, Hq * D)
    w["beta"] = rng.random((B, n + 1))
    wT, wS = 11, 3
    pre = O.layer_forward(q, k, v, x, w, wT, wS, C)
    dec = O.decode_step(q[:, L:L + 1], k, v, x[:, L:L + 1], w, L, wT, wS,
                        pre["r"][:, :L], pre["k"][:, :L], w["beta"][:, :n], C)
    np.testing.assert_allclose(dec["out"][:, 0], pre["out"][:, L], atol=1e-12, rtol=0)
    # the cache may be handed over as the teacher window only
    lo = L + 1 - wT
    dec2 = O.decode_step(q[:, L:L + 1], k[:, lo:], v[:, lo:], x[:, L:L + 1], w, L, wT, wS,
                         pre["r"][:, :L], pre["k"][:, :L], w["beta"][:, :n], C, key_offset=lo)
    np.testing.assert_allclose(dec2["out"], dec["out"], atol=1e-13, rtol=0)
    folded = O.fold_lists(w["w_down0"], pre["r"][:, :L], pre["k"][:, :L], w["beta"][:, :n], C)
    for b in range(B):
        _, Sn, states = O.fastweight_apply_prefix(pre["r"][b], pre["k"][b], w["beta"][b],
                                                  pre["z_t"][b], w["w_down0"], C,
                                                  return_states=True)
        np.testing.assert_allclose(folded[b], states[n], atol=1e-12, rtol=0)


@pytest.mark.parametrize("kc", [1, 3, 4])
def test_decode_append_token_by_token_equals_sequence_terms(kc):
    """Appending tokens one at a time (window = history + token) gives the
    write terms of the whole-sequence causal conv at every position, from a
    zero history at the sequence start and from a history handed over
    mid-sequence.  A slip in the tap orientation, the window order or the
    history shift breaks it; one token is also checked by an explicit loop."""
    rng = np.random.default_rng(31 + kc)
    B, T, d, f = 2, 13, 5, 7
    z_t, z_s = rnd(rng, B, T, f), rnd(rng, B, T, f)
    conv_t, conv_s = rnd(rng, f, kc), rnd(rng, f, kc)
    w0, wp = rnd(rng, d, f), rnd(rng, f, f)
    ref = [O.fastweight_terms(z_t[b], z_s[b], conv_t, conv_s, w0, wp) for b in range(B)]
    for start in (0, 6):
        ht = np.zeros((B, kc - 1, f))
        hs = np.zeros((B, kc - 1, f))
        for i in range(kc - 1):
            tau = start - (kc - 1) + i
            if tau >= 0:
                ht[:, i], hs[:, i] = z_t[:, tau], z_s[:, tau]
        for t in range(start, T):
            r, k, dbar, ht, hs = O.decode_append(z_t[:, t], z_s[:, t], ht, hs, conv_t, conv_s,
                                                 w0, wp)
            for b in range(B):
                np.testing.assert_allclose(r[b], ref[b][0][t], atol=1e-12, rtol=0)
                np.testing.assert_allclose(k[b], ref[b][1][t], atol=1e-12, rtol=0)
                np.testing.assert_allclose(dbar[b], ref[b][2][t], atol=1e-12, rtol=0)
    # one token by an explicit loop over features and taps
    t = 9
    ht = np.stack([z_t[:, t - (kc - 1) + i] for i in range(kc - 1)], axis=1) if kc > 1 else np.zeros((B, 0, f))
    hs = np.stack([z_s[:, t - (kc - 1) + i] for i in range(kc - 1)], axis=1) if kc > 1 else np.zeros((B, 0, f))
    r, k, dbar, _, _ = O.decode_append(z_t[:, t], z_s[:, t], ht, hs, conv_t, conv_s, w0, wp)
    for b in range(B):
        zb_t = np.zeros(f)
        zb_s = np.zeros(f)
        for c in range(f):
            for i in range(kc):
                zb_t[c] += conv_t[c, i] * z_t[b, t - (kc - 1) + i, c]
                zb_s[c] += conv_s[c, i] * z_s[b, t - (kc - 1) + i, c]
        np.testing.assert_allclose(dbar[b], zb_t - zb_s, atol=1e-12, rtol=0)
        np.testing.assert_allclose(k[b], zb_s / np.linalg.norm(zb_s), atol=1e-12, rtol=0)
        np.testing.assert_allclose(r[b], w0 @ (wp @ (zb_t - zb_s)), atol=1e-12, rtol=0)


def _on_policy_args(s, z_s=None, beta=None):
    return (s["z_t"][None], (s["z_s"] if z_s is None else z_s)[None], s["z_t"][None],
            s["conv_t"], s["conv_s"], s["w0"], s["wp"],
            (s["beta"] if beta is None else beta)[None], s["C"])


def test_on_policy_state_is_ordered_product_of_chunk_factors():
    """S_{i+1} = S_i + beta_i S_i W_proj Dbar_i^T K_i factors as
    S_i (I + beta_i W_proj Dbar_i^T K_i): the on-policy weights are W0 times
    the ordered product of per-chunk f x f factors (a ragged last chunk
    included).  A residual taken at W0 or at S_{i+1}, or the factors in the
    wrong order, breaks this."""
    rng = np.random.default_rng(31)
    s = _scan_inputs(rng, T=30, C=8)
    _, k, dbar, _ = O.fastweight_terms(s["z_t"], s["z_s"], s["conv_t"], s["conv_s"],
                                       s["w0"], s["wp"])
    out = O.fastweight_scan_on_policy(*_on_policy_args(s))
    f = s["w0"].shape[1]
    P = np.eye(f)
    y = np.zeros_like(out["y"][0])
    for i, (a, b) in enumerate(O.chunk_bounds(30, s["C"])):
        y[a:b] = s["z_t"][a:b] @ (s["w0"] @ P).T
        P = P @ (np.eye(f) + s["beta"][i] * (s["wp"] @ dbar[a:b].T @ k[a:b]))
    scale = np.abs(y).max()
    np.testing.assert_allclose(out["y"][0], y, atol=1e-12 * scale, rtol=0)
    np.testing.assert_allclose(out["state"][0], s["w0"] @ P, atol=1e-12 * np.abs(s["w0"] @ P).max(),
                               rtol=0)


def test_on_policy_agrees_with_off_policy_until_the_second_write():
    """Chunks 0 and 1 see W0 and W0 + beta_0 R_0^T K_0 under both rules
    (chunk 0's residual is taken at S_0 = W0 either way); from chunk 2 on
    the rules differ.  With beta = 0 or equal paths nothing is written."""
    rng = np.random.default_rng(32)
    s = _scan_inputs(rng, T=40, C=8)
    on = O.fastweight_scan_on_policy(*_on_policy_args(s))["y"][0]
    off = O.fastweight_scan(*_on_policy_args(s))["y"][0]
    np.testing.assert_allclose(on[:16], off[:16], atol=1e-12 * np.abs(off).max(), rtol=0)
    assert np.abs(on[16:] - off[16:]).max() > 1e-3 * np.abs(off).max()
    zero = O.fastweight_scan_on_policy(*_on_policy_args(s, beta=np.zeros_like(s["beta"])))
    np.testing.assert_allclose(zero["y"][0], s["z_t"] @ s["w0"].T, atol=1e-13, rtol=0)
    np.testing.assert_array_equal(zero["state"][0], s["w0"])
    same = O.fastweight_scan_on_policy(s["z_t"][None], s["z_t"][None], s["z_t"][None],
                                       s["conv_t"], s["conv_t"], s["w0"], s["wp"],
                                       s["beta"][None], s["C"])
    np.testing.assert_array_equal(same["state"][0], s["w0"])


def test_on_policy_equals_pure_loop_per_token_recurrence():
    """Brute force: scalar loops over tokens and features, the weight
    updated only at chunk ends, each token's residual read from the weight
    in force for its chunk."""
    rng = np.random.default_rng(33)
    s = _scan_inputs(rng, T=13, C=4, f=5, d=3)
    _, k, dbar, _ = O.fastweight_terms(s["z_t"], s["z_s"], s["conv_t"], s["conv_s"],
                                       s["w0"], s["wp"])
    d, f = s["w0"].shape
    S = [[float(s["w0"][o, c]) for c in range(f)] for o in range(d)]
    y = np.zeros((13, d))
    pend = [[0.0] * f for _ in range(d)]
    for t in range(13):
        i = t // 4
        for o in range(d):
            y[t, o] = sum(S[o][c] * s["z_t"][t, c] for c in range(f))
        u = [sum(s["wp"][a, c] * dbar[t, c] for c in range(f)) for a in range(f)]
        r = [sum(S[o][a] * u[a] for a in range(f)) for o in range(d)]
        for o in range(d):
            for c in range(f):
                pend[o][c] += s["beta"][i] * r[o] * k[t, c]
        if t % 4 == 3 or t == 12:
            S = [[S[o][c] + pend[o][c] for c in range(f)] for o in range(d)]
            pend = [[0.0] * f for _ in range(d)]
    out = O.fastweight_scan_on_policy(*_on_policy_args(s))
    np.testing.assert_allclose(out["y"][0], y, atol=1e-12, rtol=0)
    np.testing.assert_allclose(out["state"][0], np.array(S), atol=1e-12, rtol=0)


def test_eq6_write_is_minus_beta_times_autograd_gradient_of_the_loss():
    """Each chunk's write equals -beta_i times torch.autograd's gradient of
    0.5 sum_t ||W z_S,t - stopgrad(W z_T,t)||^2 at W = W0 (fp64), and the
    prefix/apply use those writes."""
    rng = np.random.default_rng(34)
    s = _scan_inputs(rng, T=29, C=8)
    out = O.fastweight_scan_eq6(s["z_t"][None], s["z_s"][None], s["z_t"][None], s["w0"],
                                s["beta"][None], s["C"])
    S = s["w0"].copy()
    for i, (a, b) in enumerate(O.chunk_bounds(29, s["C"])):
        W = torch.tensor(s["w0"], dtype=torch.float64, requires_grad=True)
        zs = torch.tensor(s["z_s"][a:b])
        zt = torch.tensor(s["z_t"][a:b])
        loss = 0.5 * ((zs @ W.T - (zt @ W.T).detach()) ** 2).sum()
        loss.backward()
        dw = -s["beta"][i] * W.grad.numpy()
        np.testing.assert_allclose(out["dw"][0, i], dw, atol=1e-13, rtol=0)
        np.testing.assert_allclose(out["y"][0, a:b], s["z_t"][a:b] @ S.T, atol=1e-12, rtol=0)
        S = S + dw
    np.testing.assert_allclose(out["state"][0], S, atol=1e-12, rtol=0)


def test_eq6_small_step_lowers_the_chunk_loss():
    """A gradient step: with a small enough beta the student's chunk loss
    at W0 + dW_i is below its value at W0; equal paths write nothing."""
    rng = np.random.default_rng(35)
    s = _scan_inputs(rng, T=16, C=16)
    beta = np.array([1e-3])
    out = O.fastweight_scan_eq6(s["z_t"][None], s["z_s"][None], s["z_t"][None], s["w0"],
                                beta[None], 16)
    loss = lambda W: 0.5 * np.sum((s["z_s"] @ W.T - s["z_t"] @ s["w0"].T) ** 2)
    assert loss(s["w0"] + out["dw"][0, 0]) < loss(s["w0"])
    same = O.fastweight_scan_eq6(s["z_t"][None], s["z_t"][None], s["z_t"][None], s["w0"],
                                 beta[None], 16)
    assert np.all(same["dw"] == 0)
