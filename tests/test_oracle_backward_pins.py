"""Pins of the oracle's backward pass (CPU): each gradient against
torch.autograd of the same forward built from torch library routines in
fp64, and against central finite differences of the oracle's own forward,
which needs no torch at all.  A dropped term, a wrong sign, a transposed
factor or a chunk off by one in the suffix sum fails one of them."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ttcd_oracle as O

torch.set_default_dtype(torch.float64)


def rnd(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def t64(a, grad=True):
    return torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=grad)


# ------------------------------------------------------------------ pieces
def test_conv_backward_matches_autograd_of_torch_conv1d():
    rng = np.random.default_rng(70)
    T, f, kc = 11, 5, 3
    z, taps, dzb = rnd(rng, T, f), rnd(rng, f, kc), rnd(rng, T, f)
    dz, dtaps = O.causal_depthwise_conv_backward(z, taps, dzb)
    zt, tt = t64(z), t64(taps)
    out = F.conv1d(zt.T[None], tt[:, None, :], padding=kc - 1, groups=f)[0, :, :T].T
    (out * torch.tensor(dzb)).sum().backward()
    np.testing.assert_allclose(dz, zt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dtaps, tt.grad.numpy(), rtol=0, atol=1e-12)


def test_l2_backward_matches_autograd_of_torch_normalize_incl_tiny_rows():
    rng = np.random.default_rng(71)
    x = rnd(rng, 6, 9)
    x[2] *= 1e-14            # below eps: the max(., eps) branch
    dk = rnd(rng, 6, 9)
    got = O.l2_normalize_backward(x, dk, 1e-12)
    xt = t64(x)
    (F.normalize(xt, dim=-1, eps=1e-12) * torch.tensor(dk)).sum().backward()
    np.testing.assert_allclose(got, xt.grad.numpy(), rtol=1e-10, atol=1e-9)


# ------------------------------------------------------------ fast weight
def torch_scan_y(z_t, z_s, z_main, conv_t, conv_s, w0, wp, beta, C, eps=1e-12):
    """The off-policy forward from torch library routines (conv1d,
    normalize, matmul), differentiable in every input."""
    B, T, f = z_t.shape
    kc = conv_t.shape[1]
    ys = []
    for b in range(B):
        zb_t = F.conv1d(z_t[b].T[None], conv_t[:, None, :], padding=kc - 1, groups=f)[0, :, :T].T
        zb_s = F.conv1d(z_s[b].T[None], conv_s[:, None, :], padding=kc - 1, groups=f)[0, :, :T].T
        r = ((zb_t - zb_s) @ wp.T) @ w0.T
        k = F.normalize(zb_s, dim=-1, eps=eps)
        S = w0
        rows = []
        for i, a in enumerate(range(0, T, C)):
            e = min(a + C, T)
            rows.append(z_main[b, a:e] @ S.T)
            S = S + beta[b, i] * (r[a:e].T @ k[a:e])
        ys.append(torch.cat(rows))
    return torch.stack(ys)


def scan_case(seed, B=2, T=23, f=6, d=4, C=5, kc=3):
    rng = np.random.default_rng(seed)
    n = -(-T // C)
    return dict(z_t=rnd(rng, B, T, f), z_s=rnd(rng, B, T, f), z_main=rnd(rng, B, T, f),
                conv_t=rnd(rng, f, kc, scale=0.6), conv_s=rnd(rng, f, kc, scale=0.6),
                w0=rnd(rng, d, f, scale=0.4), wp=rnd(rng, f, f, scale=0.4),
                beta=rng.random((B, n)), C=C, dy=rnd(rng, B, T, d))


NAMES = [("z_t", "dz_t"), ("z_s", "dz_s"), ("z_main", "dz_main"), ("conv_t", "dconv_t"),
         ("conv_s", "dconv_s"), ("w0", "dw_down0"), ("wp", "dw_proj"), ("beta", "dbeta")]


def oracle_grads(c):
    return O.fastweight_scan_backward(c["z_t"], c["z_s"], c["z_main"], c["conv_t"], c["conv_s"],
                                      c["w0"], c["wp"], c["beta"], c["C"], c["dy"])


@pytest.mark.parametrize("T,C", [(23, 5), (20, 5), (4, 5)], ids=["ragged", "whole-chunks", "T<C"])
def test_scan_backward_matches_autograd(T, C):
    c = scan_case(72, T=T, C=C)
    g = oracle_grads(c)
    ts = {n: t64(c[n]) for n, _ in NAMES}
    y = torch_scan_y(ts["z_t"], ts["z_s"], ts["z_main"], ts["conv_t"], ts["conv_s"], ts["w0"],
                     ts["wp"], ts["beta"], C)
    (y * torch.tensor(c["dy"])).sum().backward()
    for n, gn in NAMES:
        # (an input y does not depend on gets no gradient at all: zero)
        want = ts[n].grad.numpy() if ts[n].grad is not None else np.zeros(np.shape(c[n]))
        np.testing.assert_allclose(g[gn], want, rtol=1e-9, atol=1e-9 * max(1.0, np.abs(want).max()),
                                   err_msg=gn)


def test_scan_backward_matches_finite_differences_of_the_oracle():
    """Directional derivatives of L = <dy, y> along a random direction of
    each input, by central differences of the oracle's forward."""
    c = scan_case(73)
    g = oracle_grads(c)
    rng = np.random.default_rng(74)

    def loss(**over):
        a = {**c, **over}
        y = O.fastweight_scan(a["z_t"], a["z_s"], a["z_main"], a["conv_t"], a["conv_s"], a["w0"],
                              a["wp"], a["beta"], a["C"])["y"]
        return float(np.sum(y * c["dy"]))

    h = 1e-6
    for n, gn in NAMES:
        v = rng.standard_normal(np.shape(c[n]))
        fd = (loss(**{n: c[n] + h * v}) - loss(**{n: c[n] - h * v})) / (2 * h)
        an = float(np.sum(g[gn] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (gn, fd, an)


def test_scan_backward_without_writes_is_the_plain_mlp_gradient():
    """beta = 0: nothing is written, so the convs, W_proj and both paths'
    activations get no gradient through the write, W_down0 gets
    sum_t dy_t z_t^T and z_main gets W_down0^T dy."""
    c = scan_case(75)
    c["beta"] = np.zeros_like(c["beta"])
    g = oracle_grads(c)
    for n in ("dz_t", "dz_s", "dconv_t", "dconv_s", "dw_proj"):
        assert np.all(g[n] == 0), n
    want = np.einsum("btd,btf->df", c["dy"], c["z_main"])
    np.testing.assert_allclose(g["dw_down0"], want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dz_main"], c["dy"] @ c["w0"], rtol=1e-12, atol=1e-12)
    assert np.abs(g["dbeta"]).max() > 1e-3


def test_scan_backward_last_chunk_write_has_no_gradient():
    """The last chunk's write reaches no token: its beta gets zero gradient
    and its tokens' residuals and keys get none through the write."""
    c = scan_case(76, T=23, C=5)
    g = oracle_grads(c)
    assert np.all(g["dbeta"][:, -1] == 0)
    assert np.all(g["dbeta"][:, :-1] != 0)


# -------------------------------------------------------------- attention
def sdpa_window(q, k, v, window, scale):
    """One window through torch's scaled_dot_product_attention with an
    explicit boolean mask (query t sees keys j with 0 <= t-j < window)."""
    B, T, Hq, D = q.shape
    G = Hq // k.shape[2]
    t = torch.arange(T)
    diff = t[:, None] - t[None, :]
    mask = (diff >= 0) & (diff < window)
    kk = k.repeat_interleave(G, dim=2)
    vv = v.repeat_interleave(G, dim=2)
    o = F.scaled_dot_product_attention(q.transpose(1, 2), kk.transpose(1, 2), vv.transpose(1, 2),
                                       attn_mask=mask, scale=scale)
    return o.transpose(1, 2)


@pytest.mark.parametrize("shape", [(1, 13, 2, 1, 4, 5, 2), (2, 17, 6, 2, 8, 17, 3),
                                   (1, 9, 3, 3, 4, 1, 1)],
                         ids=["gqa2-w5/2", "gqa3-full/3", "mha-w1"])
def test_dual_attention_backward_matches_autograd_of_torch_sdpa(shape):
    B, T, Hq, Hkv, D, wT, wS = shape
    rng = np.random.default_rng(77)
    q, k, v = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, Hkv, D)
    do_t, do_s = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hq, D)
    dq, dk, dv = O.dual_window_attention_backward(q, k, v, wT, wS, do_t, do_s)
    qt, kt, vt = t64(q), t64(k), t64(v)
    sc = 1.0 / math.sqrt(D)
    loss = (sdpa_window(qt, kt, vt, wT, sc) * torch.tensor(do_t)).sum() + \
        (sdpa_window(qt, kt, vt, wS, sc) * torch.tensor(do_s)).sum()
    loss.backward()
    for got, want, n in ((dq, qt.grad, "dq"), (dk, kt.grad, "dk"), (dv, vt.grad, "dv")):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-9, atol=1e-10, err_msg=n)


def test_dual_attention_backward_matches_finite_differences_of_the_oracle():
    rng = np.random.default_rng(78)
    B, T, Hq, Hkv, D, wT, wS = 1, 11, 4, 2, 4, 6, 2
    q, k, v = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hkv, D), rnd(rng, B, T, Hkv, D)
    do_t, do_s = rnd(rng, B, T, Hq, D), rnd(rng, B, T, Hq, D)
    g = dict(zip(("q", "k", "v"), O.dual_window_attention_backward(q, k, v, wT, wS, do_t, do_s)))
    base = {"q": q, "k": k, "v": v}

    def loss(**over):
        a = {**base, **over}
        o_t, o_s, _, _ = O.dual_window_attention(a["q"], a["k"], a["v"], wT, wS)
        return float(np.sum(o_t * do_t) + np.sum(o_s * do_s))

    h = 1e-6
    for n in ("q", "k", "v"):
        dv_ = rng.standard_normal(base[n].shape)
        fd = (loss(**{n: base[n] + h * dv_}) - loss(**{n: base[n] - h * dv_})) / (2 * h)
        an = float(np.sum(g[n] * dv_))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (n, fd, an)
