"""Seeded synthetic inputs for the IP-TTCD layer forward.

This module only draws random numbers and rounds them to the storage type.
It contains none of the method's arithmetic, so both the fp64 oracle (through
the tests and the bench) and the HIP path can consume exactly the same bytes.

Every tensor gets its own PCG64 stream, seeded from (config seed, tensor
name), so any one tensor can be regenerated without drawing the others.
bf16 tensors are drawn in float32 and rounded to nearest-even; the rounded
values are the canonical inputs on both sides.

Shapes follow the workloads of "Learning What to Remember: Test-Time
Training via Context Distillation": a SmolLM2-360M-shaped and a
Qwen3-0.6B-shaped layer (the continued-training section of the
papernotes.org notes and of the paper's podcast transcript), 64K context
(the GitHub README's continued-training pipeline).  No dataset is used:
every value is synthetic.

Weight layouts use the column-vector convention of the pages (W_down is
d x f and acts as y = W_down z):  w_o [d, Hq*D], w_gate / w_up [f, d],
w_down0 [d, f], w_proj [f, f], conv taps [f, kc] with tap kc-1 on the
current token.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

import numpy as np

# --------------------------------------------------------------------------
# bf16 storage helpers (data conversion only)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the raw 16-bit patterns as uint16.  Inputs here are finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Tensor:
    """A host tensor in its storage type.

    ``data`` is float32 for fp32 tensors and uint16 bf16 bit patterns for
    bf16 tensors.  ``f64()`` is the exact value in float64.
    """

    data: np.ndarray
    dtype: str  # "f32" | "bf16"

    @property
    def shape(self):
        return self.data.shape

    def f32(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.data)
        return self.data

    def f64(self) -> np.ndarray:
        return self.f32().astype(np.float64)


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), zlib.crc32(name.encode())])


def _store(x32: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        return Tensor(f32_to_bf16_bits(x32), "bf16")
    if dtype == "f32":
        return Tensor(np.ascontiguousarray(x32, dtype=np.float32), "f32")
    raise ValueError(dtype)


def normal(seed: int, name: str, shape, std: float, dtype: str) -> Tensor:
    x = _rng(seed, name).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return _store(x, dtype)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class LayerConfig:
    name: str
    dtype: str
    batch: int
    seq: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    w_teacher: int
    w_student: int
    d_model: int = 0
    d_ff: int = 0
    chunk: int = 0
    conv_k: int = 4
    seed: int = 0
    # attention-only sweep (several window pairs on one Q/K/V)
    windows: Tuple[Tuple[int, int], ...] = ()
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    # decode: cache length before the new token
    cache_len: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_chunks(self) -> int:
        return -(-self.seq // self.chunk) if self.chunk else 0

    def scaled(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


CONFIGS: Dict[int, LayerConfig] = {
    1: LayerConfig(
        name="tiny_fp32", dtype="f32", batch=1, seq=1024, n_q_heads=2, n_kv_heads=1,
        head_dim=64, w_teacher=256, w_student=64, d_model=128, d_ff=384, chunk=64,
        conv_k=4, seed=1),
    2: LayerConfig(
        name="smollm2_360m_16k", dtype="bf16", batch=1, seq=16384, n_q_heads=15,
        n_kv_heads=5, head_dim=64, w_teacher=4096, w_student=256, d_model=960,
        d_ff=2560, chunk=512, conv_k=4, seed=2),
    3: LayerConfig(
        name="qwen3_0p6b_64k", dtype="bf16", batch=1, seq=65536, n_q_heads=16,
        n_kv_heads=8, head_dim=128, w_teacher=8192, w_student=512, d_model=1024,
        d_ff=3072, chunk=1024, conv_k=4, seed=3),
    4: LayerConfig(
        name="attn_b8_32k_sweep", dtype="bf16", batch=8, seq=32768, n_q_heads=16,
        n_kv_heads=8, head_dim=128, w_teacher=8192, w_student=512, seed=4,
        windows=((2048, 128), (8192, 512), (16384, 2048)), outlier_frac=0.05,
        outlier_scale=8.0),
    5: LayerConfig(
        name="decode_b32_64k", dtype="bf16", batch=32, seq=1, n_q_heads=16,
        n_kv_heads=8, head_dim=128, w_teacher=8192, w_student=512, d_model=1024,
        d_ff=3072, chunk=1024, conv_k=4, seed=5, cache_len=65536),
}


# --------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------


def attention_inputs(cfg: LayerConfig, seed: Optional[int] = None,
                     seq: Optional[int] = None) -> Dict[str, Tensor]:
    """Q [B,T,Hq,D], K/V [B,T,Hkv,D], all N(0,1).

    When the workload asks for it, a random 5 % of key rows (one row = one
    (batch, position, kv-head)) are scaled by 8 before rounding, to stress
    the softmax range.
    """
    s = cfg.seed if seed is None else seed
    T = cfg.seq if seq is None else seq
    B, Hq, Hkv, D = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    q = normal(s, "q", (B, T, Hq, D), 1.0, cfg.dtype)
    v = normal(s, "v", (B, T, Hkv, D), 1.0, cfg.dtype)
    k32 = _rng(s, "k").standard_normal(size=(B, T, Hkv, D), dtype=np.float32)
    if cfg.outlier_frac > 0.0:
        sel = _rng(s, "k_outlier").random(size=(B, T, Hkv)) < cfg.outlier_frac
        k32[sel] *= np.float32(cfg.outlier_scale)
    k = _store(k32, cfg.dtype)
    return {"q": q, "k": k, "v": v}


def layer_weights(cfg: LayerConfig, seed: Optional[int] = None) -> Dict[str, Tensor]:
    """Fan-in scaled Gaussian weights, unit RMSNorm gain.

    The write coefficients beta are drawn separately by ``beta_for``.
    """
    s = cfg.seed if seed is None else seed
    d, f, HD, kc = cfg.d_model, cfg.d_ff, cfg.n_q_heads * cfg.head_dim, cfg.conv_k
    dt = cfg.dtype
    return {
        "w_o": normal(s, "w_o", (d, HD), 1.0 / np.sqrt(HD), dt),
        "w_gate": normal(s, "w_gate", (f, d), 1.0 / np.sqrt(d), dt),
        "w_up": normal(s, "w_up", (f, d), 1.0 / np.sqrt(d), dt),
        "w_down0": normal(s, "w_down0", (d, f), 1.0 / np.sqrt(f), dt),
        "w_proj": normal(s, "w_proj", (f, f), 1.0 / np.sqrt(f), dt),
        "conv_t": normal(s, "conv_t", (f, kc), 1.0 / np.sqrt(kc), dt),
        "conv_s": normal(s, "conv_s", (f, kc), 1.0 / np.sqrt(kc), dt),
        "gamma": _store(np.ones((d,), np.float32), dt),
    }


def beta_for(cfg: LayerConfig, seed: Optional[int] = None, seq: Optional[int] = None,
             chunk_mean: bool = False) -> np.ndarray:
    """Write coefficients [B, n_chunks] (float32).

    beta_i ~ U(0,1) per (batch, chunk), the workloads' distribution: the
    exact coefficient of R_i K_i^T.  With ``chunk_mean`` the draw is divided
    by |C_i|, the number of tokens in chunk i (the last chunk may be short):
    a second, small-write regime in which the fast-weight correction is a
    few percent of the MLP output.
    """
    s = cfg.seed if seed is None else seed
    T = cfg.seq if seq is None else seq
    n = -(-T // cfg.chunk)
    u = _rng(s, "beta").random(size=(cfg.batch, n)).astype(np.float32)
    if not chunk_mean:
        return u
    sizes = np.full((n,), cfg.chunk, dtype=np.float32)
    sizes[-1] = T - cfg.chunk * (n - 1)
    return (u / sizes[None, :]).astype(np.float32)


def residual_input(cfg: LayerConfig, seed: Optional[int] = None,
                   seq: Optional[int] = None) -> Tensor:
    """x [B,T,d] ~ N(0,1): the residual stream entering the attention block."""
    s = cfg.seed if seed is None else seed
    T = cfg.seq if seq is None else seq
    return normal(s, "x", (cfg.batch, T, cfg.d_model), 1.0, cfg.dtype)


def hidden_activations(cfg: LayerConfig, seed: Optional[int] = None,
                       seq: Optional[int] = None) -> Dict[str, Tensor]:
    """Stand-alone SwiGLU activations Z_T, Z_S [B,T,f] for the fast-weight scan.

    Drawn as N(0, 0.36) (the spread of silu(g)*u for unit Gaussians g, u);
    Z_S = Z_T + an independent N(0, 0.09) perturbation, so the two paths are
    correlated the way a long and a short window over the same backbone are.
    """
    s = cfg.seed if seed is None else seed
    T = cfg.seq if seq is None else seq
    shape = (cfg.batch, T, cfg.d_ff)
    zt = _rng(s, "z_t").standard_normal(size=shape, dtype=np.float32)
    zt *= np.float32(0.6)
    pert = _rng(s, "z_s_pert").standard_normal(size=shape, dtype=np.float32)
    zs = zt + np.float32(0.3) * pert
    del pert
    return {"z_t": _store(zt, cfg.dtype), "z_s": _store(zs, cfg.dtype)}


def decode_inputs(cfg: LayerConfig, seed: Optional[int] = None) -> Dict[str, object]:
    """One decode step after a cache of ``cache_len`` tokens.

    Only the teacher window of the cache is drawn (positions
    [L - w_T + 1, L], the new token sits at L); everything older is a NaN
    sentinel on the device.  Returned K/V windows are [B, W, Hkv, D] with
    W = min(w_T, L + 1).  The fast-weight lists are drawn per sequence by
    ``decode_lists``.
    """
    s = cfg.seed if seed is None else seed
    B, L, Hq, Hkv, D = cfg.batch, cfg.cache_len, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    W = min(cfg.w_teacher, L + 1)
    dt = cfg.dtype
    out: Dict[str, object] = {}
    out["q"] = normal(s, "dec_q", (B, 1, Hq, D), 1.0, dt)
    out["k_win"] = normal(s, "dec_k", (B, W, Hkv, D), 1.0, dt)
    out["v_win"] = normal(s, "dec_v", (B, W, Hkv, D), 1.0, dt)
    out["x"] = normal(s, "dec_x", (B, 1, cfg.d_model), 1.0, dt)
    n = L // cfg.chunk
    out["beta_list"] = _rng(s, "dec_beta").random(size=(B, n)).astype(np.float32)
    out["n_chunks"] = n
    out["window_start"] = L + 1 - W
    return out


def decode_lists(cfg: LayerConfig, b: int, seed: Optional[int] = None) -> Tuple[Tensor, Tensor]:
    """Low-rank fast-weight lists of sequence ``b``: the n = L / C completed
    chunks, R rows ~ N(0, 1/L) [n*C, d] and K rows unit-norm Gaussians
    [n*C, f]."""
    s = cfg.seed if seed is None else seed
    L = cfg.cache_len
    n = L // cfg.chunk
    r = normal(s, f"dec_r_{b}", (n * cfg.chunk, cfg.d_model), 1.0 / np.sqrt(L), cfg.dtype)
    kr = _rng(s, f"dec_klist_{b}").standard_normal(size=(n * cfg.chunk, cfg.d_ff), dtype=np.float32)
    kr /= np.linalg.norm(kr, axis=-1, keepdims=True)
    return r, _store(kr, cfg.dtype)


def config_summary(cfg: LayerConfig) -> Dict[str, object]:
    keys = ["name", "dtype", "batch", "seq", "n_q_heads", "n_kv_heads", "head_dim",
            "w_teacher", "w_student", "d_model", "d_ff", "chunk", "conv_k"]
    return {k: getattr(cfg, k) for k in keys}


def to_torch(t: Tensor, device="cuda"):
    """Copy a host tensor to ``device`` in its storage type (bit exact)."""
    import torch

    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(t.data)).to(device)


def f32_to_torch(x: np.ndarray, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
