"""Thin Python binding of the C ABI in ``include/ttcd.h`` (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libttcd.so``.  PyTorch provides device memory and the current
stream.  Importing this module fails loudly if the library is missing.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libttcd.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first with "
        "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")

_lib = C.CDLL(LIB_PATH)

TTCD_F32, TTCD_BF16 = 0, 1
TTCD_MAIN_TEACHER, TTCD_MAIN_STUDENT = 0, 1

STATUS = {
    0: "TTCD_OK", 1: "TTCD_ERR_NULL_POINTER", 2: "TTCD_ERR_BAD_SHAPE",
    3: "TTCD_ERR_UNSUPPORTED", 4: "TTCD_ERR_WORKSPACE_TOO_SMALL", 5: "TTCD_ERR_ALIGNMENT",
    6: "TTCD_ERR_HIP",
}

EXPORTS = (
    "ttcd_dual_window_attn_workspace_size", "ttcd_dual_window_attn",
    "ttcd_dual_window_attn_lse_split_workspace_size", "ttcd_dual_window_attn_lse_split",
    "ttcd_dual_window_attn_backward_workspace_size", "ttcd_dual_window_attn_backward",
    "ttcd_fastweight_scan_workspace_size", "ttcd_fastweight_scan",
    "ttcd_fastweight_scan_on_policy_workspace_size", "ttcd_fastweight_scan_on_policy",
    "ttcd_fastweight_scan_eq6_workspace_size", "ttcd_fastweight_scan_eq6",
    "ttcd_fastweight_scan_backward_workspace_size", "ttcd_fastweight_scan_backward",
    "ttcd_fastweight_stream_workspace_size", "ttcd_fastweight_stream",
    "ttcd_layer_forward_workspace_size", "ttcd_layer_forward",
    "ttcd_layer_forward_noalloc_max_bytes", "ttcd_layer_forward_noalloc",
    "ttcd_fastweight_fold_workspace_size", "ttcd_fastweight_fold",
    "ttcd_fastweight_residual_proj_workspace_size", "ttcd_fastweight_residual_proj",
    "ttcd_fastweight_decode_append_workspace_size", "ttcd_fastweight_decode_append",
    "ttcd_status_string", "ttcd_last_error", "ttcd_version",
)


class AttnDesc(C.Structure):
    _fields_ = [("batch", C.c_int32), ("seq_q", C.c_int32), ("seq_k", C.c_int32),
                ("kv_rows", C.c_int32), ("q_pos0", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("w_teacher", C.c_int32),
                ("w_student", C.c_int32), ("scale", C.c_float), ("in_dtype", C.c_int32),
                ("out_dtype", C.c_int32)]


class FwDesc(C.Structure):
    _fields_ = [("batch", C.c_int32), ("seq", C.c_int32), ("d_model", C.c_int32),
                ("d_ff", C.c_int32), ("chunk", C.c_int32), ("conv_k", C.c_int32),
                ("l2_eps", C.c_float), ("in_dtype", C.c_int32), ("out_dtype", C.c_int32)]


class LayerWeights(C.Structure):
    _fields_ = [("w_o", C.c_void_p), ("rms_gamma", C.c_void_p), ("w_gate", C.c_void_p),
                ("w_up", C.c_void_p), ("w_down0", C.c_void_p), ("w_proj", C.c_void_p),
                ("conv_t", C.c_void_p), ("conv_s", C.c_void_p), ("beta", C.c_void_p)]


class LayerDesc(C.Structure):
    _fields_ = [("attn", AttnDesc), ("d_model", C.c_int32), ("d_ff", C.c_int32),
                ("chunk", C.c_int32), ("conv_k", C.c_int32), ("rms_eps", C.c_float),
                ("l2_eps", C.c_float), ("main_path", C.c_int32)]


class FwState(C.Structure):
    _fields_ = [("state_dense", C.c_void_p), ("r_list", C.c_void_p), ("k_list", C.c_void_p),
                ("beta_list", C.c_void_p), ("n_chunks", C.c_int32)]


class LayerAux(C.Structure):
    _fields_ = [("o_teacher", C.c_void_p), ("o_student", C.c_void_p),
                ("lse_teacher", C.c_void_p), ("lse_student", C.c_void_p),
                ("z_teacher", C.c_void_p), ("z_student", C.c_void_p), ("y", C.c_void_p),
                ("state_out", C.c_void_p), ("r", C.c_void_p), ("k", C.c_void_p)]


_vp, _sz = C.c_void_p, C.c_size_t
_sig = {
    "ttcd_dual_window_attn_workspace_size": (_sz, [C.POINTER(AttnDesc)]),
    "ttcd_dual_window_attn": (C.c_int, [C.POINTER(AttnDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _sz, _vp]),
    "ttcd_dual_window_attn_lse_split_workspace_size": (_sz, [C.POINTER(AttnDesc)]),
    "ttcd_dual_window_attn_lse_split": (C.c_int, [C.POINTER(AttnDesc), _vp, _vp, _vp, _vp, _vp,
                                                  _vp, _vp, _vp, _sz, _vp]),
    "ttcd_dual_window_attn_backward_workspace_size": (_sz, [C.POINTER(AttnDesc)]),
    "ttcd_dual_window_attn_backward": (C.c_int, [C.POINTER(AttnDesc)] + [_vp] * 13 + [_sz, _vp]),
    "ttcd_fastweight_scan_workspace_size": (_sz, [C.POINTER(FwDesc)]),
    "ttcd_fastweight_scan": (C.c_int, [C.POINTER(FwDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ttcd_fastweight_scan_on_policy_workspace_size": (_sz, [C.POINTER(FwDesc)]),
    "ttcd_fastweight_scan_on_policy": (C.c_int, [C.POINTER(FwDesc), _vp, _vp, _vp, _vp, _vp, _vp,
                                                 _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ttcd_fastweight_scan_eq6_workspace_size": (_sz, [C.POINTER(FwDesc)]),
    "ttcd_fastweight_scan_eq6": (C.c_int, [C.POINTER(FwDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _sz, _vp]),
    "ttcd_fastweight_scan_backward_workspace_size": (_sz, [C.POINTER(FwDesc)]),
    "ttcd_fastweight_scan_backward": (C.c_int, [C.POINTER(FwDesc)] + [_vp] * 18 + [_sz, _vp]),
    "ttcd_fastweight_stream_workspace_size": (_sz, [C.POINTER(FwDesc)]),
    "ttcd_fastweight_stream": (C.c_int, [C.POINTER(FwDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _vp, _vp, _sz, _vp]),
    "ttcd_layer_forward_workspace_size": (_sz, [C.POINTER(LayerDesc), C.POINTER(FwState)]),
    "ttcd_layer_forward": (C.c_int, [C.POINTER(LayerDesc), C.POINTER(LayerWeights), _vp, _vp,
                                     _vp, _vp, _vp, C.POINTER(FwState), C.POINTER(LayerAux),
                                     _vp, _sz, _vp]),
    "ttcd_layer_forward_noalloc_max_bytes": (_sz, []),
    "ttcd_layer_forward_noalloc": (C.c_int, [C.POINTER(LayerDesc), C.POINTER(LayerWeights), _vp,
                                             _vp, _vp, _vp, _vp, C.POINTER(FwState),
                                             C.POINTER(LayerAux), _vp]),
    "ttcd_fastweight_residual_proj_workspace_size": (_sz, [C.POINTER(FwDesc)]),
    "ttcd_fastweight_residual_proj": (C.c_int, [C.POINTER(FwDesc), _vp, _vp, _vp, _vp, _sz, _vp]),
    "ttcd_fastweight_decode_append_workspace_size": (_sz, [C.POINTER(FwDesc)]),
    "ttcd_fastweight_decode_append": (C.c_int, [C.POINTER(FwDesc), _vp, _vp, _vp, _vp, _vp, _vp,
                                                _vp, _vp, C.c_int64, _vp, C.c_int64, _vp, _sz,
                                                _vp]),
    "ttcd_fastweight_fold_workspace_size": (_sz, [C.POINTER(FwDesc), C.c_int32]),
    "ttcd_fastweight_fold": (C.c_int, [C.POINTER(FwDesc), _vp, _vp, _vp, _vp, C.c_int32, _vp,
                                       _vp, _sz, _vp]),
    "ttcd_status_string": (C.c_char_p, [C.c_int]),
    "ttcd_last_error": (C.c_char_p, []),
    "ttcd_version": (C.c_char_p, []),
}
for _name, (_res, _args) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class TTCDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.ttcd_last_error().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")


def _check(st: int, where: str) -> None:
    if st != 0:
        raise TTCDError(st, where)


def version() -> str:
    return _lib.ttcd_version().decode()


def lib() -> C.CDLL:
    return _lib


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TTCD_BF16
    if t.dtype == torch.float32:
        return TTCD_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _tdt(code: int) -> torch.dtype:
    return torch.bfloat16 if code == TTCD_BF16 else torch.float32


def _row_ptr(t: torch.Tensor) -> int:
    """Pointer of a [B, n] view whose rows are contiguous (any row stride)."""
    if not t.is_cuda:
        raise ValueError("tensors must live in GPU memory")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a [B, n] view with contiguous rows")
    return t.data_ptr()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream: Optional[torch.cuda.Stream] = None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------
# dual-window attention
# --------------------------------------------------------------------------


def attn_desc(q: torch.Tensor, k: torch.Tensor, w_teacher: int, w_student: int,
              scale: Optional[float] = None, q_pos0: int = 0, seq_k: Optional[int] = None,
              out_dtype: Optional[torch.dtype] = None) -> AttnDesc:
    B, Tq, Hq, D = q.shape
    rows = k.shape[1]
    sk = rows if seq_k is None else seq_k
    od = _dt(q) if out_dtype is None else (TTCD_BF16 if out_dtype == torch.bfloat16 else TTCD_F32)
    return AttnDesc(B, Tq, sk, rows, q_pos0, Hq, k.shape[2], D, w_teacher, w_student,
                    0.0 if scale is None else float(scale), _dt(q), od)


def dual_window_attn(q, k, v, w_teacher: int, w_student: int, *, scale=None, q_pos0: int = 0,
                     seq_k: Optional[int] = None, out_dtype=None, with_lse: bool = True,
                     out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None):
    """Teacher and student outputs of one shared Q/K/V.

    q [B,Tq,Hq,D], k/v [B,rows,Hkv,D] (rows >= seq_k).  Returns
    (o_teacher, o_student, lse_teacher, lse_student); LSEs are None unless
    ``with_lse``.
    """
    d = attn_desc(q, k, w_teacher, w_student, scale, q_pos0, seq_k, out_dtype)
    odt = _tdt(d.out_dtype)
    if out is None:
        o_t = torch.empty(q.shape, dtype=odt, device=q.device)
        o_s = torch.empty(q.shape, dtype=odt, device=q.device)
    else:
        o_t, o_s = out
    lse_t = lse_s = None
    if with_lse:
        lse_t = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
        lse_s = torch.empty_like(lse_t)
    need = _lib.ttcd_dual_window_attn_workspace_size(C.byref(d))
    ws = _workspace(need, q.device, workspace)
    _check(_lib.ttcd_dual_window_attn(C.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o_t), _ptr(o_s),
                                      _ptr(lse_t), _ptr(lse_s), _ptr(ws), ws.numel(),
                                      _stream(stream)), "ttcd_dual_window_attn")
    return o_t, o_s, lse_t, lse_s


def dual_window_attn_backward(q, k, v, o_teacher, o_student, lse_teacher, lse_student,
                              do_teacher, do_student, w_teacher: int, w_student: int, *,
                              scale=None, out_dtype=None, out=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of the teacher and student outputs given
    dO_T and dO_S (prefill: the forward's q, k, v, outputs and LSEs)."""
    d = attn_desc(q, k, w_teacher, w_student, scale, 0, None, out_dtype)
    odt = _tdt(d.out_dtype)
    if out is None:
        dq = torch.empty(q.shape, dtype=odt, device=q.device)
        dk = torch.empty(k.shape, dtype=odt, device=q.device)
        dv = torch.empty(v.shape, dtype=odt, device=q.device)
    else:
        dq, dk, dv = out
    need = _lib.ttcd_dual_window_attn_backward_workspace_size(C.byref(d))
    ws = _workspace(need, q.device, workspace)
    _check(_lib.ttcd_dual_window_attn_backward(
        C.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o_teacher), _ptr(o_student),
        _ptr(lse_teacher), _ptr(lse_student), _ptr(do_teacher), _ptr(do_student), _ptr(dq),
        _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), _stream(stream)),
        "ttcd_dual_window_attn_backward")
    return dq, dk, dv


def dual_window_attn_lse_split(q, k, v, w_teacher: int, w_student: int, *, scale=None,
                               q_pos0: int = 0, seq_k: Optional[int] = None, out_dtype=None,
                               with_lse: bool = True,
                               out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                               workspace: Optional[torch.Tensor] = None, stream=None):
    """The outputs of ``dual_window_attn`` through the LSE-combination path
    (student call, shifted far-band call, exact merge)."""
    d = attn_desc(q, k, w_teacher, w_student, scale, q_pos0, seq_k, out_dtype)
    odt = _tdt(d.out_dtype)
    if out is None:
        o_t = torch.empty(q.shape, dtype=odt, device=q.device)
        o_s = torch.empty(q.shape, dtype=odt, device=q.device)
    else:
        o_t, o_s = out
    lse_t = lse_s = None
    if with_lse:
        lse_t = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
        lse_s = torch.empty_like(lse_t)
    need = _lib.ttcd_dual_window_attn_lse_split_workspace_size(C.byref(d))
    ws = _workspace(need, q.device, workspace)
    _check(_lib.ttcd_dual_window_attn_lse_split(C.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o_t),
                                                _ptr(o_s), _ptr(lse_t), _ptr(lse_s), _ptr(ws),
                                                ws.numel(), _stream(stream)),
           "ttcd_dual_window_attn_lse_split")
    return o_t, o_s, lse_t, lse_s


# --------------------------------------------------------------------------
# fast-weight scan
# --------------------------------------------------------------------------


def fw_desc(z: torch.Tensor, d_model: int, chunk: int, conv_k: int, l2_eps: float = 0.0,
            out_dtype: torch.dtype = torch.float32) -> FwDesc:
    B, T, f = z.shape
    return FwDesc(B, T, d_model, f, chunk, conv_k, l2_eps, _dt(z),
                  TTCD_BF16 if out_dtype == torch.bfloat16 else TTCD_F32)


def fastweight_scan(z_teacher, z_student, z_main, conv_t, conv_s, w_down0, w_proj, beta,
                    chunk: int, *, out_dtype=torch.float32, want_state: bool = False,
                    r_out: Optional[torch.Tensor] = None, k_out: Optional[torch.Tensor] = None,
                    l2_eps: float = 0.0, workspace=None, stream=None):
    """y [B,T,d] = S_{t//chunk} z_main[t] with the chunk-wise prefix fast weight.

    Returns (y, state) where state is the fp32 weight after the writes of
    the T // chunk complete chunks (or None).  r_out [B,T,d] and k_out
    [B,T,f] (the inputs' dtype, caller-allocated) receive the residual terms
    and unit keys of the low-rank chunk lists when given."""
    dm = w_down0.shape[0]
    kc = conv_t.shape[1]
    d = fw_desc(z_teacher, dm, chunk, kc, l2_eps, out_dtype)
    B, T, f = z_teacher.shape
    y = torch.empty((B, T, dm), dtype=out_dtype, device=z_teacher.device)
    st = torch.empty((B, dm, f), dtype=torch.float32, device=z_teacher.device) if want_state else None
    need = _lib.ttcd_fastweight_scan_workspace_size(C.byref(d))
    ws = _workspace(need, z_teacher.device, workspace)
    _check(_lib.ttcd_fastweight_scan(C.byref(d), _ptr(z_teacher), _ptr(z_student), _ptr(z_main),
                                     _ptr(conv_t), _ptr(conv_s), _ptr(w_down0), _ptr(w_proj),
                                     _ptr(beta), _ptr(y), _ptr(st), _ptr(r_out), _ptr(k_out),
                                     _ptr(ws), ws.numel(), _stream(stream)), "ttcd_fastweight_scan")
    return y, st


def fastweight_scan_on_policy(z_teacher, z_student, z_main, conv_t, conv_s, w_down0, w_proj,
                              beta, chunk: int, *, out_dtype=torch.float32,
                              want_state: bool = False, l2_eps: float = 0.0,
                              workspace=None, stream=None):
    """fastweight_scan with the on-policy recurrence: the residual of chunk i
    is projected by the fast weight in force for chunk i, not by W_down^(0).
    Returns (y, state) as fastweight_scan does."""
    dm = w_down0.shape[0]
    kc = conv_t.shape[1]
    d = fw_desc(z_teacher, dm, chunk, kc, l2_eps, out_dtype)
    B, T, f = z_teacher.shape
    y = torch.empty((B, T, dm), dtype=out_dtype, device=z_teacher.device)
    st = torch.empty((B, dm, f), dtype=torch.float32, device=z_teacher.device) if want_state else None
    need = _lib.ttcd_fastweight_scan_on_policy_workspace_size(C.byref(d))
    ws = _workspace(need, z_teacher.device, workspace)
    _check(_lib.ttcd_fastweight_scan_on_policy(
        C.byref(d), _ptr(z_teacher), _ptr(z_student), _ptr(z_main), _ptr(conv_t), _ptr(conv_s),
        _ptr(w_down0), _ptr(w_proj), _ptr(beta), _ptr(y), _ptr(st), _ptr(ws), ws.numel(),
        _stream(stream)), "ttcd_fastweight_scan_on_policy")
    return y, st


def fastweight_scan_eq6(z_teacher, z_student, z_main, w_down0, beta, chunk: int, *,
                        out_dtype=torch.float32, want_state: bool = False, workspace=None,
                        stream=None):
    """The unprojected write: r_t = W0 (z_T - z_S), raw keys z_S, no convs or
    W_proj; chunk prefix and apply as in fastweight_scan.  Returns (y, state)."""
    dm = w_down0.shape[0]
    d = fw_desc(z_teacher, dm, chunk, 1, 0.0, out_dtype)
    B, T, f = z_teacher.shape
    y = torch.empty((B, T, dm), dtype=out_dtype, device=z_teacher.device)
    st = torch.empty((B, dm, f), dtype=torch.float32, device=z_teacher.device) if want_state else None
    need = _lib.ttcd_fastweight_scan_eq6_workspace_size(C.byref(d))
    ws = _workspace(need, z_teacher.device, workspace)
    _check(_lib.ttcd_fastweight_scan_eq6(C.byref(d), _ptr(z_teacher), _ptr(z_student),
                                         _ptr(z_main), _ptr(w_down0), _ptr(beta), _ptr(y),
                                         _ptr(st), _ptr(ws), ws.numel(), _stream(stream)),
           "ttcd_fastweight_scan_eq6")
    return y, st


def fastweight_scan_backward(z_teacher, z_student, z_main, conv_t, conv_s, w_down0, w_proj,
                             beta, dy, chunk: int, *, out_dtype=torch.float32,
                             l2_eps: float = 0.0, out=None, workspace=None, stream=None):
    """Gradients of fastweight_scan's y given dy [B,T,d] (the inputs' dtype).

    Returns a dict: dz_t, dz_s, dz_main [B,T,f] (out_dtype), dconv_t,
    dconv_s [f,kc], dw_down0 [d,f], dw_proj [f,f] (fp32, summed over the
    batch) and dbeta [B, n_chunks] (fp32).  ``out``: such a dict to write
    into (from an earlier call of the same shapes)."""
    dm = w_down0.shape[0]
    kc = conv_t.shape[1]
    d = fw_desc(z_teacher, dm, chunk, kc, l2_eps, out_dtype)
    B, T, f = z_teacher.shape
    dev = z_teacher.device
    if out is not None:
        g = out
    else:
        g = {n: torch.empty((B, T, f), dtype=out_dtype, device=dev)
             for n in ("dz_t", "dz_s", "dz_main")}
        g["dconv_t"] = torch.empty((f, kc), dtype=torch.float32, device=dev)
        g["dconv_s"] = torch.empty((f, kc), dtype=torch.float32, device=dev)
        g["dw_down0"] = torch.empty((dm, f), dtype=torch.float32, device=dev)
        g["dw_proj"] = torch.empty((f, f), dtype=torch.float32, device=dev)
        g["dbeta"] = torch.empty((B, -(-T // chunk)), dtype=torch.float32, device=dev)
    shapes = {"dz_t": (B, T, f), "dz_s": (B, T, f), "dz_main": (B, T, f), "dconv_t": (f, kc),
              "dconv_s": (f, kc), "dw_down0": (dm, f), "dw_proj": (f, f),
              "dbeta": (B, -(-T // chunk))}
    for n, shp in shapes.items():
        want = out_dtype if n.startswith("dz") else torch.float32
        if tuple(g[n].shape) != shp or g[n].dtype != want or not g[n].is_contiguous():
            raise ValueError(f"fastweight_scan_backward: out[{n!r}] must be a contiguous "
                             f"{want} tensor of shape {shp}")
    need = _lib.ttcd_fastweight_scan_backward_workspace_size(C.byref(d))
    ws = _workspace(need, dev, workspace)
    _check(_lib.ttcd_fastweight_scan_backward(
        C.byref(d), _ptr(z_teacher), _ptr(z_student), _ptr(z_main), _ptr(conv_t), _ptr(conv_s),
        _ptr(w_down0), _ptr(w_proj), _ptr(beta), _ptr(dy), _ptr(g["dz_t"]), _ptr(g["dz_s"]),
        _ptr(g["dz_main"]), _ptr(g["dconv_t"]), _ptr(g["dconv_s"]), _ptr(g["dw_down0"]),
        _ptr(g["dw_proj"]), _ptr(g["dbeta"]), _ptr(ws), ws.numel(), _stream(stream)),
        "ttcd_fastweight_scan_backward")
    return g


def stream_pad(seq: int) -> int:
    return (seq + 63) // 64 * 64


def fastweight_stream(z_teacher, z_student, conv_t, conv_s, beta, chunk: int, *,
                      l2_eps: float = 0.0, out=None, workspace=None, stream=None):
    """The stream step alone.  Returns (dbar [B,Tp,f], zbar_s_t [B,f,Tp],
    key_scale [B,Tp]) with Tp = stream_pad(T); rows >= T are zero."""
    B, T, f = z_teacher.shape
    kc = conv_t.shape[1]
    d = fw_desc(z_teacher, 8, chunk, kc, l2_eps)
    Tp = stream_pad(T)
    dev, dt = z_teacher.device, z_teacher.dtype
    if out is None:
        out = (torch.empty((B, Tp, f), dtype=dt, device=dev),
               torch.empty((B, f, Tp), dtype=dt, device=dev),
               torch.empty((B, Tp), dtype=torch.float32, device=dev))
    dbar, zbt, ks = out
    need = _lib.ttcd_fastweight_stream_workspace_size(C.byref(d))
    ws = _workspace(need, dev, workspace)
    _check(_lib.ttcd_fastweight_stream(C.byref(d), _ptr(z_teacher), _ptr(z_student), _ptr(conv_t),
                                       _ptr(conv_s), _ptr(beta), _ptr(dbar), _ptr(zbt), _ptr(ks),
                                       _ptr(ws), ws.numel(), _stream(stream)),
           "ttcd_fastweight_stream")
    return dbar, zbt, ks


def fastweight_residual_proj(w_down0, w_proj, *, workspace=None, stream=None):
    """M = W_down0 W_proj [d, f] in the weights' dtype (decode set-up)."""
    dm, f = w_down0.shape
    d = FwDesc(1, 1, dm, f, 16, 1, 0.0, _dt(w_down0), TTCD_F32)
    m = torch.empty((dm, f), dtype=w_down0.dtype, device=w_down0.device)
    ws = _workspace(_lib.ttcd_fastweight_residual_proj_workspace_size(C.byref(d)),
                    w_down0.device, workspace)
    _check(_lib.ttcd_fastweight_residual_proj(C.byref(d), _ptr(w_down0), _ptr(w_proj), _ptr(m),
                                              _ptr(ws), ws.numel(), _stream(stream)),
           "ttcd_fastweight_residual_proj")
    return m


def fastweight_decode_append(z_teacher, z_student, hist_t, hist_s, conv_t, conv_s, m,
                             r_out, k_out, *, l2_eps: float = 0.0, workspace=None,
                             stream=None):
    """The fast-weight stream for one generated token per sequence.

    z_teacher, z_student [B, f] (or [B, 1, f]); hist_t, hist_s [B, kc-1, f]
    advance in place; r_out [B, d] and k_out [B, f] may be row views of
    chunk-list buffers (stride(1) must be 1).
    """
    B, f = r_out.shape[0], k_out.shape[-1]
    dm = r_out.shape[-1]
    kc = conv_t.shape[1]
    if r_out.stride(-1) != 1 or k_out.stride(-1) != 1:
        raise ValueError("r_out and k_out rows must be contiguous")
    d = FwDesc(B, 1, dm, f, 16, kc, l2_eps, _dt(z_teacher), TTCD_F32)
    ws = _workspace(_lib.ttcd_fastweight_decode_append_workspace_size(C.byref(d)),
                    z_teacher.device, workspace)
    _check(_lib.ttcd_fastweight_decode_append(
        C.byref(d), _ptr(z_teacher), _ptr(z_student), _ptr(hist_t), _ptr(hist_s), _ptr(conv_t),
        _ptr(conv_s), _ptr(m), _row_ptr(r_out), int(r_out.stride(0)), _row_ptr(k_out),
        int(k_out.stride(0)), _ptr(ws), ws.numel(), _stream(stream)),
        "ttcd_fastweight_decode_append")


def fastweight_fold(w_down0, r_list, k_list, beta_list, chunk: int, *, workspace=None,
                    stream=None):
    """Dense fp32 weight W_down0 + sum_j beta_j R_j^T K_j from chunk lists."""
    B = r_list.shape[0]
    n = beta_list.shape[1]
    dm, f = w_down0.shape
    d = FwDesc(B, max(1, n * chunk), dm, f, chunk, 1, 0.0, _dt(w_down0), TTCD_F32)
    out = torch.empty((B, dm, f), dtype=torch.float32, device=w_down0.device)
    need = _lib.ttcd_fastweight_fold_workspace_size(C.byref(d), n)
    ws = _workspace(need, w_down0.device, workspace)
    _check(_lib.ttcd_fastweight_fold(C.byref(d), _ptr(w_down0), _ptr(r_list), _ptr(k_list),
                                     _ptr(beta_list), n, _ptr(out), _ptr(ws), ws.numel(),
                                     _stream(stream)), "ttcd_fastweight_fold")
    return out


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------


def layer_desc(q, k, d_model: int, d_ff: int, w_teacher: int, w_student: int, chunk: int,
               conv_k: int, *, rms_eps: float = 1e-6, l2_eps: float = 1e-12,
               main_path: str = "teacher", q_pos0: int = 0, seq_k: Optional[int] = None,
               scale=None) -> LayerDesc:
    a = attn_desc(q, k, w_teacher, w_student, scale, q_pos0, seq_k)
    mp = TTCD_MAIN_TEACHER if main_path == "teacher" else TTCD_MAIN_STUDENT
    return LayerDesc(a, d_model, d_ff, chunk, conv_k, rms_eps, l2_eps, mp)


def layer_forward(q, k, v, x, w: Dict[str, torch.Tensor], w_teacher: int, w_student: int,
                  chunk: int, *, rms_eps: float = 1e-6, l2_eps: float = 1e-12,
                  main_path: str = "teacher", aux: bool = False,
                  decode: Optional[Dict[str, object]] = None, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None,
                  no_alloc: bool = False):
    """IP-TTCD layer forward.  Returns out [B,Tq,d] fp32, or (out, aux dict).
    aux=True returns every intermediate; aux="fw" only the fast-weight ones
    (y, and in a prefill the state and the chunk lists R, K), which keeps the
    layer's O and Z internal (the launch configuration of a plain call).

    w: w_o, w_gate, w_up, w_down0, w_proj, conv_t, conv_s, beta, optional
    gamma.  decode: dict(pos=L, state_dense=..., r_list=, k_list=,
    beta_list=) for one generated token (q is [B,1,Hq,D], k/v hold the
    cache with the new token at row L).  no_alloc: run through
    ttcd_layer_forward_noalloc (the library's own scratch; no workspace is
    allocated here).
    """
    dm, f = w["w_down0"].shape
    kc = w["conv_t"].shape[1] if w.get("conv_t") is not None else 4
    if decode is None:
        desc = layer_desc(q, k, dm, f, w_teacher, w_student, chunk, kc, rms_eps=rms_eps,
                          l2_eps=l2_eps, main_path=main_path)
        dec_p = None
        dec = None
    else:
        pos = int(decode["pos"])
        desc = layer_desc(q, k, dm, f, w_teacher, w_student, chunk, kc, rms_eps=rms_eps,
                          l2_eps=l2_eps, main_path=main_path, q_pos0=pos, seq_k=pos + 1)
        bl = decode.get("beta_list")
        dec = FwState(_ptr(decode.get("state_dense")), _ptr(decode.get("r_list")),
                      _ptr(decode.get("k_list")), _ptr(bl),
                      0 if bl is None else int(bl.shape[1]))
        dec_p = C.byref(dec)
    wt = LayerWeights(_ptr(w["w_o"]), _ptr(w.get("gamma")), _ptr(w["w_gate"]), _ptr(w["w_up"]),
                      _ptr(w["w_down0"]), _ptr(w.get("w_proj")), _ptr(w.get("conv_t")),
                      _ptr(w.get("conv_s")), _ptr(w.get("beta")))
    B, Tq = q.shape[0], q.shape[1]
    dev = q.device
    if out is None:
        out = torch.empty((B, Tq, dm), dtype=torch.float32, device=dev)
    aux_t: Dict[str, torch.Tensor] = {}
    aux_s = None
    if aux:
        Hq = q.shape[2]
        if aux != "fw":
            aux_t["o_teacher"] = torch.empty(q.shape, dtype=q.dtype, device=dev)
            aux_t["o_student"] = torch.empty(q.shape, dtype=q.dtype, device=dev)
            aux_t["lse_teacher"] = torch.empty((B, Hq, Tq), dtype=torch.float32, device=dev)
            aux_t["lse_student"] = torch.empty((B, Hq, Tq), dtype=torch.float32, device=dev)
            aux_t["z_teacher"] = torch.empty((B, Tq, f), dtype=q.dtype, device=dev)
            # in a decode step both Z are returned too: they feed the
            # fast-weight append of the token (fastweight_decode_append)
            aux_t["z_student"] = torch.empty((B, Tq, f), dtype=q.dtype, device=dev)
        aux_t["y"] = torch.empty((B, Tq, dm), dtype=torch.float32, device=dev)
        if decode is None:
            aux_t["state_out"] = torch.empty((B, dm, f), dtype=torch.float32, device=dev)
            aux_t["r"] = torch.empty((B, Tq, dm), dtype=q.dtype, device=dev)
            aux_t["k"] = torch.empty((B, Tq, f), dtype=q.dtype, device=dev)
        aux_s = LayerAux(*[_ptr(aux_t.get(n)) for n, _ in LayerAux._fields_])
    aux_p = C.byref(aux_s) if aux_s is not None else None
    if no_alloc:
        _check(_lib.ttcd_layer_forward_noalloc(C.byref(desc), C.byref(wt), _ptr(q), _ptr(k),
                                               _ptr(v), _ptr(x), _ptr(out), dec_p, aux_p,
                                               _stream(stream)), "ttcd_layer_forward_noalloc")
    else:
        need = _lib.ttcd_layer_forward_workspace_size(C.byref(desc), dec_p)
        ws = _workspace(need, dev, workspace)
        _check(_lib.ttcd_layer_forward(C.byref(desc), C.byref(wt), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(x), _ptr(out), dec_p, aux_p, _ptr(ws), ws.numel(),
                                       _stream(stream)), "ttcd_layer_forward")
    if aux:
        return out, aux_t
    return out


def layer_workspace_bytes(q, k, d_model, d_ff, w_teacher, w_student, chunk, conv_k=4,
                          decode_chunks: Optional[int] = None, pos: Optional[int] = None) -> int:
    if decode_chunks is None:
        desc = layer_desc(q, k, d_model, d_ff, w_teacher, w_student, chunk, conv_k)
        return int(_lib.ttcd_layer_forward_workspace_size(C.byref(desc), None))
    desc = layer_desc(q, k, d_model, d_ff, w_teacher, w_student, chunk, conv_k, q_pos0=pos,
                      seq_k=pos + 1)
    dec = FwState(None, None, None, None, decode_chunks)
    return int(_lib.ttcd_layer_forward_workspace_size(C.byref(desc), C.byref(dec)))
