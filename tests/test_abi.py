"""The C-ABI library loads on the host, exports every symbol the header
declares, sizes workspaces and rejects bad arguments before touching the GPU.
CPU only: no call here reaches a kernel launch."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttcd.h")
LIB = os.path.join(ROOT, "dual_window_attention_amd", "libttcd.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libttcd.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s\*]*?\b(ttcd_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_function_is_exported():
    lib = C.CDLL(LIB)
    names = header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    from dual_window_attention_amd import ttcd
    assert sorted(ttcd.EXPORTS) == names


def test_version_and_status_strings():
    from dual_window_attention_amd import ttcd
    assert "gfx950" in ttcd.version()
    lib = ttcd.lib()
    assert lib.ttcd_status_string(0) == b"TTCD_OK"
    assert lib.ttcd_status_string(4) == b"TTCD_ERR_WORKSPACE_TOO_SMALL"


def _attn(**kw):
    from dual_window_attention_amd import ttcd
    base = dict(batch=1, seq_q=65536, seq_k=65536, kv_rows=0, q_pos0=0, n_q_heads=16,
                n_kv_heads=8, head_dim=128, w_teacher=8192, w_student=512, scale=0.0,
                in_dtype=1, out_dtype=1)
    base.update(kw)
    return ttcd.AttnDesc(**base)


def test_workspace_sizes():
    from dual_window_attention_amd import ttcd
    lib = ttcd.lib()
    d = _attn()
    # the transposed V staging copy: B * Hkv * D * T bf16
    assert lib.ttcd_dual_window_attn_workspace_size(C.byref(d)) == 8 * 128 * 65536 * 2
    dd = _attn(seq_q=1, q_pos0=65536, seq_k=65537, batch=32)
    assert 0 < lib.ttcd_dual_window_attn_workspace_size(C.byref(dd)) < 64 << 20
    fw = ttcd.FwDesc(1, 65536, 1024, 3072, 1024, 4, 0.0, 1, 0)
    n = lib.ttcd_fastweight_scan_workspace_size(C.byref(fw))
    # dbar + zbar^T (2 x T f) + 63 prefix weights (d f) + ...
    assert n > (2 * 65536 * 3072 + 63 * 1024 * 3072) * 2
    bad = _attn(head_dim=96)
    assert lib.ttcd_dual_window_attn_workspace_size(C.byref(bad)) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 3),
    (dict(w_student=9000), 2),
    (dict(w_student=0), 2),
    (dict(n_q_heads=12, n_kv_heads=8), 2),
    (dict(seq_q=10, seq_k=5), 2),
    (dict(in_dtype=7), 3),
])
def test_attention_rejects_bad_descriptors(kw, status):
    from dual_window_attention_amd import ttcd
    lib = ttcd.lib()
    d = _attn(**kw)
    fake = C.c_void_p(1 << 20)
    st = lib.ttcd_dual_window_attn(C.byref(d), fake, fake, fake, fake, fake, None, None, fake,
                                   1 << 40, None)
    assert st == status, lib.ttcd_last_error()
    assert lib.ttcd_last_error() != b""


@pytest.mark.parametrize("kw", [dict(seq_q=0), dict(seq_q=0, seq_k=0), dict(batch=0),
                                dict(seq_q=1, seq_k=0)])
def test_empty_attention_is_an_error(kw):
    """An empty call is TTCD_ERR_BAD_SHAPE (the header's stated behaviour),
    before any device work, and sizes no workspace."""
    from dual_window_attention_amd import ttcd
    lib = ttcd.lib()
    d = _attn(**kw)
    fake = C.c_void_p(1 << 20)
    assert lib.ttcd_dual_window_attn(C.byref(d), fake, fake, fake, fake, fake, None, None, fake,
                                     1 << 40, None) == 2
    assert b">= 1" in lib.ttcd_last_error()
    assert lib.ttcd_dual_window_attn_workspace_size(C.byref(d)) == 0


def test_empty_fastweight_and_layer_are_errors():
    from dual_window_attention_amd import ttcd
    lib = ttcd.lib()
    fake = C.c_void_p(1 << 20)
    for b, t in ((1, 0), (0, 64)):
        fw = ttcd.FwDesc(b, t, 1024, 3072, 64, 4, 0.0, 1, 0)
        assert lib.ttcd_fastweight_scan_workspace_size(C.byref(fw)) == 0
        assert lib.ttcd_fastweight_scan(C.byref(fw), *([fake] * 12), fake, 1 << 40, None) == 2
    ld = ttcd.LayerDesc(_attn(seq_q=0, seq_k=0), 1024, 3072, 1024, 4, 0.0, 0.0, 0)
    w = ttcd.LayerWeights(*([1 << 20] * 8), 1 << 20)
    assert lib.ttcd_layer_forward_workspace_size(C.byref(ld), None) == 0
    assert lib.ttcd_layer_forward(C.byref(ld), C.byref(w), fake, fake, fake, fake, fake, None,
                                  None, fake, 1 << 40, None) == 2


def test_size_limits_at_and_past_the_maximum():
    """The largest accepted sizes are sized (no overflow in the size
    arithmetic), one row more is rejected: attention rows
    batch * max(seq_q, kv_rows) * n_q_heads < 2^31 (32-bit row indices in
    the kernels), fast-weight and layer tokens batch * seq <= 2^28."""
    from dual_window_attention_amd import ttcd
    lib = ttcd.lib()
    top = (1 << 27) - 1                                       # x 16 q heads < 2^31
    d = _attn(seq_q=top, seq_k=top)
    assert lib.ttcd_dual_window_attn_workspace_size(C.byref(d)) == 8 * 128 * ((top + 63) // 64 * 64) * 2
    d = _attn(seq_q=top + 1, seq_k=top + 1)
    assert lib.ttcd_dual_window_attn_workspace_size(C.byref(d)) == 0
    d = _attn(seq_q=1, q_pos0=100, seq_k=101, kv_rows=top + 1)    # a decode cache counts too
    assert lib.ttcd_dual_window_attn_workspace_size(C.byref(d)) == 0
    fw = ttcd.FwDesc(1, 1 << 28, 64, 64, 64, 4, 0.0, 1, 0)
    assert lib.ttcd_fastweight_scan_workspace_size(C.byref(fw)) > (1 << 28) * 64 * 2 * 2
    fw = ttcd.FwDesc(2, (1 << 27) + 1, 64, 64, 64, 4, 0.0, 1, 0)
    assert lib.ttcd_fastweight_scan_workspace_size(C.byref(fw)) == 0
    one = dict(n_q_heads=1, n_kv_heads=1, head_dim=64, w_teacher=64, w_student=16)
    ld = ttcd.LayerDesc(_attn(batch=4, seq_q=1 << 26, seq_k=1 << 26, **one), 64, 64, 64, 4,
                        0.0, 0.0, 0)
    assert lib.ttcd_layer_forward_workspace_size(C.byref(ld), None) > 0
    ld = ttcd.LayerDesc(_attn(batch=5, seq_q=1 << 26, seq_k=1 << 26, **one), 64, 64, 64, 4,
                        0.0, 0.0, 0)
    assert lib.ttcd_layer_forward_workspace_size(C.byref(ld), None) == 0


def test_attention_rejects_null_misaligned_and_small_workspace():
    from dual_window_attention_amd import ttcd
    lib = ttcd.lib()
    d = _attn()
    fake = C.c_void_p(1 << 20)
    assert lib.ttcd_dual_window_attn(C.byref(d), None, fake, fake, fake, fake, None, None, fake,
                                     1 << 40, None) == 1
    odd = C.c_void_p((1 << 20) + 2)
    assert lib.ttcd_dual_window_attn(C.byref(d), fake, odd, fake, fake, fake, None, None, fake,
                                     1 << 40, None) == 5
    assert lib.ttcd_dual_window_attn(C.byref(d), fake, fake, fake, fake, fake, None, None, fake,
                                     16, None) == 4
    assert b"workspace" in lib.ttcd_last_error()


def test_fastweight_and_layer_reject_bad_shapes():
    from dual_window_attention_amd import ttcd
    lib = ttcd.lib()
    fake = C.c_void_p(1 << 20)
    fw = ttcd.FwDesc(1, 100, 1024, 3072, 24, 4, 0.0, 1, 0)     # chunk not a multiple of 16
    assert lib.ttcd_fastweight_scan(C.byref(fw), *([fake] * 12), fake, 1 << 40, None) == 2
    fw = ttcd.FwDesc(1, 100, 1024, 3072, 64, 9, 0.0, 1, 0)      # conv_k > 8
    assert lib.ttcd_fastweight_scan(C.byref(fw), *([fake] * 12), fake, 1 << 40, None) == 2
    # the list outputs are optional but must be aligned when given
    fw = ttcd.FwDesc(1, 100, 1024, 3072, 64, 4, 0.0, 1, 0)
    odd = C.c_void_p((1 << 20) + 2)
    assert lib.ttcd_fastweight_scan(C.byref(fw), *([fake] * 10), odd, None, fake, 1 << 40,
                                    None) == 5
    assert lib.ttcd_fastweight_scan(C.byref(fw), *([fake] * 10), None, odd, fake, 1 << 40,
                                    None) == 5
    a = _attn(seq_q=128, seq_k=128)
    ld = ttcd.LayerDesc(a, 1004, 3072, 1024, 4, 0.0, 0.0, 0)   # d_model not a multiple of 8
    w = ttcd.LayerWeights(*([1 << 20] * 8), 1 << 20)
    assert lib.ttcd_layer_forward(C.byref(ld), C.byref(w), fake, fake, fake, fake, fake, None,
                                  None, fake, 1 << 40, None) == 2
    ld = ttcd.LayerDesc(_attn(seq_q=1, seq_k=128, q_pos0=127), 1024, 3072, 1024, 4, 0.0, 0.0, 0)
    # one query without a decode state is not a prefill
    assert lib.ttcd_layer_forward(C.byref(ld), C.byref(w), fake, fake, fake, fake, fake, None,
                                  None, fake, 1 << 40, None) == 2
    dec = ttcd.FwState(None, None, None, None, 3)
    assert lib.ttcd_layer_forward(C.byref(ld), C.byref(w), fake, fake, fake, fake, fake,
                                  C.byref(dec), None, fake, 1 << 40, None) == 1
    # the list outputs of a prefill are not outputs of a decode step
    dec = ttcd.FwState(fake, None, None, None, 0)
    aux = ttcd.LayerAux(*([None] * 8), fake, None)
    assert lib.ttcd_layer_forward(C.byref(ld), C.byref(w), fake, fake, fake, fake, fake,
                                  C.byref(dec), C.byref(aux), fake, 1 << 40, None) == 2
    assert b"prefill-only" in lib.ttcd_last_error()


def test_no_oracle_import_in_product_code():
    """The product path (package + C sources) never imports the oracle."""
    pkg = os.path.join(ROOT, "dual_window_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, flags=re.M), fn
                assert "ttcd_oracle" not in text, fn


def test_update_rule_variants_validate_before_any_launch():
    """The on-policy and unprojected-write entry points check shapes,
    pointers and workspace size on the host and return an error code."""
    from dual_window_attention_amd import ttcd
    lib = ttcd.lib()
    fake = C.c_void_p(1 << 20)
    good = ttcd.FwDesc(1, 65536, 1024, 3072, 1024, 4, 0.0, 1, 0)
    n_scan = lib.ttcd_fastweight_scan_workspace_size(C.byref(good))
    n_on = lib.ttcd_fastweight_scan_on_policy_workspace_size(C.byref(good))
    n_e6 = lib.ttcd_fastweight_scan_eq6_workspace_size(C.byref(good))
    # on-policy adds the fp32 running state, U = Dbar W_proj^T and the split partials
    assert n_on >= n_scan + (1024 * 3072 * 4 + 65536 * 3072 * 2)
    # the unprojected write adds one row of unit taps
    assert n_scan < n_e6 <= n_scan + 3072 * 2 + 256
    bad = ttcd.FwDesc(1, 100, 1024, 3072, 24, 4, 0.0, 1, 0)     # chunk not a multiple of 16
    assert lib.ttcd_fastweight_scan_on_policy_workspace_size(C.byref(bad)) == 0
    assert lib.ttcd_fastweight_scan_eq6_workspace_size(C.byref(bad)) == 0
    assert lib.ttcd_fastweight_scan_on_policy(C.byref(bad), *([fake] * 10), fake, 1 << 40,
                                              None) == 2
    assert lib.ttcd_fastweight_scan_eq6(C.byref(bad), *([fake] * 7), fake, 1 << 40, None) == 2
    # a NULL input, then too small a workspace
    args = [fake] * 10
    args[0] = None
    assert lib.ttcd_fastweight_scan_on_policy(C.byref(good), *args, fake, 1 << 40, None) == 1
    assert lib.ttcd_fastweight_scan_eq6(C.byref(good), None, *([fake] * 6), fake, 1 << 40,
                                        None) == 1
    assert lib.ttcd_fastweight_scan_on_policy(C.byref(good), *([fake] * 10), fake, n_on - 1,
                                              None) == 4
    assert lib.ttcd_fastweight_scan_eq6(C.byref(good), *([fake] * 7), fake, n_e6 - 1, None) == 4


def test_noalloc_layer_entry_rejects_calls_beyond_its_scratch():
    """The no-allocation layer entry point states its scratch size and
    rejects, on the host, a call whose workspace would not fit (a 64K
    prefill) and a call with a NULL input."""
    from dual_window_attention_amd import ttcd
    lib = ttcd.lib()
    assert lib.ttcd_layer_forward_noalloc_max_bytes() == 64 << 20
    fake = C.c_void_p(1 << 20)
    a = _attn(seq_q=65536, seq_k=65536)
    ld = ttcd.LayerDesc(a, 1024, 3072, 1024, 4, 0.0, 0.0, 0)
    w = ttcd.LayerWeights(*([1 << 20] * 8), 1 << 20)
    assert lib.ttcd_layer_forward_workspace_size(C.byref(ld), None) > 64 << 20
    assert lib.ttcd_layer_forward_noalloc(C.byref(ld), C.byref(w), fake, fake, fake, fake, fake,
                                          None, None, None) == 4
    assert b"no-allocation" in lib.ttcd_last_error()
    assert lib.ttcd_layer_forward_noalloc(C.byref(ld), C.byref(w), None, fake, fake, fake, fake,
                                          None, None, None) == 1


def header_param_counts():
    """Number of parameters of every function the header declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(ttcd_\w+)\s*\(([^;{]*?)\)\s*;", text, flags=re.S):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argument_counts_match_the_header():
    """Every ctypes signature in the binding passes exactly the header's
    parameters (an argument too few shifts the stream handle into a
    variadic slot, where ctypes passes it as a 32-bit int)."""
    from dual_window_attention_amd import ttcd
    counts = header_param_counts()
    assert set(counts) == set(ttcd.EXPORTS)
    for name in ttcd.EXPORTS:
        fn = getattr(ttcd.lib(), name)
        assert len(fn.argtypes) == counts[name], (name, len(fn.argtypes), counts[name])
