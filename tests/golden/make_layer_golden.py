"""Write the stored expected values of the full-size 64K layer parity test.

Runs the fp64 oracle (and nothing else) over the whole Qwen3-0.6B-shaped
layer at 64K context (seeded synthetic inputs, 16/8 heads x 128, d_model
1024, d_ff 3072, w_T 8192, w_S 512, chunk 1024) and keeps a sample of its
outputs: every output of a fixed set of token rows (window edges, chunk
edges, the last token), including the residual terms r and unit keys k of
the chunk lists, and a fixed random sample of the final fast-weight state.
The write coefficients are the workload's beta_i ~ U(0,1).  A fingerprint of the inputs is stored beside them so the test can
tell when the generators changed and this file must be rewritten.

    python tests/golden/make_layer_golden.py      # ~5 min, ~20 GB RAM

The result goes to tests/golden/layer_qwen3_64k_rows.npz (float32 arrays;
fp32 rounding is far below the comparison tolerance, a 1e-2 relative bound
with a 2e-2 absolute floor).
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from dual_window_attention_amd import inputs as I  # noqa: E402
from oracle import ttcd_oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "layer_qwen3_64k_rows.npz")

# token rows: start, student-window edge, chunk edges, teacher-window edge, tail
ROWS = np.array([0, 1, 511, 512, 1023, 1024, 1025, 2047, 8191, 8192, 8193, 16384,
                 30001, 47104, 65534, 65535], dtype=np.int64)
N_STATE = 4096


def fingerprint(tensors):
    """Sum and sum of squares of each input in fp64 (bit-level input changes
    show up here long before they matter to a 2e-2 bound)."""
    out = {}
    for name, arr in tensors.items():
        a = np.asarray(arr, dtype=np.float64).ravel()
        out["fp_" + name] = np.array([a.size, a.sum(), (a * a).sum()], dtype=np.float64)
    return out


def inputs64(cfg):
    att = I.attention_inputs(cfg)
    w = {n: t.f64() for n, t in I.layer_weights(cfg).items()}
    w["beta"] = I.beta_for(cfg).astype(np.float64)
    x = I.residual_input(cfg).f64()
    return att["q"].f64(), att["k"].f64(), att["v"].f64(), x, w


def main():
    cfg = I.CONFIGS[3]
    q, k, v, x, w = inputs64(cfg)
    fp = fingerprint({"q": q, "k": k, "v": v, "x": x, **w})
    t0 = time.time()
    ref = O.layer_forward(q, k, v, x, w, cfg.w_teacher, cfg.w_student, cfg.chunk)
    print(f"oracle layer: {time.time() - t0:.0f} s", flush=True)
    d, f = cfg.d_model, cfg.d_ff
    rng = np.random.default_rng(12345)
    si = rng.integers(0, d, N_STATE)
    sj = rng.integers(0, f, N_STATE)
    store = {
        "rows": ROWS,
        "out": ref["out"][0, ROWS], "y": ref["y"][0, ROWS],
        "o_t": ref["o_t"][0, ROWS], "o_s": ref["o_s"][0, ROWS],
        "lse_t": ref["lse_t"][0][:, ROWS], "lse_s": ref["lse_s"][0][:, ROWS],
        "z_t": ref["z_t"][0, ROWS], "z_s": ref["z_s"][0, ROWS],
        "r": ref["r"][0, ROWS], "k": ref["k"][0, ROWS],
        "state_i": si, "state_j": sj, "state": ref["state"][0, si, sj],
    }
    store = {n: (a.astype(np.float32) if a.dtype == np.float64 else a) for n, a in store.items()}
    store.update(fp)
    np.savez_compressed(OUT, **store)
    print("wrote", OUT, os.path.getsize(OUT), "bytes")


if __name__ == "__main__":
    main()
