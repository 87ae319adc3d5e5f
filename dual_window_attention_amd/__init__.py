"""MI355X (gfx950) implementation of the IP-TTCD layer forward.

``dual_window_attention_amd.ttcd`` is the Python binding of the C ABI in
``include/ttcd.h`` (it loads ``libttcd.so`` and fails if it is missing);
``dual_window_attention_amd.inputs`` holds the seeded synthetic workloads.
"""

__all__ = ["ttcd", "inputs"]
