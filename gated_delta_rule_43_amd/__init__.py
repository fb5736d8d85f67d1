"""KDA (Kimi Delta Attention) chunked forward for AMD MI355X (gfx950).

The compute lives in ``libkda.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/kda.h``); ``gated_delta_rule_43_amd.kda`` is the thin
ctypes binding over it.  Importing this package loads nothing; the library is
loaded on first use of the binding.
"""
__all__ = ["kda", "synthetic"]
