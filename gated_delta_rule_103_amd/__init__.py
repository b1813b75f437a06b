"""MI355X-native Kimi Delta Attention (KDA): chunked/varlen prefill and decode.

The compute lives in libkda.so (hand-written HIP kernels for gfx950 behind the
C ABI of include/kda.h); ``kda`` is its ctypes binding.
"""
from .kda import (KDAError, gdn_decode, gdn_prefill, kda_decode, kda_output_gate, kda_prefill,  # noqa: F401
                  kda_prefill_noalloc, kda_prefill_snapshots, kda_prefill_workspace_size, load_library)

__all__ = ["kda_prefill", "kda_prefill_noalloc", "kda_prefill_snapshots", "kda_decode", "gdn_prefill", "gdn_decode",
           "kda_output_gate", "kda_prefill_workspace_size", "load_library", "KDAError"]
