"""fp64 CPU oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no
code with the HIP library in ``gated_delta_rule_103_amd`` and imports
nothing from it; the two meet only through the seeded input generators.

Two independent implementations live here:

* ``recurrent``: the per-token recurrence in C (``kda_oracle.c``), threaded
  over the independent (sequence, head) chains. It is the oracle.
* ``chunked_naive.chunked``: the chunked (FlashKDA-style) matrix form in
  numpy, written separately, used only to cross-check the recurrence.

``l2norm`` is the q/k pre-normalisation of the KDA block (explainer, input
processing paragraph: L2 norm on q and k), written out as its definition.
``output_gate`` is the block's output side (same paragraph: per-head
normalisation, then an output forget gate), written out as its definition
under the readings stated in its docstring.

Both follow the Kimi K3 explainer (SemiAnalysis, Chinese translation):
DeltaNet section (delta rule), GDN/KDA paragraph (per-channel diagonal
forget gate) and FlashKDA paragraph (recurrence with D_t and u_t, chunk
unrolling, UT transform). Parity status: pinned, see
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``kda_oracle.c`` into ``libkda_oracle.so`` with the host C compiler."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O3", "-fPIC", "-shared", "-pthread", "-std=c99",
               "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kda_oracle_run.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                       ctypes.POINTER(ctypes.c_int64),
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int]
        lib.kda_oracle_run.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads(chains: int) -> int:
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return max(1, min(cores, 16, chains))


def _f64(x) -> np.ndarray:
    """Exact upcast to a C-contiguous float64 array (accepts torch tensors)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def recurrent(q, k, v, g, beta, S0=None, cu_seqlens: Optional[Sequence[int]] = None,
              nthreads: Optional[int] = None, want_state: bool = True):
    """Run the fp64 per-token recurrence.

    Layouts (packed, one row per token): q, k, g ``[T, H, Dk]``; v ``[T, H, Dv]``;
    beta ``[T, H]``; S0 ``[N, H, Dk, Dv]`` with rows = key channels (the state is
    stored as S^T). A leading batch axis ``[B, T, ...]`` is also accepted when
    ``cu_seqlens`` is None; then every batch row is its own sequence.

    Returns ``(o, S_out)`` as float64 arrays; ``o`` has the input's leading shape.
    """
    q, k, v, g, beta = (_f64(t) for t in (q, k, v, g, beta))
    lead = q.shape[:-2]
    if cu_seqlens is None:
        if q.ndim == 4:
            B, T = q.shape[0], q.shape[1]
            cu = np.arange(B + 1, dtype=np.int64) * T
        else:
            cu = np.array([0, q.shape[0]], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64))
    H, Dk = q.shape[-2], q.shape[-1]
    Dv = v.shape[-1]
    q = q.reshape(-1, H, Dk)
    k = k.reshape(-1, H, Dk)
    g = g.reshape(-1, H, Dk)
    v = v.reshape(-1, H, Dv)
    beta = beta.reshape(-1, H)
    T_total = q.shape[0]
    N = len(cu) - 1
    if cu[-1] != T_total:
        raise ValueError("cu_seqlens[-1] must equal the number of tokens")
    out = np.zeros((T_total, H, Dv), dtype=np.float64)
    S_out = np.zeros((N, H, Dk, Dv), dtype=np.float64) if want_state else None
    s0 = None if S0 is None else _f64(S0).reshape(N, H, Dk, Dv)
    dp = ctypes.POINTER(ctypes.c_double)

    def ptr(a):
        return None if a is None else a.ctypes.data_as(dp)

    nt = nthreads if nthreads is not None else default_threads(N * H)
    rc = _load().kda_oracle_run(ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(s0),
                                ptr(out), ptr(S_out),
                                cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                N, H, Dk, Dv, nt)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_run failed with code {rc}")
    return out.reshape(*lead, H, Dv), S_out


def decode_step(q, k, v, g, beta, S, nthreads: Optional[int] = None):
    """One token per sequence: ``q, k, g [N, H, Dk]``, ``v [N, H, Dv]``,
    ``beta [N, H]``, state ``S [N, H, Dk, Dv]``. Returns ``(o [N, H, Dv], S_new)``."""
    q = _f64(q)
    N = q.shape[0]
    cu = np.arange(N + 1, dtype=np.int64)
    return recurrent(q, k, v, g, beta, S0=S, cu_seqlens=cu, nthreads=nthreads)


def l2norm(x, eps: float):
    """x / sqrt(sum over the last axis of x^2 + eps), in fp64 (the L2 norm the
    explainer's KDA block applies to q and k before the recurrence; eps as the
    library takes it)."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def output_gate(o, gate, weight=None, eps: float = 1e-6):
    """Per-head output norm and output gate of the KDA block, in fp64.

    The explainer's KDA input/output paragraph says the output is normalised
    per head and then controlled by an output forget gate. It names neither
    the norm nor the gate's activation; the reading taken here is an RMS norm
    over the head's Dv channels with eps inside the square root, a
    per-channel weight shared by the heads, and a logistic sigmoid of the
    gate pre-activation:
        out = o / sqrt(mean(o^2) + eps) * weight * 1 / (1 + exp(-gate))
    o, gate: [..., H, Dv]; weight: [Dv] or None (ones)."""
    o, z = _f64(o), _f64(gate)
    w = np.ones(o.shape[-1]) if weight is None else _f64(weight)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o / rms * w / (1.0 + np.exp(-z))
