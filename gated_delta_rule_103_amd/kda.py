"""Thin Python binding of libkda (ctypes): argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
declared in ``include/kda.h``; this module turns torch tensors into device
pointers, sizes and dtype codes, and raises on a non-zero status. PyTorch is
used for device memory and streams only. There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
_DT = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}
_STATUS = {0: "KDA_OK", -1: "KDA_ERR_INVALID_ARG", -2: "KDA_ERR_UNSUPPORTED",
           -3: "KDA_ERR_WORKSPACE", -4: "KDA_ERR_HIP"}

_lib = None


class KDAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed: {_STATUS.get(status, status)} ({status})")
        self.status = status


class Options(ctypes.Structure):
    """kda_options of include/kda.h."""
    _fields_ = [("gate", ctypes.c_int), ("qk_l2norm", ctypes.c_int), ("l2norm_eps", ctypes.c_float),
                ("snapshot_every", ctypes.c_int), ("max_snapshots", ctypes.c_int),
                ("snapshots", ctypes.c_void_p)]


GATE_CHANNEL, GATE_HEAD = 0, 1


def load_library() -> ctypes.CDLL:
    """Load libkda.so from the package directory (built by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(hipcc, gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.kda_version.restype = i
    lib.kda_version.argtypes = []
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [i]
    lib.kda_prefill_workspace_size.restype = sz
    lib.kda_prefill_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.kda_prefill.restype = i
    lib.kda_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                i, i, i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.kda_prefill_noalloc.restype = i
    lib.kda_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        i, i, i, i, i, i, i, i, i, i, vp]
    lib.kda_prefill_snapshots.restype = i
    lib.kda_prefill_snapshots.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          i, i, i, i, i, i, i, i, i, i, i, i, vp, vp, sz, vp]
    lib.kda_decode.restype = i
    lib.kda_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
    lib.gdn_prefill.restype = i
    lib.gdn_prefill.argtypes = lib.kda_prefill.argtypes
    lib.gdn_decode.restype = i
    lib.gdn_decode.argtypes = lib.kda_decode.argtypes
    op = ctypes.POINTER(Options)
    lib.kda_prefill_ex.restype = i
    lib.kda_prefill_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   i, i, i, i, i, i, i, i, i, i, op, vp, sz, vp]
    lib.kda_decode_ex.restype = i
    lib.kda_decode_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, op, vp]
    lib.kda_output_gate.restype = i
    lib.kda_output_gate.argtypes = [vp, vp, vp, vp, i, i, i, ctypes.c_float, i, i, i, vp]
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libkda must be contiguous")
    return t.data_ptr()


def _stream(stream, device) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


_FLOAT_IO = (torch.float32, torch.bfloat16)


def _expect(t, name, shape, dtypes, optional=False):
    """Raise ValueError unless tensor ``t`` has exactly ``shape`` and a dtype in ``dtypes``."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {[str(d) for d in dtypes]}, got {t.dtype}")


def _same_gpu(**tensors) -> torch.device:
    """Every given tensor is a contiguous GPU tensor on one device; returns that device.
    Checked after shapes and dtypes, so that those errors are reported on any device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (libkda reads device memory), got {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, other tensors on {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return dev


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def kda_prefill_workspace_size(N: int, T_total: int, H: int, Dk: int, Dv: int, C: int,
                               io_dtype: torch.dtype) -> int:
    return int(load_library().kda_prefill_workspace_size(N, T_total, H, Dk, Dv, C, _DT[io_dtype]))


def _check_prefill(q, k, v, g, beta, S0, out, S_out, cu_seqlens, workspace, g_head, snapshots=None,
                   max_snapshots=0):
    """Shapes, dtypes and devices of a prefill call, checked before the library sees a pointer
    (the C ABI receives raw pointers and cannot tell an int64 cu_seqlens from an int32 one)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B, T, H, Dk]")
    B, T, H, Dk = q.shape
    _expect(q, "q", (B, T, H, Dk), _FLOAT_IO)
    _expect(k, "k", (B, T, H, Dk), (q.dtype,))
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("v must be a 4-D tensor [B, T, H, Dv]")
    Dv = v.shape[-1]
    _expect(v, "v", (B, T, H, Dv), (q.dtype,))
    if g_head:
        _expect(g, "g", (B, T, H), (torch.float32,), optional=True)
    else:
        _expect(g, "g", (B, T, H, Dk), (torch.float32,))
    _expect(beta, "beta", (B, T, H), _FLOAT_IO)
    if cu_seqlens is not None:
        if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be a 1-D tensor of N + 1 >= 2 offsets")
        if cu_seqlens.dtype != torch.int32:
            raise ValueError(f"cu_seqlens must be int32, got {cu_seqlens.dtype}")
        if B != 1:
            raise ValueError("packed sequences (cu_seqlens) need B == 1")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    _expect(S0, "S0", (N, H, Dv, Dk), (torch.float32,), optional=True)
    _expect(out, "out", (B, T, H, Dv), _FLOAT_IO, optional=True)
    _expect(S_out, "S_out", (N, H, Dv, Dk), (torch.float32,), optional=True)
    if snapshots is not None:
        _expect(snapshots, "snapshots", (N, H, max_snapshots, Dv, Dk), (torch.float32,))
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or workspace.dim() != 1 or
                                  workspace.dtype != torch.uint8):
        raise ValueError("workspace must be a 1-D uint8 tensor")
    return _same_gpu(q=q, k=k, v=v, g=g, beta=beta, S0=S0, out=out, S_out=S_out, cu_seqlens=cu_seqlens,
                     snapshots=snapshots, workspace=workspace)


def _prefill_buffers(lib, q, v, beta, cu_seqlens, C, out, S_out, out_dtype, workspace, return_state):
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if out is None:
        out = torch.empty(B, T, H, Dv, dtype=out_dtype or q.dtype, device=q.device)
    if S_out is None and return_state:
        S_out = torch.empty(N, H, Dv, Dk, dtype=torch.float32, device=q.device)
    need = int(lib.kda_prefill_workspace_size(N, B * T, H, Dk, Dv, C, _dt(q)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (B, T, H, Dk, Dv, N), out, S_out, workspace, ws_bytes


def _prefill(entry, q, k, v, g, beta, S0, out, S_out, cu_seqlens, C, out_dtype, workspace, stream,
             return_state, qk_l2norm=False, l2norm_eps=1e-6):
    lib = load_library()
    dev = _check_prefill(q, k, v, g, beta, S0, out, S_out, cu_seqlens, workspace, entry == "gdn_prefill")
    with torch.cuda.device(dev):
        (B, T, H, Dk, Dv, N), out, S_out, workspace, ws_bytes = _prefill_buffers(
            lib, q, v, beta, cu_seqlens, C, out, S_out, out_dtype, workspace, return_state)
        args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_out),
                _ptr(cu_seqlens), N, B, T, H, Dk, Dv, C, _dt(q), _dt(beta), _dt(out))
        if qk_l2norm:
            opt = Options(gate=GATE_HEAD if entry == "gdn_prefill" else GATE_CHANNEL, qk_l2norm=1,
                          l2norm_eps=l2norm_eps)
            entry = "kda_prefill_ex"
            st = lib.kda_prefill_ex(*args, ctypes.byref(opt), _ptr(workspace), ws_bytes, _stream(stream, dev))
        else:
            st = getattr(lib, entry)(*args, _ptr(workspace), ws_bytes, _stream(stream, dev))
    if st != 0:
        raise KDAError(st, entry)
    return out, S_out


def kda_prefill(q, k, v, g, beta, S0=None, *, out=None, S_out=None, cu_seqlens=None, C: int = 64,
                out_dtype: Optional[torch.dtype] = None, workspace=None, stream=None,
                return_state: bool = True, qk_l2norm: bool = False, l2norm_eps: float = 1e-6):
    """Chunked KDA prefill. q, k, g: [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H];
    S0: [N, H, Dv, Dk] fp32 (the state S, row = value channel) or None; cu_seqlens: int32 [N+1] device tensor (B == 1) or None.
    qk_l2norm: L2-normalise q and k over Dk inside the kernels (x / sqrt(sum x^2 + eps)).
    Returns (out [B, T, H, Dv], S_out [N, H, Dv, Dk] or None)."""
    return _prefill("kda_prefill", q, k, v, g, beta, S0, out, S_out, cu_seqlens, C, out_dtype, workspace,
                    stream, return_state, qk_l2norm, l2norm_eps)


def kda_prefill_noalloc(q, k, v, g, beta, S0=None, *, out=None, S_out=None, cu_seqlens=None, C: int = 64,
                        out_dtype: Optional[torch.dtype] = None, stream=None, return_state: bool = True):
    """kda_prefill with the library's fixed per-device workspace (no allocation inside the
    call; ``out`` and ``S_out`` are allocated here only when not given). Sizes whose
    workspace exceeds the fixed array raise KDAError(KDA_ERR_WORKSPACE). Calls that
    overlap in time on one GPU share that array and race."""
    lib = load_library()
    dev = _check_prefill(q, k, v, g, beta, S0, out, S_out, cu_seqlens, None, False)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if out is None:
        out = torch.empty(B, T, H, Dv, dtype=out_dtype or q.dtype, device=q.device)
    if S_out is None and return_state:
        S_out = torch.empty(N, H, Dv, Dk, dtype=torch.float32, device=q.device)
    with torch.cuda.device(dev):
        st = lib.kda_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(out),
                                     _ptr(S_out), _ptr(cu_seqlens), N, B, T, H, Dk, Dv, C, _dt(q), _dt(beta),
                                     _dt(out), _stream(stream, dev))
    if st != 0:
        raise KDAError(st, "kda_prefill_noalloc")
    return out, S_out


def gdn_prefill(q, k, v, g, beta, S0=None, *, out=None, S_out=None, cu_seqlens=None, C: int = 64,
                out_dtype: Optional[torch.dtype] = None, workspace=None, stream=None,
                return_state: bool = True, qk_l2norm: bool = False, l2norm_eps: float = 1e-6):
    """Chunked prefill with the scalar gate of Gated DeltaNet: g [B, T, H] fp32 (one
    log-decay per token and head), or None for DeltaNet (no decay). Otherwise as
    kda_prefill."""
    return _prefill("gdn_prefill", q, k, v, g, beta, S0, out, S_out, cu_seqlens, C, out_dtype, workspace,
                    stream, return_state, qk_l2norm, l2norm_eps)


def kda_prefill_snapshots(q, k, v, g, beta, S0=None, *, snapshot_every: int, max_snapshots: int,
                          snapshots=None, out=None, S_out=None, cu_seqlens=None, C: int = 64,
                          out_dtype: Optional[torch.dtype] = None, workspace=None, stream=None,
                          return_state: bool = True):
    """kda_prefill that also writes the state after every ``snapshot_every`` tokens of
    each sequence into ``snapshots`` [N, H, max_snapshots, Dv, Dk] fp32 (slots past a
    sequence's end are not written). Returns (out, S_out, snapshots)."""
    lib = load_library()
    if snapshots is None:
        if not isinstance(q, torch.Tensor) or q.dim() != 4 or not isinstance(v, torch.Tensor) or v.dim() != 4:
            raise ValueError("q must be [B, T, H, Dk] and v [B, T, H, Dv]")
        N = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
        snapshots = torch.full((N, q.shape[2], max_snapshots, v.shape[3], q.shape[3]), float("nan"),
                               dtype=torch.float32, device=q.device)
    dev = _check_prefill(q, k, v, g, beta, S0, out, S_out, cu_seqlens, workspace, False, snapshots,
                         max_snapshots)
    with torch.cuda.device(dev):
        (B, T, H, Dk, Dv, N), out, S_out, workspace, ws_bytes = _prefill_buffers(
            lib, q, v, beta, cu_seqlens, C, out, S_out, out_dtype, workspace, return_state)
        st = lib.kda_prefill_snapshots(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(out),
                                       _ptr(S_out), _ptr(cu_seqlens), N, B, T, H, Dk, Dv, C, _dt(q),
                                       _dt(beta), _dt(out), snapshot_every, max_snapshots, _ptr(snapshots),
                                       _ptr(workspace), ws_bytes, _stream(stream, dev))
    if st != 0:
        raise KDAError(st, "kda_prefill_snapshots")
    return out, S_out, snapshots


def _decode(entry, q, k, v, g, beta, S, out, out_dtype, stream, qk_l2norm=False, l2norm_eps=1e-6):
    lib = load_library()
    if not isinstance(q, torch.Tensor) or q.dim() != 3 or not isinstance(v, torch.Tensor) or v.dim() != 3:
        raise ValueError("q must be [N, H, Dk] and v [N, H, Dv]")
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    _expect(q, "q", (N, H, Dk), _FLOAT_IO)
    _expect(k, "k", (N, H, Dk), (q.dtype,))
    _expect(v, "v", (N, H, Dv), (q.dtype,))
    if entry == "gdn_decode":
        _expect(g, "g", (N, H), (torch.float32,), optional=True)
    else:
        _expect(g, "g", (N, H, Dk), (torch.float32,))
    _expect(beta, "beta", (N, H), _FLOAT_IO)
    _expect(S, "S", (N, H, Dv, Dk), (torch.float32,))
    _expect(out, "out", (N, H, Dv), _FLOAT_IO, optional=True)
    dev = _same_gpu(q=q, k=k, v=v, g=g, beta=beta, S=S, out=out)
    if out is None:
        out = torch.empty(N, H, Dv, dtype=out_dtype or q.dtype, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(out), N, H, Dk, Dv, _dt(q),
            _dt(beta), _dt(out))
    with torch.cuda.device(dev):
        if qk_l2norm:
            opt = Options(gate=GATE_HEAD if entry == "gdn_decode" else GATE_CHANNEL, qk_l2norm=1,
                          l2norm_eps=l2norm_eps)
            entry = "kda_decode_ex"
            st = lib.kda_decode_ex(*args, ctypes.byref(opt), _stream(stream, dev))
        else:
            st = getattr(lib, entry)(*args, _stream(stream, dev))
    if st != 0:
        raise KDAError(st, entry)
    return out


def kda_decode(q, k, v, g, beta, S, *, out=None, out_dtype: Optional[torch.dtype] = None,
               stream=None, qk_l2norm: bool = False, l2norm_eps: float = 1e-6):
    """One decode step, state S [N, H, Dv, Dk] fp32 (row = value channel) updated in place.
    q, k, g: [N, H, Dk]; v: [N, H, Dv]; beta: [N, H]. Returns out [N, H, Dv]."""
    return _decode("kda_decode", q, k, v, g, beta, S, out, out_dtype, stream, qk_l2norm, l2norm_eps)


def gdn_decode(q, k, v, g, beta, S, *, out=None, out_dtype: Optional[torch.dtype] = None,
               stream=None, qk_l2norm: bool = False, l2norm_eps: float = 1e-6):
    """kda_decode with the scalar gate of Gated DeltaNet: g [N, H] fp32, or None
    for DeltaNet (no decay)."""
    return _decode("gdn_decode", q, k, v, g, beta, S, out, out_dtype, stream, qk_l2norm, l2norm_eps)


def kda_output_gate(o, gate, weight=None, *, eps: float = 1e-6, out=None,
                    out_dtype: Optional[torch.dtype] = None, stream=None):
    """Per-head RMS norm of o with a per-channel weight and a sigmoid output gate:
    out = o / sqrt(mean(o^2 over Dv) + eps) * weight * sigmoid(gate).
    o, gate: [..., H, Dv] (same shape); weight: [Dv] fp32 or None (ones).
    ``out`` may be ``o`` itself when the dtypes match. Returns out."""
    lib = load_library()
    if not isinstance(o, torch.Tensor) or o.dim() < 2:
        raise ValueError("o must be a tensor [..., H, Dv]")
    _expect(o, "o", o.shape, _FLOAT_IO)
    _expect(gate, "gate", o.shape, _FLOAT_IO)
    H, Dv = o.shape[-2], o.shape[-1]
    rows = o.numel() // (H * Dv) if o.numel() else 0
    _expect(weight, "weight", (Dv,), (torch.float32,), optional=True)
    _expect(out, "out", o.shape, _FLOAT_IO, optional=True)
    dev = _same_gpu(o=o, gate=gate, weight=weight, out=out)
    if out is None:
        out = torch.empty(o.shape, dtype=out_dtype or o.dtype, device=o.device)
    with torch.cuda.device(dev):
        st = lib.kda_output_gate(_ptr(o), _ptr(gate), _ptr(weight), _ptr(out), rows, H, Dv, float(eps),
                                 _dt(o), _dt(gate), _dt(out), _stream(stream, dev))
    if st != 0:
        raise KDAError(st, "kda_output_gate")
    return out
