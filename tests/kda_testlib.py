"""Shared helpers for the KDA tests: error metric, oracle calls, GPU runs."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# Tolerances, as max|gpu - oracle| / RMS(oracle) over a whole tensor.
TOL_F32 = dict(o=1e-4, S=1e-4)          # fp32 arithmetic path
TOL_BF16 = dict(o=2e-2, S=5e-3)         # bf16 MFMA contractions, fp32 accumulation / state


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.abs(got - ref).max()) if got.size else 0.0
    return float(np.abs(got - ref).max() / rms) if got.size else 0.0


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def to_dev(p, device="cuda"):
    """Copy a PrefillInputs to the GPU (same values)."""
    from dataclasses import replace
    mv = lambda t: None if t is None else t.to(device).contiguous()
    return replace(p, q=mv(p.q), k=mv(p.k), v=mv(p.v), g=mv(p.g), beta=mv(p.beta), S0=mv(p.S0),
                   cu_seqlens=mv(p.cu_seqlens))


def orc_state(S):
    """A state in the library's layout, S [..., Dv, Dk] (value channel x key
    channel), as the oracle takes it, M = S^T [..., Dk, Dv]; the same swap maps
    the oracle's states back. float64 numpy (a torch tensor is upcast); None
    passes through."""
    if S is None:
        return None
    S = host64(S) if hasattr(S, "detach") else np.asarray(S, dtype=np.float64)
    return np.ascontiguousarray(np.swapaxes(S, -1, -2))


def oracle_recurrent(q, k, v, g, beta, S0=None, **kw):
    """oracle.recurrent with its states (S0 in, S_out out) in the library's layout."""
    o, S = oracle.recurrent(q, k, v, g, beta, S0=orc_state(S0), **kw)
    return o, orc_state(S)


def oracle_decode_step(q, k, v, g, beta, S, **kw):
    """oracle.decode_step with the state in the library's layout."""
    o, S_new = oracle.decode_step(q, k, v, g, beta, orc_state(S), **kw)
    return o, orc_state(S_new)


def oracle_prefill(p, chains=None):
    """fp64 oracle on the exact (rounded) inputs of PrefillInputs p.
    Returns (o [T_total, H, Dv], S [N, H, Dv, Dk]) as float64, the state in
    the library's layout."""
    H = p.q.shape[2]
    q, k, v, g = (host64(x).reshape(-1, H, x.shape[-1]) for x in (p.q, p.k, p.v, p.g))
    beta = host64(p.beta).reshape(-1, H)
    if p.cu_seqlens is not None:
        cu = p.cu_seqlens.detach().cpu().numpy().astype(np.int64)
    else:
        B, T = p.q.shape[0], p.q.shape[1]
        cu = np.arange(B + 1, dtype=np.int64) * T
    return oracle_recurrent(q, k, v, g, beta, S0=p.S0, cu_seqlens=cu)


def gpu_prefill(p, out_dtype=None, S_out=True, C=None):
    from gated_delta_rule_103_amd import kda_prefill
    out, S = kda_prefill(p.q, p.k, p.v, p.g, p.beta, p.S0, cu_seqlens=p.cu_seqlens,
                         C=C or p.C, out_dtype=out_dtype, return_state=S_out)
    torch.cuda.synchronize()
    return out, S


def bf16_round(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)
