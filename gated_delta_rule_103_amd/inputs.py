"""Seeded synthetic inputs for KDA prefill and decode.

This module holds no part of the method's arithmetic: it only draws random
tensors with the shapes, dtypes and distributions of the workloads below.
Both the HIP path and the fp64 oracle are fed from it (the oracle receives
exact fp64 upcasts of the rounded tensors).

Recipe (all five workloads):
  q, k ~ N(0, 1), L2-normalised over the head dimension in fp32, then
       rounded to the I/O dtype (the kernels never normalise: inputs arrive
       normalised, as the KDA layer's pre-processing leaves them);
  v    ~ N(0, 1) in the I/O dtype;
  g    = -softplus(N(0, 1) + shift), fp32, one natural-log decay per
       (token, head, key channel); alpha = exp(g) lies in (0, 1);
  beta = sigmoid(N(0, 1)) in the beta dtype;
  S0 / decode state ~ N(0, std^2) fp32 where the workload has one.
Draw order per generator: lengths (varlen only), q, k, v, g-noise,
beta-noise, S0, then per-step decode tensors.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch
import torch.nn.functional as F

# The five workloads (sizes and distributions as specified for the KDA hot path).
WORKLOADS: Dict[str, dict] = {
    "tiny_f32": dict(kind="prefill", B=1, H=2, T=256, D=64, C=16, io="f32",
                     shift=2.0, s0_std=None, seed=1000),
    "single_seq_8k": dict(kind="prefill", B=1, H=32, T=8192, D=128, C=64, io="bf16",
                          shift=2.0, s0_std=None, seed=1001),
    "varlen_16x": dict(kind="prefill", N=16, len_lo=512, len_hi=16384, H=32, D=128, C=64,
                       io="bf16", shift=2.0, s0_std=0.02, seed=1002),
    "decode_512x32": dict(kind="decode", N=512, H=32, D=128, steps=64, io="bf16",
                          shift=2.0, state_std=0.02, seed=1003),
    "long_1m": dict(kind="prefill", B=1, H=16, T=1048576, D=128, C=64, io="bf16",
                    shift=4.0, s0_std=None, seed=1004),
    # ungraded stress companion of long_1m: the same shape with slow decay,
    # g = -softplus(N(0,1) - 4) (alpha ~ 0.97), so the state carries far
    "long_1m_slow": dict(kind="prefill", B=1, H=16, T=1048576, D=128, C=64, io="bf16",
                         shift=-4.0, s0_std=None, seed=1005),
}
WORKLOAD_ORDER: List[str] = ["tiny_f32", "single_seq_8k", "varlen_16x", "decode_512x32", "long_1m"]

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


@dataclass
class PrefillInputs:
    q: torch.Tensor            # [B, T, H, Dk] io dtype
    k: torch.Tensor            # [B, T, H, Dk] io dtype
    v: torch.Tensor            # [B, T, H, Dv] io dtype
    g: torch.Tensor            # [B, T, H, Dk] fp32
    beta: torch.Tensor         # [B, T, H]     beta dtype
    S0: Optional[torch.Tensor]  # [N, H, Dv, Dk] fp32 (the state S, row = value channel) or None
    cu_seqlens: Optional[torch.Tensor]  # int32 [N+1] (B == 1) or None
    C: int
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return self.q.shape[0] if self.cu_seqlens is None else self.cu_seqlens.numel() - 1

    @property
    def num_tokens(self) -> int:
        return self.q.shape[0] * self.q.shape[1]


def prefill(H: int, D: int, *, B: int = 1, T: Optional[int] = None,
            lengths: Optional[List[int]] = None, C: int = 64, io: str = "bf16",
            beta_io: Optional[str] = None, shift: float = 2.0, gate: str = "softplus",
            s0_std: Optional[float] = None, seed: int = 0, device="cpu",
            v_zero: bool = False, beta_one: bool = False, Dv: Optional[int] = None,
            qk_scale: Optional[tuple] = None) -> PrefillInputs:
    """Draw one prefill problem.

    Either dense ``(B, T)`` or packed ``lengths`` (then B = 1 and cu_seqlens is
    returned). ``gate``: "softplus" -> g = -softplus(N + shift); "zero" -> g = 0
    (alpha = 1); "slow" -> g = -softplus(N - 4) (alpha ~ 0.97).
    ``qk_scale=(lo, hi)``: q and k rows are multiplied by factors drawn from
    U[lo, hi] before rounding (inputs for the fused L2 normalisation; drawn
    last, so the other tensors are those of the same seed without it).
    """
    dev = torch.device(device)
    gen = _gen(seed, dev)
    Dk, Dv = D, (Dv or D)
    cu = None
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        B, T = 1, sum(lengths)
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
        cu = cu.to(dev)
    assert T is not None
    dt = _DT[io]
    bdt = _DT[beta_io or io]
    rn = lambda *s: torch.randn(*s, generator=gen, device=dev, dtype=torch.float32)
    q = _unit(rn(B, T, H, Dk)).to(dt)
    k = _unit(rn(B, T, H, Dk)).to(dt)
    v = rn(B, T, H, Dv).to(dt)
    gn = rn(B, T, H, Dk)
    if gate == "softplus":
        g = -F.softplus(gn + shift)
    elif gate == "slow":
        g = -F.softplus(gn - 4.0)
    elif gate == "zero":
        g = torch.zeros_like(gn)
    else:
        raise ValueError(gate)
    beta = torch.sigmoid(rn(B, T, H)).to(bdt)
    N = B if cu is None else cu.numel() - 1
    S0 = None if s0_std is None else (rn(N, H, Dv, Dk) * s0_std)
    if v_zero:
        v = torch.zeros_like(v)
    if beta_one:
        beta = torch.ones_like(beta)
    if qk_scale is not None:
        lo, hi = qk_scale
        u = lambda: lo + (hi - lo) * torch.rand(B, T, H, 1, generator=gen, device=dev, dtype=torch.float32)
        q = (q.float() * u()).to(dt)
        k = (k.float() * u()).to(dt)
    return PrefillInputs(q, k, v, g.contiguous(), beta, S0, cu, C,
                         meta=dict(H=H, Dk=Dk, Dv=Dv, B=B, T=T, io=io, seed=seed,
                                   gate=gate, shift=shift, lengths=lengths))


def varlen_lengths(n: int, lo: int, hi: int, seed: int) -> List[int]:
    """n lengths drawn uniformly from the inclusive range [lo, hi] (CPU generator)."""
    gen = _gen(seed, "cpu")
    return torch.randint(lo, hi + 1, (n,), generator=gen).tolist()


def workload_prefill(name: str, device="cpu") -> PrefillInputs:
    w = WORKLOADS[name]
    assert w["kind"] == "prefill"
    if "N" in w:
        lengths = varlen_lengths(w["N"], w["len_lo"], w["len_hi"], w["seed"])
        return prefill(w["H"], w["D"], lengths=lengths, C=w["C"], io=w["io"],
                       shift=w["shift"], s0_std=w["s0_std"], seed=w["seed"],
                       device=device)
    return prefill(w["H"], w["D"], B=w["B"], T=w["T"], C=w["C"], io=w["io"],
                   shift=w["shift"], s0_std=w["s0_std"], seed=w["seed"], device=device)


@dataclass
class DecodeInputs:
    q: torch.Tensor     # [steps, N, H, Dk] io dtype
    k: torch.Tensor     # [steps, N, H, Dk]
    v: torch.Tensor     # [steps, N, H, Dv]
    g: torch.Tensor     # [steps, N, H, Dk] fp32
    beta: torch.Tensor  # [steps, N, H]
    state: torch.Tensor  # [N, H, Dv, Dk] fp32 (initial; the kernel updates a copy in place)


def decode(N: int, H: int, D: int, steps: int, *, io: str = "bf16", shift: float = 2.0,
           gate: str = "softplus", state_std: float = 0.02, seed: int = 0,
           device="cpu", qk_scale: Optional[tuple] = None) -> DecodeInputs:
    dev = torch.device(device)
    gen = _gen(seed, dev)
    dt = _DT[io]
    rn = lambda *s: torch.randn(*s, generator=gen, device=dev, dtype=torch.float32)
    state = rn(N, H, D, D) * state_std
    q = _unit(rn(steps, N, H, D)).to(dt)
    k = _unit(rn(steps, N, H, D)).to(dt)
    v = rn(steps, N, H, D).to(dt)
    gn = rn(steps, N, H, D)
    if gate == "softplus":
        g = -F.softplus(gn + shift)
    elif gate == "slow":
        g = -F.softplus(gn - 4.0)
    elif gate == "zero":
        g = torch.zeros_like(gn)
    else:
        raise ValueError(gate)
    beta = torch.sigmoid(rn(steps, N, H)).to(dt)
    if qk_scale is not None:                 # as in prefill(): drawn last
        lo, hi = qk_scale
        u = lambda: lo + (hi - lo) * torch.rand(steps, N, H, 1, generator=gen, device=dev, dtype=torch.float32)
        q = (q.float() * u()).to(dt)
        k = (k.float() * u()).to(dt)
    return DecodeInputs(q, k, v, g.contiguous(), beta, state)


def workload_decode(name: str = "decode_512x32", device="cpu") -> DecodeInputs:
    w = WORKLOADS[name]
    return decode(w["N"], w["H"], w["D"], w["steps"], io=w["io"], shift=w["shift"],
                  state_std=w["state_std"], seed=w["seed"], device=device)


@dataclass
class OutputGateInputs:
    o: torch.Tensor            # [rows, H, Dv] o dtype
    gate: torch.Tensor         # [rows, H, Dv] gate dtype (pre-activation)
    weight: Optional[torch.Tensor]   # [Dv] fp32 or None


def output_gate(rows: int, H: int, Dv: int, *, o_io: str = "bf16", gate_io: str = "bf16",
                o_std: float = 1.0, with_weight: bool = True, seed: int = 0,
                device="cpu") -> OutputGateInputs:
    """Inputs of the output norm and gate: o ~ N(0, o_std^2) (an attention output),
    gate pre-activation ~ N(0, 2^2), weight ~ N(1, 0.1^2) fp32. Draw order: o, gate,
    weight."""
    gen = _gen(seed, device)
    o = (torch.randn(rows, H, Dv, generator=gen, device=device) * o_std).to(_DT[o_io])
    gate = (torch.randn(rows, H, Dv, generator=gen, device=device) * 2.0).to(_DT[gate_io])
    w = 1.0 + 0.1 * torch.randn(Dv, generator=gen, device=device)
    return OutputGateInputs(o=o, gate=gate, weight=w if with_weight else None)
