"""GPU parity of gdn_prefill / gdn_decode: the scalar forget gate of Gated
DeltaNet (one log-decay per token and head) and DeltaNet (no gate), run through
the KDA kernels.

The fp64 oracle takes a per-channel gate; a per-head gate is the same
recurrence with that value in every key channel (alpha_t I = Diag(alpha_t, ...,
alpha_t)), and no gate is g = 0. The per-head gate is taken from channel 0 of
the generated per-channel gate, so the inputs come from the shared generator.
Tolerances as for kda_prefill / kda_decode.
"""
import sys
from dataclasses import replace

import pytest
import torch

from gated_delta_rule_103_amd import gdn_decode, gdn_prefill, inputs
from kda_testlib import TOL_BF16, TOL_F32, host64, oracle_decode_step, oracle_prefill, rel_err, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _oracle_inputs(p, g_head):
    """p with its per-channel gate replaced by g_head broadcast (or zeros)."""
    g = torch.zeros_like(p.g) if g_head is None else g_head[..., None].expand_as(p.g).contiguous()
    return replace(p, g=g)


PREFILL_CASES = [
    ("bf16 dense, per-head gate", dict(H=2, D=128, B=2, T=700, C=64, io="bf16", seed=81), True),
    ("bf16 packed, S0, slow per-head gate", dict(H=3, D=128, lengths=[0, 70, 513, 200], C=64, io="bf16",
                                                  s0_std=0.02, gate="slow", seed=82), True),
    ("bf16 per-head gate below FLT_MIN per block (exact path)", dict(H=2, D=128, B=1, T=200, C=64,
                                                                     io="bf16", shift=8.0, seed=83), True),
    ("bf16 DeltaNet (no gate)", dict(H=2, D=128, B=1, T=300, C=64, io="bf16", seed=84), False),
    ("fp32 D=64 C=16, per-head gate", dict(H=2, D=64, B=1, T=250, C=16, io="f32", seed=85), True),
    ("fp32 packed DeltaNet", dict(H=2, D=64, lengths=[33, 0, 97], C=16, io="f32", s0_std=0.02, seed=86), False),
]


@pytest.mark.parametrize("label,kw,gated", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_gdn_prefill(label, kw, gated):
    p = inputs.prefill(**kw)
    say(f"[gdn prefill] {label}: {kw}")
    g_head = p.g[..., 0].contiguous() if gated else None
    d = to_dev(p)
    out, S = gdn_prefill(d.q, d.k, d.v, None if g_head is None else g_head.cuda(), d.beta, d.S0,
                         cu_seqlens=d.cu_seqlens, C=p.C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rS = oracle_prefill(_oracle_inputs(p, g_head))
    tol = TOL_F32 if kw["io"] == "f32" else TOL_BF16
    eo = rel_err(host64(out).reshape(ro.shape), ro)
    eS = rel_err(host64(S), rS)
    say(f"    err o={eo:.3e} S={eS:.3e}")
    assert eo <= tol["o"] and eS <= tol["S"]


def test_gdn_prefill_matches_kda_prefill_with_uniform_gate():
    """A per-channel gate equal across channels gives the same result through
    kda_prefill, up to the order of rounding."""
    from gated_delta_rule_103_amd import kda_prefill
    p = inputs.prefill(2, 128, B=1, T=320, C=64, io="bf16", seed=87)
    g_head = p.g[..., 0].contiguous()
    d = to_dev(_oracle_inputs(p, g_head))
    o1, S1 = kda_prefill(d.q, d.k, d.v, d.g, d.beta, cu_seqlens=None, C=64, out_dtype=torch.float32)
    o2, S2 = gdn_prefill(d.q, d.k, d.v, g_head.cuda(), d.beta, cu_seqlens=None, C=64, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("gated", [True, False])
def test_gdn_decode(D, gated):
    N, H, steps = 5, 3, 4
    x = inputs.decode(N, H, D, steps, io="bf16", seed=90 + D + int(gated))
    say(f"[gdn decode] D={D} gated={gated}")
    S = x.state.cuda()
    Sref = host64(x.state)
    for s in range(steps):
        gh = x.g[s][..., 0].contiguous() if gated else None
        args = [t[s].cuda().contiguous() for t in (x.q, x.k, x.v)]
        o = gdn_decode(*args, None if gh is None else gh.cuda(), x.beta[s].cuda().contiguous(), S,
                       out_dtype=torch.float32)
        gref = torch.zeros_like(x.g[s]) if gh is None else gh[..., None].expand_as(x.g[s])
        ro, Sref = oracle_decode_step(x.q[s], x.k[s], x.v[s], gref, x.beta[s], Sref)
        torch.cuda.synchronize()
        assert rel_err(host64(o), ro) <= 1e-5
    assert rel_err(host64(S), Sref) <= 1e-5
