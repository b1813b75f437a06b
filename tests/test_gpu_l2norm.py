"""GPU parity of the fused q/k L2 normalisation (qk_l2norm): the kernels take
q and k with arbitrary row norms and normalise them on the fly; the fp64
oracle gets oracle.l2norm(q), oracle.l2norm(k) of the same (rounded) inputs.
Tolerances as for the plain calls.
"""
import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_103_amd import gdn_decode, gdn_prefill, inputs, kda_decode, kda_prefill
from kda_testlib import TOL_BF16, TOL_F32, host64, oracle_decode_step, oracle_prefill, rel_err, to_dev

pytestmark = pytest.mark.gpu
EPS = 1e-6


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _normalised(p):
    """Oracle inputs: q and k replaced by their fp64 L2-normalised rows."""
    qn = torch.from_numpy(oracle.l2norm(host64(p.q), EPS))
    kn = torch.from_numpy(oracle.l2norm(host64(p.k), EPS))
    return replace(p, q=qn, k=kn)


CASES = [
    ("bf16 dense", dict(H=2, D=128, B=2, T=600, C=64, io="bf16", seed=101), False),
    ("bf16 packed with S0", dict(H=3, D=128, lengths=[130, 0, 64, 301], C=64, io="bf16", s0_std=0.02,
                                 seed=102), False),
    ("bf16 per-head gate", dict(H=2, D=128, B=1, T=400, C=64, io="bf16", gate="slow", seed=103), True),
    ("bf16 exact path", dict(H=2, D=128, B=1, T=130, C=64, io="bf16", shift=8.0, seed=104), False),
    ("fp32 D=64 C=16", dict(H=2, D=64, B=1, T=200, C=16, io="f32", seed=105), False),
]


@pytest.mark.parametrize("label,kw,head_gate", CASES, ids=[c[0] for c in CASES])
def test_prefill_qk_l2norm(label, kw, head_gate):
    p = inputs.prefill(qk_scale=(0.25, 4.0), **kw)
    say(f"[l2norm prefill] {label}: {kw}")
    d = to_dev(p)
    if head_gate:
        gh = p.g[..., 0].contiguous()
        out, S = gdn_prefill(d.q, d.k, d.v, gh.cuda(), d.beta, d.S0, cu_seqlens=d.cu_seqlens, C=p.C,
                             out_dtype=torch.float32, qk_l2norm=True, l2norm_eps=EPS)
        ref = replace(_normalised(p), g=gh[..., None].expand_as(p.g).contiguous())
    else:
        out, S = kda_prefill(d.q, d.k, d.v, d.g, d.beta, d.S0, cu_seqlens=d.cu_seqlens, C=p.C,
                             out_dtype=torch.float32, qk_l2norm=True, l2norm_eps=EPS)
        ref = _normalised(p)
    torch.cuda.synchronize()
    ro, rS = oracle_prefill(ref)
    tol = TOL_F32 if kw["io"] == "f32" else TOL_BF16
    eo = rel_err(host64(out).reshape(ro.shape), ro)
    eS = rel_err(host64(S), rS)
    say(f"    err o={eo:.3e} S={eS:.3e}")
    assert eo <= tol["o"] and eS <= tol["S"]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("head_gate", [False, True])
def test_decode_qk_l2norm(D, head_gate):
    N, H, steps = 5, 3, 4
    x = inputs.decode(N, H, D, steps, io="bf16", seed=110 + D, qk_scale=(0.25, 4.0))
    say(f"[l2norm decode] D={D} head_gate={head_gate}")
    S = x.state.cuda()
    Sref = host64(x.state)
    for s in range(steps):
        q, k, v, b = (t[s].cuda().contiguous() for t in (x.q, x.k, x.v, x.beta))
        if head_gate:
            gh = x.g[s][..., 0].contiguous()
            o = gdn_decode(q, k, v, gh.cuda(), b, S, out_dtype=torch.float32, qk_l2norm=True, l2norm_eps=EPS)
            gref = gh[..., None].expand_as(x.g[s])
        else:
            o = kda_decode(q, k, v, x.g[s].cuda().contiguous(), b, S, out_dtype=torch.float32, qk_l2norm=True,
                           l2norm_eps=EPS)
            gref = x.g[s]
        ro, Sref = oracle_decode_step(oracle.l2norm(host64(x.q[s]), EPS), oracle.l2norm(host64(x.k[s]), EPS),
                                      x.v[s], gref, x.beta[s], Sref)
        torch.cuda.synchronize()
        assert rel_err(host64(o), ro) <= 1e-5
    assert rel_err(host64(S), Sref) <= 1e-5


def test_bad_norm_options():
    from gated_delta_rule_103_amd.kda import KDAError
    p = inputs.prefill(2, 128, B=1, T=64, C=64, io="bf16", seed=106)
    d = to_dev(p)
    with pytest.raises(KDAError) as e:
        kda_prefill(d.q, d.k, d.v, d.g, d.beta, qk_l2norm=True, l2norm_eps=0.0)
    assert e.value.status == -1
