"""GPU parity of kda_output_gate (per-head RMS norm, per-channel weight, sigmoid
output gate) against the fp64 oracle, through the C ABI.

Bar: an fp32 out is within 1e-5 x RMS of the oracle (max abs error; the op is
a norm and a logistic in fp32, whose rounding is of order 1e-7); a bf16 out is
bit-exactly the round-to-nearest-even of the fp32 out of the same call, and so
within half a bf16 ulp (2^-9 relative) of it.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_103_amd import inputs, kda_output_gate
from gated_delta_rule_103_amd.kda import KDAError
from kda_testlib import host64, rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-5
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _run(x, out_dtype, eps=1e-6):
    dev = [None if t is None else t.cuda() for t in (x.o, x.gate, x.weight)]
    out = kda_output_gate(*dev, eps=eps, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("Dv", [64, 128])
@pytest.mark.parametrize("o_io,gate_io", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("rows,H,weight", [(1, 1, True), (37, 3, False), (1000, 2, True)])
def test_output_gate_matches_oracle(Dv, o_io, gate_io, rows, H, weight):
    say(f"output_gate Dv={Dv} o={o_io} gate={gate_io} rows={rows} H={H} weight={weight}")
    x = inputs.output_gate(rows, H, Dv, o_io=o_io, gate_io=gate_io, with_weight=weight, seed=rows + Dv)
    ref = oracle.output_gate(host64(x.o), host64(x.gate), None if x.weight is None else host64(x.weight), 1e-6)
    o32 = _run(x, torch.float32)
    assert rel_err(host64(o32), ref) <= TOL
    o16 = _run(x, torch.bfloat16)
    assert torch.equal(o16.cpu(), o32.cpu().to(torch.bfloat16))


@pytest.mark.parametrize("o_std,eps", [(1e-3, 1e-6), (1e-4, 1e-2), (3e4, 1e-6), (1e15, 1e-6)])
def test_output_gate_scales_and_eps(o_std, eps):
    say(f"output_gate o_std={o_std} eps={eps}")
    x = inputs.output_gate(64, 4, 128, o_io="f32", gate_io="f32", o_std=o_std, seed=11)
    ref = oracle.output_gate(host64(x.o), host64(x.gate), host64(x.weight), eps)
    assert rel_err(host64(_run(x, torch.float32, eps)), ref) <= TOL


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_output_gate_in_place(io):
    x = inputs.output_gate(300, 5, 128, o_io=io, gate_io="bf16", seed=3)
    want = _run(x, DT[io])
    o = x.o.cuda()
    got = kda_output_gate(o, x.gate.cuda(), x.weight.cuda(), out=o)
    torch.cuda.synchronize()
    assert got.data_ptr() == o.data_ptr() and torch.equal(got.cpu(), want.cpu())


def test_output_gate_zero_rows_and_errors():
    x = inputs.output_gate(0, 2, 64, seed=1)
    out = _run(x, torch.float32)
    assert out.numel() == 0
    y = inputs.output_gate(4, 2, 64, o_io="bf16", seed=2)
    o = y.o.cuda()
    # in place with a dtype change: the binding refuses the reinterpreted view (its shape
    # differs) before the C ABI, which refuses it too (test_abi_cpu)
    with pytest.raises(ValueError):
        kda_output_gate(o, y.gate.cuda(), out=o.view(torch.float32))
    with pytest.raises(KDAError):                       # eps must be > 0
        kda_output_gate(o, y.gate.cuda(), eps=0.0)
    with pytest.raises(KDAError):                       # Dv outside {64, 128}
        z = inputs.output_gate(4, 2, 96, seed=2)
        _run(z, torch.float32)


def test_output_gate_on_prefill_output_full_size():
    """The 8k single-sequence prefill's o shape (8192 tokens x 32 heads x 128), every row."""
    say("output_gate full size 8192x32x128")
    x = inputs.output_gate(8192, 32, 128, o_io="bf16", gate_io="bf16", o_std=0.3, seed=1001)
    ref = oracle.output_gate(host64(x.o), host64(x.gate), host64(x.weight), 1e-6)
    out = _run(x, torch.float32)
    assert rel_err(host64(out), ref) <= TOL
