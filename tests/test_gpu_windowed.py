"""GPU parity of the long-sequence pipeline of kda_prefill.

One sequence of at least 2,048 chunks runs as windows of 512 chunks: the
preparation of the next window on a second stream beside the scan of the
current one, the state passing from window to window through the workspace.
Every token and head is compared with the fp64 oracle (same tolerances as the
other bf16 tests), with a ragged last window, initial states, optional
outputs, slow decay, snapshots whose positions straddle window borders, the packed and
per-head-gate kernel variants, run-to-run determinism, and a HIP-graph
capture (where the pipeline stays on the captured stream) replayed several
times with eager work between the replays.
"""
import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

from gated_delta_rule_103_amd import gdn_prefill, inputs, kda_prefill, kda_prefill_snapshots
from gated_delta_rule_103_amd.kda import kda_prefill_workspace_size
from kda_testlib import TOL_BF16, host64, oracle_prefill, oracle_recurrent, rel_err, to_dev

pytestmark = pytest.mark.gpu

C = 64
# 4 full windows of 512 chunks, then 7 chunks, the last one 37 tokens long
T_LONG = 4 * 512 * C + 6 * C + 37


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from gated_delta_rule_103_amd import load_library
    load_library()


def _errs(o, S, ro, rS):
    H, Dv = o.shape[-2], o.shape[-1]
    eo = rel_err(host64(o).reshape(-1, H, Dv), ro)
    eS = rel_err(host64(S), rS) if S is not None else 0.0
    say(f"    err o={eo:.3e} S={eS:.3e}")
    return eo, eS


def test_windowed_dense_with_initial_state():
    p = inputs.prefill(2, 128, B=1, T=T_LONG, C=C, io="bf16", s0_std=0.05, seed=301)
    say(f"[windowed] dense: T={T_LONG} H=2, S0 given")
    d = to_dev(p)
    o32, S = kda_prefill(d.q, d.k, d.v, d.g, d.beta, d.S0, C=C, out_dtype=torch.float32)
    ob, S2 = kda_prefill(d.q, d.k, d.v, d.g, d.beta, d.S0, C=C)
    torch.cuda.synchronize()
    assert torch.equal(S, S2), "S_out differs between the fp32- and bf16-output runs"
    assert torch.equal(ob, o32.to(torch.bfloat16)), "bf16 output is not RNE of the fp32 output"
    ro, rS = oracle_prefill(p)
    eo, eS = _errs(o32, S, ro, rS)
    assert eo <= TOL_BF16["o"] and eS <= TOL_BF16["S"]


def test_windowed_deterministic_and_optional_outputs():
    """Two runs are bit-identical; without S0 and without S_out the outputs are those
    of the run that returns the state."""
    p = inputs.prefill(2, 128, B=1, T=T_LONG, C=C, io="bf16", seed=302)
    d = to_dev(p)
    o1, S1 = kda_prefill(d.q, d.k, d.v, d.g, d.beta, None, C=C, out_dtype=torch.float32)
    o2, S2 = kda_prefill(d.q, d.k, d.v, d.g, d.beta, None, C=C, out_dtype=torch.float32)
    o3, S3 = kda_prefill(d.q, d.k, d.v, d.g, d.beta, None, C=C, out_dtype=torch.float32, return_state=False)
    torch.cuda.synchronize()
    assert S3 is None
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(o1, o3)
    ro, rS = oracle_prefill(p)
    eo, eS = _errs(o1, S1, ro, rS)
    assert eo <= TOL_BF16["o"] and eS <= TOL_BF16["S"]


def test_windowed_packed_single_sequence():
    """cu_seqlens with one sequence: the packed kernel variant, windowed."""
    p = inputs.prefill(2, 128, lengths=[T_LONG], C=C, io="bf16", s0_std=0.02, seed=303)
    say(f"[windowed] packed: one sequence of {T_LONG} tokens, H=2")
    d = to_dev(p)
    o, S = kda_prefill(d.q, d.k, d.v, d.g, d.beta, d.S0, cu_seqlens=d.cu_seqlens, C=C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rS = oracle_prefill(p)
    eo, eS = _errs(o, S, ro, rS)
    assert eo <= TOL_BF16["o"] and eS <= TOL_BF16["S"]


def test_windowed_per_head_gate():
    """gdn_prefill (one log-decay per token and head), windowed; the oracle takes that
    value in every key channel."""
    p = inputs.prefill(1, 128, B=1, T=T_LONG, C=C, io="bf16", seed=304)
    g_head = p.g[..., 0].contiguous()
    d = to_dev(p)
    o, S = gdn_prefill(d.q, d.k, d.v, g_head.cuda(), d.beta, None, C=C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rS = oracle_prefill(replace(p, g=g_head[..., None].expand_as(p.g).contiguous()))
    eo, eS = _errs(o, S, ro, rS)
    assert eo <= TOL_BF16["o"] and eS <= TOL_BF16["S"]


def test_windowed_slow_decay():
    """Slow decay (alpha ~ 0.97): the state carries across every window border;
    every token and head against the oracle."""
    p = inputs.prefill(2, 128, B=1, T=T_LONG, C=C, io="bf16", gate="slow", s0_std=0.02, seed=308)
    say(f"[windowed] slow decay: T={T_LONG} H=2")
    d = to_dev(p)
    o, S = kda_prefill(d.q, d.k, d.v, d.g, d.beta, d.S0, C=C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rS = oracle_prefill(p)
    eo, eS = _errs(o, S, ro, rS)
    assert eo <= TOL_BF16["o"] and eS <= TOL_BF16["S"]


def test_windowed_many_heads_in_order():
    """32 heads: the scan takes every CU, so the windows run in order on the caller's
    stream (no side stream); every token and head against the oracle."""
    p = inputs.prefill(32, 128, B=1, T=T_LONG, C=C, io="bf16", s0_std=0.02, seed=307)
    say(f"[windowed] in order: T={T_LONG} H=32")
    d = to_dev(p)
    o, S = kda_prefill(d.q, d.k, d.v, d.g, d.beta, d.S0, C=C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rS = oracle_prefill(p)
    eo, eS = _errs(o, S, ro, rS)
    assert eo <= TOL_BF16["o"] and eS <= TOL_BF16["S"]


def test_windowed_snapshots_across_window_borders():
    """Snapshots every 300 chunks: slots 1..6 fall inside windows 0..3 at varying
    offsets; slots 7 and 8 lie past the end and stay untouched."""
    every, max_snaps = 300 * C, 8
    p = inputs.prefill(1, 128, B=1, T=T_LONG, C=C, io="bf16", s0_std=0.02, seed=305)
    d = to_dev(p)
    o_ref, S_ref = kda_prefill(d.q, d.k, d.v, d.g, d.beta, d.S0, C=C, out_dtype=torch.float32)
    o, S, snaps = kda_prefill_snapshots(d.q, d.k, d.v, d.g, d.beta, d.S0, snapshot_every=every,
                                        max_snapshots=max_snaps, C=C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    H = 1
    q, k, v, g = (host64(x).reshape(-1, H, 128) for x in (p.q, p.k, p.v, p.g))
    beta = host64(p.beta).reshape(-1, H)
    sn = host64(snaps)
    state = host64(p.S0)
    for slot in range(max_snaps):
        a, b = slot * every, (slot + 1) * every
        if b > T_LONG:
            assert np.isnan(sn[0, :, slot]).all(), slot
            continue
        _, state = oracle_recurrent(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], S0=state,
                                    cu_seqlens=np.array([0, b - a], dtype=np.int64))
        e = rel_err(sn[0, :, slot], state[0])
        say(f"    slot {slot} (token {b}): err {e:.3e}")
        assert e <= TOL_BF16["S"], (slot, e)


def test_windowed_graph_capture_replays():
    """Captured into a HIP graph (the pipeline then runs on the captured stream alone),
    replayed three times with eager work and synchronisation between the replays:
    every replay equals the eager (two-stream) result bit for bit."""
    p = inputs.prefill(2, 128, B=1, T=T_LONG, C=C, io="bf16", s0_std=0.02, seed=306)
    d = to_dev(p)
    H, N = 2, 1
    ws = torch.empty(kda_prefill_workspace_size(N, T_LONG, H, 128, 128, C, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    o_e, S_e = kda_prefill(d.q, d.k, d.v, d.g, d.beta, d.S0, C=C, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(o_e)
    S_out = torch.empty_like(S_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, capture_error_mode="relaxed"):
        kda_prefill(d.q, d.k, d.v, d.g, d.beta, d.S0, C=C, out=out, S_out=S_out, workspace=ws)
    torch.cuda.synchronize()
    junk = torch.empty(1 << 20, device="cuda")
    for r in range(3):
        out.fill_(float("nan"))
        S_out.fill_(float("nan"))
        junk.normal_()                       # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"    replay {r}: out equal {torch.equal(out, o_e)}, S equal {torch.equal(S_out, S_e)}")
        assert torch.equal(out, o_e) and torch.equal(S_out, S_e), r
