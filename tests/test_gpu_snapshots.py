"""GPU parity of kda_prefill_snapshots (prefix-cache state snapshots).

Slot k-1 of sequence n must hold the state after its first k * every tokens,
i.e. the oracle's final state for that prefix (same tolerances as S_out);
slots past the sequence end or past the capacity must stay untouched (the
binding fills them with NaN), and out / S_out must be bit-identical to a
plain kda_prefill of the same inputs.
"""
import sys

import numpy as np
import pytest
import torch

from gated_delta_rule_103_amd import inputs, kda_prefill, kda_prefill_snapshots
from kda_testlib import TOL_BF16, TOL_F32, host64, oracle_recurrent, rel_err, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _host(p):
    H = p.q.shape[2]
    q, k, v, g = (host64(x).reshape(-1, H, x.shape[-1]) for x in (p.q, p.k, p.v, p.g))
    beta = host64(p.beta).reshape(-1, H)
    if p.cu_seqlens is not None:
        cu = p.cu_seqlens.detach().cpu().numpy().astype(np.int64)
    else:
        B, T = p.q.shape[0], p.q.shape[1]
        cu = np.arange(B + 1, dtype=np.int64) * T
    s0 = None if p.S0 is None else host64(p.S0)
    return q, k, v, g, beta, s0, cu


def _check(p, every, max_snaps, tol, label):
    say(f"[snapshots] {label}: every={every} max={max_snaps}")
    d = to_dev(p)
    o_ref, S_ref = kda_prefill(d.q, d.k, d.v, d.g, d.beta, d.S0, cu_seqlens=d.cu_seqlens, C=p.C,
                               out_dtype=torch.float32)
    o, S, snaps = kda_prefill_snapshots(d.q, d.k, d.v, d.g, d.beta, d.S0, snapshot_every=every,
                                        max_snapshots=max_snaps, cu_seqlens=d.cu_seqlens, C=p.C,
                                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    q, k, v, g, beta, s0, cu = _host(p)
    sn = host64(snaps)
    N = len(cu) - 1
    written = 0
    for n in range(N):
        length = int(cu[n + 1] - cu[n])
        for slot in range(max_snaps):
            t = (slot + 1) * every
            if t > length:
                assert np.isnan(sn[n, :, slot]).all(), (n, slot)
                continue
            a, b = int(cu[n]), int(cu[n]) + t
            _, ref = oracle_recurrent(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b],
                                      S0=None if s0 is None else s0[n:n + 1])
            e = rel_err(sn[n, :, slot], ref[0])
            assert e <= tol["S"], (n, slot, e)
            written += 1
    say(f"    {written} snapshots checked")
    assert written > 0


def test_snapshots_dense_bf16_mfma():
    p = inputs.prefill(2, 128, B=2, T=700, C=64, io="bf16", seed=71)
    _check(p, 128, 4, TOL_BF16, "dense bf16, capacity below the sequence")
    _check(p, 192, 8, TOL_BF16, "dense bf16, slots past the end")


def test_snapshots_varlen_bf16_mfma_with_state():
    p = inputs.prefill(2, 128, lengths=[0, 64, 200, 513], C=64, io="bf16", s0_std=0.02,
                       gate="slow", seed=72)
    _check(p, 64, 10, TOL_BF16, "varlen bf16 with S0, slow decay")


def test_snapshots_many_chains_wide_scan_tiles():
    """192 chains (12 packed sequences x 16 heads) take the scan's 32-column workgroups."""
    p = inputs.prefill(16, 128, lengths=[130, 0, 64, 1, 257, 191, 65, 128, 320, 63, 200, 96], C=64,
                       io="bf16", s0_std=0.02, gate="slow", seed=75)
    _check(p, 64, 4, TOL_BF16, "many chains, wide scan tiles")


def test_snapshots_most_chains_64_column_scan_tiles():
    """Twice as many chains as CUs (the ragged lengths above repeated, 16 heads) take
    the scan's 64-column workgroups, dispatched longest sequence first."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    base = [130, 0, 64, 1, 257, 191, 65, 128, 320, 63, 200, 96]
    n = -(-2 * cus // 16)
    lengths = [base[i % len(base)] for i in range(n)]
    p = inputs.prefill(16, 128, lengths=lengths, C=64, io="bf16", s0_std=0.02, gate="slow", seed=76)
    _check(p, 64, 4, TOL_BF16, f"{16 * n} chains, 64-column scan tiles")


def test_snapshots_f32_path():
    p = inputs.prefill(2, 64, B=1, T=150, C=16, io="f32", seed=73)
    _check(p, 32, 6, TOL_F32, "fp32 path, D=64, C=16")


def test_snapshots_bad_arguments():
    from gated_delta_rule_103_amd.kda import KDAError
    p = inputs.prefill(2, 128, B=1, T=128, C=64, io="bf16", seed=74)
    d = to_dev(p)
    with pytest.raises(KDAError) as e:       # not a multiple of the chunk
        kda_prefill_snapshots(d.q, d.k, d.v, d.g, d.beta, snapshot_every=100, max_snapshots=2, C=64)
    assert e.value.status == -2
    with pytest.raises(KDAError) as e:
        kda_prefill_snapshots(d.q, d.k, d.v, d.g, d.beta, snapshot_every=64, max_snapshots=0, C=64)
    assert e.value.status == -1
