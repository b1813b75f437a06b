"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol declared in include/kda.h, and rejects bad arguments with the
documented status before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from gated_delta_rule_103_amd import load_library
    return load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for required in ("kda_prefill", "kda_decode", "kda_prefill_workspace_size",
                     "kda_status_string", "kda_version"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.kda_status_string(0) == b"KDA_OK"
    assert lib.kda_status_string(-3) == b"KDA_ERR_WORKSPACE"
    assert lib.kda_status_string(99) == b"KDA_UNKNOWN_STATUS"


def _prefill(lib, entry="kda_prefill", **kw):
    fake = ctypes.c_void_p(256)          # never dereferenced: checks return first
    a = dict(q=fake, k=fake, v=fake, g=fake, beta=fake, S0=None, out=fake, S_out=None,
             cu=None, N=1, B=1, T=64, H=2, Dk=64, Dv=64, C=16, io=1, bd=1, od=1,
             ws=None, wsb=0, stream=None)
    a.update(kw)
    return getattr(lib, entry)(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["out"], a["S_out"],
                           a["cu"], a["N"], a["B"], a["T"], a["H"], a["Dk"], a["Dv"], a["C"],
                           a["io"], a["bd"], a["od"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(beta=None), -1),
    (dict(N=0), -1), (dict(H=0), -1), (dict(T=-1), -1), (dict(N=2), -1),
    (dict(io=7), -1), (dict(od=3), -1),
    (dict(cu=ctypes.c_void_p(512), B=2, N=2), -1),
    (dict(Dk=96, Dv=96), -2), (dict(Dk=64, Dv=128), -2), (dict(C=8), -2), (dict(C=128), -2),
    (dict(io=0, bd=1, od=0), -2), (dict(io=0, bd=0, od=1), -2),
    (dict(H=70000, Dk=128, Dv=128, C=64), -2),     # a chunk spans more than 2^31 bytes
    (dict(ws=None, wsb=0, io=0, bd=0, od=0), -3),
    (dict(q=ctypes.c_void_p(264)), -1), (dict(g=ctypes.c_void_p(260)), -1),
    (dict(v=ctypes.c_void_p(258)), -1),
    (dict(ws=ctypes.c_void_p(256), wsb=16), -3),
])
def test_prefill_argument_errors(lib, kw, status):
    assert _prefill(lib, **kw) == status


def _prefill_snap(lib, every=64, max_snaps=2, snaps=ctypes.c_void_p(1 << 20), **kw):
    fake = ctypes.c_void_p(256)
    a = dict(q=fake, k=fake, v=fake, g=fake, beta=fake, S0=None, out=fake, S_out=None,
             cu=None, N=1, B=1, T=64, H=2, Dk=64, Dv=64, C=16, io=1, bd=1, od=1,
             ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.kda_prefill_snapshots(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["out"],
                                     a["S_out"], a["cu"], a["N"], a["B"], a["T"], a["H"], a["Dk"],
                                     a["Dv"], a["C"], a["io"], a["bd"], a["od"], every, max_snaps,
                                     snaps, a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("every,max_snaps,snaps,status", [
    (64, 2, None, -1), (0, 2, ctypes.c_void_p(1 << 20), -1), (64, 0, ctypes.c_void_p(1 << 20), -1),
    (24, 2, ctypes.c_void_p(1 << 20), -2),
])
def test_prefill_snapshots_argument_errors(lib, every, max_snaps, snaps, status):
    assert _prefill_snap(lib, every, max_snaps, snaps) == status


def test_prefill_workspace_misaligned(lib):
    need = lib.kda_prefill_workspace_size(1, 64, 2, 64, 64, 16, 1)
    assert need > 0
    assert _prefill(lib, ws=ctypes.c_void_p(4096 + 64), wsb=need) == -3
    # the bf16 MFMA configuration (Dk = Dv = 128, C = 64) keeps one record per (chunk, head)
    assert lib.kda_prefill_workspace_size(1, 8192, 32, 128, 128, 64, 1) >= 129 * 32 * 65536


def test_workspace_of_one_long_sequence_is_bounded(lib):
    """One sequence of at least 2,048 chunks runs in windows of 512 chunks: its workspace
    holds two windows of 66,304-byte records and one fp32 state per head, whatever its
    length; two sequences of the same length keep one record per (chunk, head)."""
    T = 4 * 512 * 64 + 6 * 64 + 37
    one = lib.kda_prefill_workspace_size(1, T, 2, 128, 128, 64, 1)
    longer = lib.kda_prefill_workspace_size(1, 8 * T, 2, 128, 128, 64, 1)
    rec = 2 * 512 * 2 * 66304
    assert rec + 2 * 128 * 128 * 4 <= one < rec + 2 * 128 * 128 * 4 + (1 << 20)
    assert 0 <= longer - one < (1 << 20)
    assert lib.kda_prefill_workspace_size(2, 2 * T, 2, 128, 128, 64, 1) >= 2 * 2055 * 2 * 66304
    # just below the threshold (2,047 chunks) the records cover every chunk
    assert lib.kda_prefill_workspace_size(1, 2047 * 64, 2, 128, 128, 64, 1) >= 2047 * 2 * 66304
    # the long-context workload: 1,048,576 tokens at H = 16, about 1.09 GB instead of 17.4 GB
    assert lib.kda_prefill_workspace_size(1, 1 << 20, 16, 128, 128, 64, 1) < 1_100_000_000


def test_workspace_size_is_pure_and_rejects_bad_sizes(lib):
    a = lib.kda_prefill_workspace_size(16, 135000, 32, 128, 128, 64, 0)
    assert a > 0 and a == lib.kda_prefill_workspace_size(16, 135000, 32, 128, 128, 64, 0)
    assert lib.kda_prefill_workspace_size(0, 100, 2, 64, 64, 16, 1) == 0
    assert lib.kda_prefill_workspace_size(1, 100, 2, 96, 96, 16, 1) == 0
    assert lib.kda_prefill_workspace_size(1, 100, 2, 64, 64, 12, 1) == 0


def _decode(lib, entry="kda_decode", **kw):
    fake = ctypes.c_void_p(256)
    a = dict(q=fake, k=fake, v=fake, g=fake, beta=fake, S=fake, out=fake, N=4, H=2, Dk=128,
             Dv=128, io=1, bd=1, od=1, stream=None)
    a.update(kw)
    return getattr(lib, entry)(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S"], a["out"], a["N"],
                          a["H"], a["Dk"], a["Dv"], a["io"], a["bd"], a["od"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(S=None), -1), (dict(out=None), -1), (dict(g=None), -1), (dict(N=0), -1),
    (dict(H=-1), -1), (dict(io=5), -1), (dict(Dk=32, Dv=32), -2), (dict(Dk=128, Dv=64), -2),
])
def test_decode_argument_errors(lib, kw, status):
    assert _decode(lib, **kw) == status


# gdn_prefill / gdn_decode: a NULL gate is allowed (DeltaNet), so these cases reach
# the later checks; a per-head gate needs 4-byte, not 16-byte, alignment
@pytest.mark.parametrize("kw,status", [
    (dict(g=None, N=0), -1), (dict(g=None, Dk=96, Dv=96), -2), (dict(g=None, q=None), -1),
    (dict(g=ctypes.c_void_p(258)), -1), (dict(g=ctypes.c_void_p(260), C=8), -2),
    (dict(g=None, ws=None, wsb=0, io=0, bd=0, od=0), -3),
])
def test_gdn_prefill_argument_errors(lib, kw, status):
    assert _prefill(lib, "gdn_prefill", **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(g=None, Dk=32, Dv=32), -2), (dict(g=None, S=None), -1), (dict(g=ctypes.c_void_p(258)), -1),
    (dict(g=ctypes.c_void_p(260), N=0), -1),
])
def test_gdn_decode_argument_errors(lib, kw, status):
    assert _decode(lib, "gdn_decode", **kw) == status


def test_cost_models_match_the_pages():
    """The explainer's closed forms at (C, D) = (64, 128): 12C^3 + 8C^2 D + 6CD^2
    FLOPs and 8C^2 + 22CD bytes per chunk per head; decode 7D^2 FLOPs, 8D^2 bytes."""
    from gated_delta_rule_103_amd import costs
    assert costs.prefill_flops_per_chunk(64, 128) == 13_631_488
    assert costs.pages_prefill_bytes_per_chunk(64, 128) == 212_992
    assert costs.prefill_flops(8192, 32, 64, 128) == 128 * 32 * 13_631_488
    assert costs.decode_flops_per_head(128) == 114_688
    assert costs.decode_bytes_per_head(128) == 131_072
    assert costs.prefill_flops_per_chunk(16, 64) == 573_440
    # minimum traffic per token-head at the bf16 workloads: 1538 bytes
    assert costs.prefill_min_bytes(1, 1, 128, 128, 0, writes_state=False) == 1538


def test_input_generators_are_deterministic():
    from gated_delta_rule_103_amd import inputs
    a = inputs.prefill(2, 64, B=1, T=40, io="bf16", seed=5, s0_std=0.02)
    b = inputs.prefill(2, 64, B=1, T=40, io="bf16", seed=5, s0_std=0.02)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.g, b.g), (a.beta, b.beta), (a.S0, b.S0)):
        assert x.dtype == y.dtype and bool((x == y).all())
    import torch
    n = a.q.float().norm(dim=-1)
    assert float((n - 1).abs().max()) < 1e-2
    assert float(a.g.max()) < 0
    lens = inputs.varlen_lengths(16, 512, 16384, 1002)
    assert len(lens) == 16 and min(lens) >= 512 and max(lens) <= 16384
    assert lens == inputs.varlen_lengths(16, 512, 16384, 1002)


def _opts(**kw):
    from gated_delta_rule_103_amd.kda import Options
    return ctypes.byref(Options(**kw))


def _prefill_ex(lib, opt, **kw):
    fake = ctypes.c_void_p(256)
    a = dict(q=fake, k=fake, v=fake, g=fake, beta=fake, S0=None, out=fake, S_out=None,
             cu=None, N=1, B=1, T=64, H=2, Dk=64, Dv=64, C=16, io=1, bd=1, od=1,
             ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.kda_prefill_ex(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["out"], a["S_out"],
                              a["cu"], a["N"], a["B"], a["T"], a["H"], a["Dk"], a["Dv"], a["C"], a["io"],
                              a["bd"], a["od"], opt, a["ws"], a["wsb"], a["stream"])


# options are checked first; valid options fall through to kda_prefill's checks
@pytest.mark.parametrize("opt,kw,status", [
    (dict(gate=2), {}, -1), (dict(gate=-1), {}, -1),
    (dict(qk_l2norm=1, l2norm_eps=0.0), {}, -1), (dict(qk_l2norm=1, l2norm_eps=-1.0), {}, -1),
    (dict(qk_l2norm=1, l2norm_eps=float("nan")), {}, -1),
    (dict(qk_l2norm=1, l2norm_eps=1e-6), dict(C=8), -2),
    (dict(gate=1), dict(g=None, Dk=96, Dv=96), -2),          # per-head gate: NULL g allowed
    (dict(gate=0), dict(g=None), -1),                        # per-channel gate: g required
    (dict(snapshots=1 << 20, snapshot_every=16, max_snapshots=0), {}, -1),
    (None, dict(q=None), -1),
])
def test_prefill_ex_argument_errors(lib, opt, kw, status):
    assert _prefill_ex(lib, None if opt is None else _opts(**opt), **kw) == status


def test_decode_ex_argument_errors(lib):
    fake = ctypes.c_void_p(256)
    call = lambda opt, **kw: lib.kda_decode_ex(fake, fake, fake, kw.get("g", fake), fake, fake, fake, 4, 2,
                                               kw.get("D", 128), kw.get("D", 128), 1, 1, 1, opt, None)
    assert call(_opts(snapshots=1 << 20)) == -1               # no snapshots in decode
    assert call(_opts(qk_l2norm=1, l2norm_eps=0.0)) == -1
    assert call(_opts(gate=3)) == -1
    assert call(_opts(gate=1), g=None, D=32) == -2
    assert call(None, D=32) == -2


def _output_gate(lib, **kw):
    fake = ctypes.c_void_p(256)          # never dereferenced: checks return first
    a = dict(o=fake, gate=fake, w=None, out=ctypes.c_void_p(4096), rows=4, H=2, Dv=64, eps=1e-6,
             od=1, gd=1, outd=1, stream=None)
    a.update(kw)
    return lib.kda_output_gate(a["o"], a["gate"], a["w"], a["out"], a["rows"], a["H"], a["Dv"],
                               a["eps"], a["od"], a["gd"], a["outd"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), -1), (dict(gate=None), -1), (dict(out=None), -1),
    (dict(rows=-1), -1), (dict(H=0), -1), (dict(Dv=0), -1),
    (dict(eps=0.0), -1), (dict(eps=-1.0), -1), (dict(eps=float("nan")), -1),
    (dict(od=2), -1), (dict(gd=5), -1), (dict(outd=-1), -1),
    (dict(o=ctypes.c_void_p(264)), -1), (dict(w=ctypes.c_void_p(260)), -1),
    (dict(out=ctypes.c_void_p(256), outd=0), -1),            # in place with a dtype change
    (dict(rows=1 << 20, H=4096), -1),
    (dict(Dv=96), -2), (dict(Dv=256), -2),
    (dict(rows=0), 0),                                        # nothing to do, nothing launched
    (dict(rows=0, o=None, gate=None, out=None), 0),           # empty tensors may be NULL
    (dict(rows=0, o=None, gate=None, out=None, outd=0), 0),
])
def test_output_gate_argument_errors(lib, kw, status):
    assert _output_gate(lib, **kw) == status


def test_host_paths_from_several_threads(lib):
    """The host side (argument checks, workspace sizing) is a pure function of its
    arguments: the same answers from 8 threads at once."""
    import threading
    want_ws = lib.kda_prefill_workspace_size(3, 1000, 4, 128, 128, 64, 1)
    want_err = _prefill(lib, N=0)
    bad = []

    def work():
        for _ in range(2000):
            if lib.kda_prefill_workspace_size(3, 1000, 4, 128, 128, 64, 1) != want_ws or \
                    _prefill(lib, N=0) != want_err:
                bad.append(1)

    ts = [threading.Thread(target=work) for _ in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert want_ws > 0 and want_err == -1 and not bad


def test_noalloc_checks_before_touching_the_device(lib):
    """kda_prefill_noalloc validates every argument, then the workspace size against its
    fixed array, before it looks the array up on a device (none is needed here)."""
    fake = ctypes.c_void_p(256)
    call = lambda **kw: lib.kda_prefill_noalloc(
        kw.get("q", fake), fake, fake, fake, fake, None, fake, None, None, 1, 1, kw.get("T", 64), 32, 128, 128,
        kw.get("C", 64), 1, 1, 1, None)
    assert call(q=None) == -1
    assert call(C=8) == -2
    assert call(T=65536) == -3          # 65536 x 32 heads needs ~1.1 GB of records
