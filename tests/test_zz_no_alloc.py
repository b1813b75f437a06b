"""kda_prefill_noalloc, called through the C ABI, against kda_prefill with a caller
workspace: the same kernels run, so out and S_out must be bit-identical. Two calls
in a row on the library's shared per-device array, the second smaller, then the
fp32 path, one long single sequence (windows run in order), then a size beyond the
array (rejected before any launch)."""
import ctypes

import pytest
import torch

from gated_delta_rule_103_amd import inputs, kda_prefill, load_library
from kda_testlib import to_dev

pytestmark = pytest.mark.gpu

KDA_F32, KDA_BF16 = 0, 1
_DT = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}


def _noalloc(lib, p, out, S_out):
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    B, T, H, Dk = p.q.shape
    Dv = p.v.shape[-1]
    N = B if p.cu_seqlens is None else p.cu_seqlens.numel() - 1
    return lib.kda_prefill_noalloc(ptr(p.q), ptr(p.k), ptr(p.v), ptr(p.g), ptr(p.beta), ptr(p.S0), ptr(out),
                                   ptr(S_out), ptr(p.cu_seqlens), N, B, T, H, Dk, Dv, p.C, _DT[p.q.dtype],
                                   _DT[p.beta.dtype], _DT[out.dtype],
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _case(lib, p):
    d = to_dev(p)
    o_ref, S_ref = kda_prefill(d.q, d.k, d.v, d.g, d.beta, d.S0, cu_seqlens=d.cu_seqlens, C=p.C)
    out, S_out = torch.full_like(o_ref, float("nan")), torch.full_like(S_ref, float("nan"))
    assert _noalloc(lib, d, out, S_out) == 0
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(S_out, S_ref)


def test_noalloc_matches_kda_prefill_twice_then_smaller():
    lib = load_library()
    _case(lib, inputs.prefill(8, 128, lengths=[300, 0, 129, 250], C=64, io="bf16", s0_std=0.2, seed=71))
    _case(lib, inputs.prefill(4, 128, lengths=[65, 1], C=64, io="bf16", s0_std=0.2, seed=72))
    _case(lib, inputs.prefill(2, 64, B=2, T=90, C=16, io="f32", s0_std=0.1, seed=73))


def test_noalloc_long_single_sequence_in_order():
    """One sequence of 2,055 chunks at H = 1: the windowed workspace (two windows of
    records) fits the array; the windows run in order on the stream, bit-identical to
    kda_prefill's overlapped run."""
    lib = load_library()
    T = 4 * 512 * 64 + 6 * 64 + 37
    assert lib.kda_prefill_workspace_size(1, T, 1, 128, 128, 64, KDA_BF16) <= (128 << 20)
    _case(lib, inputs.prefill(1, 128, B=1, T=T, C=64, io="bf16", s0_std=0.02, seed=74))


def test_noalloc_rejects_sizes_beyond_its_array():
    lib = load_library()
    assert lib.kda_prefill_workspace_size(1, 65536, 32, 128, 128, 64, KDA_BF16) > (128 << 20)
    fake = ctypes.c_void_p(256)
    st = lib.kda_prefill_noalloc(fake, fake, fake, fake, fake, None, fake, None, None, 1, 1, 65536, 32, 128, 128,
                                 64, KDA_BF16, KDA_BF16, KDA_BF16, None)
    assert st == -3
