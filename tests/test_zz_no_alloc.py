"""The decode step without allocation (mzattn_decode_noalloc) against the
step with a caller workspace (mzattn_decode), through the C ABI: the same
kernels on the same inputs, so the outputs must be bit-identical; each is
also held to the oracle.  Two calls in a row, the second smaller, share
the library's scratch array."""
import ctypes

import numpy as np
import pytest
import torch

import masked_bidirectional_attention_amd as mz
from masked_bidirectional_attention_amd import _binding as B
from masked_bidirectional_attention_amd import workloads as W
from tests.gpu_helpers import DEV, assert_parity, bits, dev, oracle_decode

pytestmark = pytest.mark.gpu


def _both(case, span=None):
    span = case.span if span is None else span
    kw = dict(span=span, mask=dev(case.mask), scale=case.scale, rope_base=case.rope_base, q_pos=dev(case.q_pos),
              rope_style=case.rope_style)
    q, k, v = dev(case.q), dev(case.k_cache), dev(case.v_cache)
    o_ws = mz.mzattn_decode(q, k, v, **kw)
    o_na = mz.mzattn_decode_noalloc(q, k, v, **kw)
    torch.cuda.synchronize()
    return o_ws, o_na


def test_noalloc_equals_decode_two_calls():
    big = W.vox_decode(3100, span=3328)                       # 26 chunks x 4 units, 8 rows
    small = W.random_decode(81, 1, 8, 2, 3, 700, 64, "bf16", 600, 640, rope_base=1e4, mask_heads=True)
    for case in (big, small):                                 # the second call is smaller
        o_ws, o_na = _both(case)
        assert np.array_equal(bits(o_na), bits(o_ws)), f"{case.name}: noalloc differs from mzattn_decode"
        assert_parity(case.dtype, o_na, oracle_decode(case), f"noalloc {case.name}")
    # and back to the larger shape: nothing left from the smaller call leaks
    o_ws, o_na = _both(big)
    assert np.array_equal(bits(o_na), bits(o_ws))


def test_noalloc_rejects_a_step_above_the_scratch():
    """A cache whose partials exceed the fixed scratch is refused on the
    host (MZ_ERR_WORKSPACE), before anything is launched."""
    L = mz.lib()
    a = B.new_decode_args()
    a.dtype, a.batch, a.heads_q, a.heads_kv, a.q_len, a.head_dim = B.MZ_BF16, 16, 64, 8, 1, 128
    a.cache_len = a.span = 1 << 20
    need = ctypes.c_size_t(0)
    assert L.mzattn_decode_workspace_size(ctypes.byref(a), ctypes.byref(need)) == 0
    assert need.value > (16 << 20)
    buf = torch.zeros(64, dtype=torch.uint8, device=DEV)      # pointers only; never read
    for name in ("q", "k_cache", "v_cache", "o"):
        setattr(a, name, buf.data_ptr())
    st = L.mzattn_decode_noalloc(ctypes.byref(a), None)
    assert st == B.MZ_ERR_WORKSPACE, st
    assert b"scratch" in L.mzattn_last_error()
