"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: fp32 max |d| <= 1e-5; fp16 / bf16 relative L2 <= 4e-3 and
max |d| <= 2e-2 * max |ref| (checked by ``mzref.within_tolerance``).
"""
import zlib

import numpy as np
import pytest
import torch

from masked_bidirectional_attention_amd import workloads as W
from oracle import mzref
from tests.gpu_helpers import (DEV, assert_parity, bits, dev, log_parity, oracle_decode, oracle_fwd, run_decode,
                               run_fwd, to64)

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------
# the five named workloads at their full sizes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("materialized", [False, True])
def test_tiny_cfg_fp32(materialized):
    case = W.tiny_cfg(materialized)
    o, lse = run_fwd(case, return_lse=True)
    ref, lse_ref = oracle_fwd(case)
    assert_parity("f32", o, ref, case.name)
    np.testing.assert_allclose(to64(lse), lse_ref, atol=1e-5)


def test_f5_dit_layer_fp16():
    case = W.f5_dit_layer()
    o = run_fwd(case)
    ref, _ = oracle_fwd(case)
    assert_parity("f16", o, ref, case.name)


def test_qwen_padded_bf16():
    case = W.qwen_cfg_padded()
    o, lse = run_fwd(case, return_lse=True)
    ref, lse_ref = oracle_fwd(case)
    assert_parity("bf16", o, ref, case.name)
    # padded query rows of row 1 have no live key: exactly zero, lse -inf
    assert torch.all(o[1, :, W.QWEN_UNCOND:] == 0)
    assert torch.all(torch.isinf(lse[1, :, W.QWEN_UNCOND:]))
    fin = np.isfinite(lse_ref)
    np.testing.assert_allclose(to64(lse)[fin], lse_ref[fin], atol=2e-2)


@pytest.mark.parametrize("as_bool", [False, True])
def test_qwen_packed_bf16(as_bool):
    padded = W.qwen_cfg_padded()
    case = W.qwen_cfg_packed(as_bool_mask=as_bool, padded=padded)
    o = run_fwd(case)
    ref, _ = oracle_fwd(case)
    assert_parity("bf16", o, ref, case.name)


def test_packed_equals_separate_rows():
    """OmniVoice page, 'Memory and speed': the packed row computes what the
    two padded rows compute, segment by segment."""
    padded = W.qwen_cfg_padded()
    packed = W.qwen_cfg_packed(padded=padded)
    op = run_fwd(packed)
    o2 = run_fwd(padded)
    S, U = W.QWEN_S, W.QWEN_UNCOND
    a = torch.cat([o2[0:1], o2[1:2, :, :U]], dim=2)
    st = mzref.parity_stats(to64(op), to64(a))
    same = torch.equal(op, a)
    print(f"[packed vs padded] max_abs={st['max_abs']:.3e} rel_l2={st['rel_l2']:.3e} bitwise={same}", flush=True)
    log_parity({"what": "packed vs padded rows", "bitwise": same, **st})
    assert mzref.within_tolerance("bf16", st)
    # Both segments start on query-tile (128) and key-tile (64) boundaries,
    # the K rotation and the cos / sin rows are the same for the same
    # positions, and keys past the segment end are excluded by a select in
    # both forms (zeros read past the row end, masked keys in the padded
    # row), so every output takes the same operations in the same order.
    assert same, "packed row differs from the separate rows"


@pytest.mark.parametrize("filled", W.VOX_FILLED)
def test_vox_decode(filled):
    full = W.vox_decode(filled)
    o_full = run_decode(full)
    ref = oracle_decode(full)
    assert_parity("bf16", o_full, ref, f"{full.name} span=8192")
    span = W.ceil256(filled)
    o_cut = run_decode(full, span=span)
    assert_parity("bf16", o_cut, ref, f"{full.name} span={span}")
    # the cut past the last live key changes no bit
    assert np.array_equal(bits(o_full), bits(o_cut)), "span truncation changed bits"


# --------------------------------------------------------------------------
# random shapes: ragged tails, several tiles, GQA, dtypes, mask kinds
# --------------------------------------------------------------------------

FWD_SHAPES = [
    # B, Hq, Hkv, Sq, Sk, D
    (1, 2, 1, 1, 1, 64),
    (2, 2, 2, 7, 9, 128),
    (1, 4, 2, 63, 65, 64),
    (2, 8, 1, 129, 300, 128),
    (1, 2, 2, 300, 129, 64),
    (1, 16, 2, 257, 513, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", FWD_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("kind", ["none", "bool_full", "bool_key", "bool_blocky", "segment"])
def test_random_fwd(dtype, shape, kind):
    B, Hq, Hkv, Sq, Sk, D = shape
    seed = zlib.crc32(repr((dtype, shape, kind)).encode()) % 10000
    if kind == "segment":
        if Sq != Sk:
            pytest.skip("segment mode here packs self-attention rows")
        case = W.random_fwd(seed, B, Hq, Hkv, Sq, Sk, D, dtype, W.MASK_SEGMENT, rope_base=1e4, n_segments=3)
    elif kind == "none":
        case = W.random_fwd(seed, B, Hq, Hkv, Sq, Sk, D, dtype, W.MASK_NONE, rope_base=1e4)
    else:
        mshape = {"bool_full": "full", "bool_key": "key", "bool_blocky": "blocky"}[kind]
        case = W.random_fwd(seed, B, Hq, Hkv, Sq, Sk, D, dtype, W.MASK_BOOL, mask_shape=mshape,
                            rope_base=1e6 if Hq != Hkv else 1e4,
                            pe_attn_head=-1 if Hq != Hkv else 1)
    o, lse = run_fwd(case, return_lse=True)
    ref, lse_ref = oracle_fwd(case)
    assert_parity(dtype, o, ref, f"{case.name} {shape}")
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(to64(lse)), fin)
    np.testing.assert_allclose(to64(lse)[fin], lse_ref[fin], atol=1e-4 if dtype == "f32" else 3e-2)


KS_SHAPES = [
    (1, 4, 2, 200, 256, 128),   # 4 key tiles: both streams take two
    (2, 8, 1, 129, 300, 128),   # 5 key tiles: stream 1 takes one fewer
    (1, 2, 2, 300, 129, 64),    # 3 key tiles, D 64
    (1, 16, 2, 257, 513, 128),  # 9 key tiles, ragged tails on both axes
]


@pytest.mark.parametrize("streams", [1, 2])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", KS_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("kind", ["none", "bool_blocky", "bool_key", "segment"])
def test_key_streams(streams, dtype, shape, kind):
    """Both work-group shapes of the MFMA kernel (one key stream, or two
    streams over alternate key tiles merged at the end) against the oracle,
    with odd and even live tile counts and tile classes that skip tiles."""
    B, Hq, Hkv, Sq, Sk, D = shape
    seed = zlib.crc32(repr(("ks", dtype, shape, kind)).encode()) % 10000
    if kind == "segment":
        case = W.random_fwd(seed, B, Hq, Hkv, Sq, Sq, D, dtype, W.MASK_SEGMENT, rope_base=1e4, n_segments=3)
    elif kind == "none":
        case = W.random_fwd(seed, B, Hq, Hkv, Sq, Sk, D, dtype, W.MASK_NONE, rope_base=1e4)
    else:
        case = W.random_fwd(seed, B, Hq, Hkv, Sq, Sk, D, dtype, W.MASK_BOOL,
                            mask_shape={"bool_blocky": "blocky", "bool_key": "key"}[kind], rope_base=1e4)
    o, lse = run_fwd(case, return_lse=True, key_streams=streams)
    ref, lse_ref = oracle_fwd(case)
    assert_parity(dtype, o, ref, f"{case.name} {shape} streams={streams}")
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(to64(lse)), fin)
    np.testing.assert_allclose(to64(lse)[fin], lse_ref[fin], atol=3e-2)


CAUSAL_SHAPES = [
    (1, 2, 2, 1, 1, 64),        # one query, one key
    (2, 4, 2, 300, 300, 128),   # square, ragged tail, GQA
    (1, 8, 1, 129, 500, 128),   # fewer queries than keys (top-left band)
    (2, 2, 2, 400, 70, 64),     # more queries than keys: the last ones see every key
    (1, 16, 2, 1024, 1024, 128),
]


@pytest.mark.parametrize("streams", [1, 2])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", CAUSAL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_causal(streams, dtype, shape):
    """Causal kind (key j live for query i iff j <= i) against the oracle,
    with RoPE, under both work-group shapes of the MFMA kernel."""
    B, Hq, Hkv, Sq, Sk, D = shape
    if dtype == "f32" and Sq * Sk > 300 * 500:
        pytest.skip("fp32 path: small shapes only")
    seed = zlib.crc32(repr(("causal", dtype, shape)).encode()) % 10000
    case = W.random_fwd(seed, B, Hq, Hkv, Sq, Sk, D, dtype, W.MASK_CAUSAL, rope_base=1e4)
    o, lse = run_fwd(case, return_lse=True, key_streams=streams)
    ref, lse_ref = oracle_fwd(case)
    assert_parity(dtype, o, ref, f"{case.name} {shape} streams={streams}")
    np.testing.assert_allclose(to64(lse), lse_ref, atol=1e-4 if dtype == "f32" else 3e-2)
    # query 0 sees key 0 alone: its output is v_0 rounded once
    assert torch.equal(o[:, :, 0].cpu(), case.v[:, torch.arange(Hq) // (Hq // Hkv), 0].to(o.dtype))


def test_causal_equals_bool_tril():
    """The causal kind equals the boolean kind under the explicit
    lower-triangular mask (both on the GPU, same inputs)."""
    import masked_bidirectional_attention_amd as mz
    case = W.random_fwd(77, 2, 8, 2, 700, 900, 128, "bf16", W.MASK_CAUSAL, rope_base=1e6)
    a = run_fwd(case)
    tril = torch.arange(900)[None, :] <= torch.arange(700)[:, None]
    b = mz.mzattn_fwd(dev(case.q), dev(case.k), dev(case.v), mask=dev(tril[None, None]), rope_base=1e6)
    torch.cuda.synchronize()
    ref, _ = oracle_fwd(case, heads=[0, 5])
    for x in (a, b):
        assert_parity("bf16", x[:, [0, 5]], ref[:, [0, 5]], "causal vs tril")
    # both walk the same key tiles in the same order with the same live keys
    assert torch.equal(a, b)


HALF_SHAPES = [
    (1, 4, 4, 100, 140, 64),
    (2, 8, 2, 257, 300, 128),
    (1, 16, 2, 129, 129, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", HALF_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("kind", ["none", "segment", "causal", "bool_key"])
def test_rope_half_split(dtype, shape, kind):
    """Half-split RoPE pairs (x_i, x_i+D/2) on q and k, against the oracle,
    with explicit positions for the plain kind, derived ones for segments."""
    B, Hq, Hkv, Sq, Sk, D = shape
    seed = zlib.crc32(repr(("half", dtype, shape, kind)).encode()) % 10000
    if kind == "segment":
        case = W.random_fwd(seed, B, Hq, Hkv, Sq, Sq, D, dtype, W.MASK_SEGMENT, rope_base=1e4, n_segments=3)
    elif kind == "causal":
        case = W.random_fwd(seed, B, Hq, Hkv, Sq, Sk, D, dtype, W.MASK_CAUSAL, rope_base=1e6)
    elif kind == "bool_key":
        case = W.random_fwd(seed, B, Hq, Hkv, Sq, Sk, D, dtype, W.MASK_BOOL, mask_shape="key", rope_base=1e4,
                            pe_attn_head=-1 if Hq != Hkv else 1)
    else:
        case = W.random_fwd(seed, B, Hq, Hkv, Sq, Sk, D, dtype, W.MASK_NONE, rope_base=1e4, explicit_pos=True)
    case.rope_style = "half"
    o = run_fwd(case)
    ref, _ = oracle_fwd(case)
    assert_parity(dtype, o, ref, f"{case.name} {shape} half")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_rope_half_split(dtype, D):
    """Decode with half-split q rotation at q_pos."""
    case = W.random_decode(41 + D, 2, 8, 2, 3, 700, D, dtype, filled=600, span=640, rope_base=1e4)
    case.rope_style = "half"
    o = run_decode(case)
    assert_parity(dtype, o, oracle_decode(case), f"decode half D{D}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_explicit_positions(dtype):
    case = W.random_fwd(11, 2, 4, 4, 100, 140, 64, dtype, W.MASK_NONE, rope_base=1e4, explicit_pos=True)
    o = run_fwd(case)
    ref, _ = oracle_fwd(case)
    assert_parity(dtype, o, ref, "explicit positions")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", [
    # B, Hq, Hkv, q_len, cache, D, filled, span
    (1, 2, 1, 1, 64, 64, 64, 64),
    (2, 16, 2, 1, 1000, 128, 700, 768),
    (1, 8, 8, 3, 300, 64, 1, 300),
    (2, 4, 1, 16, 513, 128, 513, 513),
    (1, 32, 2, 4, 2048, 128, 1500, 1536),
    (1, 4, 4, 2, 256, 128, 100, 0),
], ids=lambda s: "x".join(map(str, s)))
def test_random_decode(dtype, shape):
    B, Hq, Hkv, T, C, D, filled, span = shape
    case = W.random_decode(zlib.crc32(repr((dtype, shape)).encode()) % 10000, B, Hq, Hkv, T, C, D, dtype, filled, span,
                           mask_heads=True, rope_base=1e4 if T > 1 else 0.0)
    o = run_decode(case)
    ref = oracle_decode(case)
    assert_parity(dtype, o, ref, f"decode {shape}")


# --------------------------------------------------------------------------
# invariants and edge cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_single_live_key_is_exact(dtype):
    """One live key: p = 1, l = 1, so the output is v_j bit for bit."""
    case = W.random_fwd(21, 1, 2, 2, 70, 90, 64, dtype, W.MASK_BOOL, mask_shape="full")
    m = torch.zeros(1, 2, 70, 90, dtype=torch.bool)
    js = torch.randint(0, 90, (2, 70), generator=torch.Generator().manual_seed(3))
    for h in range(2):
        m[0, h, torch.arange(70), js[h]] = True
    case.mask = m
    o = run_fwd(case).cpu()
    for h in range(2):
        assert torch.equal(o[0, h], case.v[0, h, js[h]]), f"head {h}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_masked_garbage_bitwise(dtype):
    """Finite junk in masked K/V positions leaves the output bit-identical."""
    case = W.random_fwd(22, 2, 4, 2, 150, 200, 128, dtype, W.MASK_BOOL, mask_shape="key")
    case.mask[:, :, :, 150:] = False
    o1 = run_fwd(case)
    k2, v2 = case.k.clone(), case.v.clone()
    g = torch.Generator().manual_seed(5)
    k2[:, :, 150:] = (torch.randn(k2[:, :, 150:].shape, generator=g) * 1000).to(k2.dtype)
    v2[:, :, 150:] = (torch.randn(v2[:, :, 150:].shape, generator=g) * 1000).to(v2.dtype)
    o2 = run_fwd(case, k=dev(k2), v=dev(v2))
    assert torch.equal(o1, o2)


def test_decode_masked_garbage_bitwise():
    case = W.random_decode(23, 2, 16, 2, 1, 1024, 128, "bf16", 300, 1024, garbage=1000.0)
    clean = W.random_decode(23, 2, 16, 2, 1, 1024, 128, "bf16", 300, 1024)
    assert torch.equal(run_decode(case), run_decode(clean))


def test_fully_masked_and_empty():
    case = W.random_fwd(24, 1, 2, 2, 40, 50, 64, "bf16", W.MASK_BOOL, mask_shape="full")
    case.mask[:, :, 5:9] = False
    o, lse = run_fwd(case, return_lse=True)
    assert torch.all(o[:, :, 5:9] == 0) and torch.all(torch.isinf(lse[:, :, 5:9]))
    # no keys at all
    e = W.random_fwd(25, 1, 2, 2, 10, 0, 64, "bf16")
    oe = run_fwd(e)
    assert oe.shape == (1, 2, 10, 64) and torch.all(oe == 0)
    # no queries: a legal no-op
    z = W.random_fwd(26, 1, 2, 2, 0, 10, 64, "bf16")
    assert run_fwd(z).shape == (1, 2, 0, 64)
    # no keys under a boolean mask (the mask itself is empty): zeros, lse -inf
    for dtype in ("bf16", "f32"):
        eb = W.random_fwd(25, 2, 2, 2, 10, 0, 64, dtype, W.MASK_BOOL, mask_shape="key")
        ob, lb = run_fwd(eb, return_lse=True)
        assert ob.shape == (2, 2, 10, 64) and torch.all(ob == 0) and torch.all(torch.isinf(lb))


def test_deterministic():
    case = W.random_fwd(27, 2, 8, 2, 333, 333, 128, "bf16", W.MASK_SEGMENT, rope_base=1e6, n_segments=3)
    a = run_fwd(case)
    b = run_fwd(case)
    assert torch.equal(a, b)
    d = W.vox_decode(3100)
    assert torch.equal(run_decode(d), run_decode(d))


def test_calls_on_two_streams_at_once():
    """Forward and decode calls issued on two streams with nothing ordering
    them (each call with its own workspace: the one-shot entry points keep
    one per stream) give the bits of the same calls made one at a time."""
    import masked_bidirectional_attention_amd as mz
    fa = W.random_fwd(96, 2, 8, 2, 333, 333, 128, "bf16", W.MASK_SEGMENT, rope_base=1e6, n_segments=3)
    fb = W.random_fwd(97, 2, 16, 16, 300, 300, 64, "f16", W.MASK_BOOL, mask_shape="blocky", rope_base=1e4)
    dc = W.vox_decode(3100)
    ref = [run_fwd(fa), run_fwd(fb), run_decode(dc)]
    ins = [[dev(x) for x in (c.q, c.k, c.v)] for c in (fa, fb)]
    seg, mask = dev(fa.seg_q), dev(fb.mask)
    dq, dk, dv, dm = dev(dc.q), dev(dc.k_cache), dev(dc.v_cache), dev(dc.mask)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            oa = mz.mzattn_fwd(*ins[0], seg_q=seg, seg_k=seg, rope_base=1e6, stream=s1)
            od = mz.mzattn_decode(dq, dk, dv, span=dc.span, mask=dm, scale=dc.scale, stream=s1)
        with torch.cuda.stream(s2):
            ob = mz.mzattn_fwd(*ins[1], mask=mask, rope_base=1e4, stream=s2)
        outs.append((oa, ob, od))
    torch.cuda.synchronize()
    for oa, ob, od in outs:
        assert torch.equal(oa, ref[0]) and torch.equal(ob, ref[1]) and torch.equal(od, ref[2])


def test_gqa_equals_repeated_heads():
    case = W.random_fwd(28, 1, 8, 2, 200, 200, 128, "bf16", W.MASK_BOOL, mask_shape="bcast_h", rope_base=1e6)
    a = run_fwd(case)
    rep = W.FwdCase(case.name, case.dtype, case.q, case.k.repeat_interleave(4, 1),
                    case.v.repeat_interleave(4, 1), rope_base=case.rope_base, mask_kind=case.mask_kind,
                    mask=case.mask)
    b = run_fwd(rep)
    assert torch.equal(a, b)


def test_decode_matches_fwd_single_query():
    """A decode step with q_len 1 equals the forward with Sq = 1 over the
    same keys (two different kernels; tolerance, not bits)."""
    d = W.random_decode(29, 2, 8, 2, 1, 600, 128, "bf16", 600, 600, mask_heads=True)
    od = run_decode(d)
    f = W.FwdCase("fwd1", "bf16", d.q, d.k_cache, d.v_cache, mask_kind=W.MASK_BOOL, mask=d.mask)
    of = run_fwd(f)
    st = mzref.parity_stats(to64(od), to64(of))
    assert mzref.within_tolerance("bf16", st), st


def test_plan_then_execute_equals_fwd():
    import masked_bidirectional_attention_amd as mz
    case = W.random_fwd(30, 1, 8, 2, 500, 500, 128, "bf16", W.MASK_SEGMENT, rope_base=1e6, n_segments=3)
    a = run_fwd(case)
    call = mz.FwdCall(dev(case.q), dev(case.k), dev(case.v), seg_q=dev(case.seg_q), seg_k=dev(case.seg_k),
                      rope_base=case.rope_base)
    call.plan()
    call.execute()
    call.execute()  # executing again over the same plan is allowed
    torch.cuda.synchronize()
    assert torch.equal(call.out, a)
    # the plan depends on the layout only: new Q/K/V under the same plan
    # (K rotated again by execute) give what a full call on them gives
    case2 = W.random_fwd(31, 1, 8, 2, 500, 500, 128, "bf16", W.MASK_SEGMENT, rope_base=1e6, n_segments=3)
    case2.seg_q, case2.seg_k = case.seg_q, case.seg_k
    b2 = run_fwd(case2)
    call.set_inputs(dev(case2.q), dev(case2.k), dev(case2.v))
    call.rotate_k()
    call.attend()
    torch.cuda.synchronize()
    assert torch.equal(call.out, b2)


def test_plan_survives_other_calls_on_the_stream():
    """A planned call keeps its plan while other calls (one-shot and
    planned, with other masks and shapes) run on the same stream between
    its plan and its executes."""
    import masked_bidirectional_attention_amd as mz
    a = W.random_fwd(34, 2, 8, 2, 300, 400, 128, "bf16", W.MASK_BOOL, mask_shape="blocky", rope_base=1e6)
    b = W.random_fwd(35, 2, 8, 2, 300, 400, 128, "bf16", W.MASK_BOOL, mask_shape="full", rope_base=1e4)
    c = W.random_fwd(36, 1, 8, 2, 257, 257, 128, "bf16", W.MASK_SEGMENT, rope_base=1e6, n_segments=3)
    call_a = mz.FwdCall(dev(a.q), dev(a.k), dev(a.v), mask=dev(a.mask), rope_base=a.rope_base)
    call_a.plan()
    run_fwd(b)                      # one-shot call in between
    run_fwd(c)
    call_b = mz.FwdCall(dev(b.q), dev(b.k), dev(b.v), mask=dev(b.mask), rope_base=b.rope_base)
    call_b.plan()                   # another plan in between
    call_a.execute()
    call_b.execute()
    torch.cuda.synchronize()
    ref_a, _ = oracle_fwd(a)
    assert_parity("bf16", call_a.out, ref_a, "plan kept across other calls")
    ref_b, _ = oracle_fwd(b)
    assert_parity("bf16", call_b.out, ref_b, "second planned call")


def _segment_rows(rng, B, S, ids, pad_front):
    """Non-decreasing id rows of length S over the given ids (random run
    lengths), with an optional run of padding (-1) in front."""
    rows = []
    for b in range(B):
        cuts = np.sort(rng.choice(np.arange(1, S), size=len(ids) - 1, replace=False))
        row = np.full(S, ids[0], dtype=np.int32)
        for c, v in zip(cuts, ids[1:]):
            row[c:] = v
        if pad_front and b == 0:
            row[:int(rng.integers(1, S // 6))] = -1
        rows.append(row)
    return torch.from_numpy(np.stack(rows))


@pytest.mark.parametrize("cfg", [
    # B, Hq, Hkv, Sq, Sk, D, dtype, query ids, key ids
    (2, 4, 2, 300, 500, 128, "bf16", [0, 1, 2], [0, 1, 2, 3]),
    (1, 2, 2, 260, 130, 64, "f16", [0, 2, 3], [0, 1, 2]),
    (2, 2, 1, 100, 170, 64, "f32", [1, 2], [0, 1, 2]),
], ids=lambda c: f"{c[3]}x{c[4]}-{c[6]}")
def test_segment_rows_of_different_lengths(cfg):
    """Segment mode with seq_q != seq_k and distinct id rows: query i and
    key j are live together iff their ids are equal and >= 0; positions
    restart at 0 in every run on each axis separately.  Ids present on one
    axis only leave their queries with no live key (zero output)."""
    import masked_bidirectional_attention_amd as mz
    B, Hq, Hkv, Sq, Sk, D, dtype, qids, kids = cfg
    rng = np.random.default_rng(zlib.crc32(repr(cfg).encode()) % 10000)
    case = W.random_fwd(int(rng.integers(1 << 20)), B, Hq, Hkv, Sq, Sk, D, dtype, rope_base=1e4)
    sq = _segment_rows(rng, B, Sq, qids, pad_front=True)
    sk = _segment_rows(rng, B, Sk, kids, pad_front=False)
    o, lse = mz.mzattn_fwd(dev(case.q), dev(case.k), dev(case.v), seg_q=dev(sq), seg_k=dev(sk), rope_base=1e4,
                           return_lse=True)
    torch.cuda.synchronize()
    ref, lse_ref = mzref.mzref_fwd(dtype, W.to_bits(case.q), W.to_bits(case.k), W.to_bits(case.v), rope_base=1e4,
                                   mask_kind="segment", seg_q=sq.numpy(), seg_k=sk.numpy())
    assert_parity(dtype, o, ref, f"segments {Sq}x{Sk}")
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(to64(lse)), fin) and not fin.all()
    np.testing.assert_allclose(to64(lse)[fin], lse_ref[fin], atol=1e-4 if dtype == "f32" else 3e-2)


@pytest.mark.parametrize("S", [4096, 5000])
def test_long_segment_rows_fwd(S):
    """Segment rows longer than the LDS search buffer take the global path."""
    case = W.random_fwd(31, 1, 2, 1, S, S, 64, "bf16", W.MASK_SEGMENT, rope_base=1e4, n_segments=4)
    o = run_fwd(case)
    ref, _ = oracle_fwd(case)
    assert_parity("bf16", o, ref, f"long segments S={S}")


@pytest.mark.parametrize("streams", [1, 2])
@pytest.mark.parametrize("Sk", [4096, 4097, 4200])
def test_bool_mask_dead_tiles(Sk, streams):
    """A boolean mask with whole dead 64-key tiles between live and mixed
    ones, on rows of exactly 64 key tiles (the per-row tile sets fit one
    64-bit word) and of 65 or 66 (they do not): skipped tiles, boundary tests and
    the live-tile count of the two-stream split against the oracle."""
    case = W.random_fwd(77 + Sk, 2, 4, 2, 130, Sk, 64, "bf16", W.MASK_NONE, rope_base=1e4)
    i = torch.arange(130)[:, None]
    j = torch.arange(Sk)[None, :]
    m = (((j // 192) + (i // 100)) % 2 == 0) | ((j % 7 == 0) & (i % 5 == 0))
    case.mask_kind, case.mask = W.MASK_BOOL, torch.stack([m, ~m])[:, None].contiguous()
    o = run_fwd(case, key_streams=streams)
    ref, _ = oracle_fwd(case)
    assert_parity("bf16", o, ref, f"dead tiles Sk={Sk} streams={streams}")


@pytest.mark.parametrize("kind", ["none", "bool_key"])
def test_max_key_length_fwd(kind):
    """The longest key row the forward accepts (2^20 keys: 16384 key tiles,
    class bytes read from global memory, two key streams over one query
    tile) against the oracle."""
    Sk = 1 << 20
    if kind == "none":
        case = W.random_fwd(91, 1, 2, 1, 40, Sk, 64, "bf16", W.MASK_NONE, rope_base=1e4)
    else:
        case = W.random_fwd(92, 1, 2, 1, 40, Sk, 64, "bf16", W.MASK_BOOL, mask_shape="key", rope_base=1e4)
    o = run_fwd(case)
    ref, _ = oracle_fwd(case)
    assert_parity("bf16", o, ref, f"max key length {kind}")


@pytest.mark.parametrize("shape,dtype,kind", [
    ((65535, 1, 1, 3, 5, 64), "bf16", "bool_key"),   # largest batch, K rotated in the attention kernel
    ((65535, 1, 1, 3, 5, 64), "f32", "bool_key"),
    ((1, 65535, 1, 3, 70, 64), "bf16", "none"),      # largest head count, one kv-head (G = 65535), K pass
], ids=["batch-bf16", "batch-f32", "heads-bf16"])
def test_max_batch_and_heads(shape, dtype, kind):
    """The largest batch and head counts the forward accepts (65535 each)
    against the oracle: grids of 65535 work-groups and K-pass grids with
    65535 batch rows."""
    B, Hq, Hkv, Sq, Sk, D = shape
    mk = W.MASK_BOOL if kind == "bool_key" else W.MASK_NONE
    case = W.random_fwd(94, B, Hq, Hkv, Sq, Sk, D, dtype, mk, mask_shape="key", rope_base=1e4)
    o = run_fwd(case)
    ref, _ = oracle_fwd(case)
    assert_parity(dtype, o, ref, f"max batch / heads {shape} {dtype}")


def test_decode_max_cache():
    """The largest static cache the decode accepts (2^24 positions, 131072
    chunks, 2048 merge super-groups): 1000 live keys, the rest finite junk
    under the mask.  Full span and the span cut after the live keys give the
    same bits, and both match the oracle on the live part."""
    import masked_bidirectional_attention_amd as mz
    C, small = 1 << 24, 1024
    case = W.random_decode(93, 1, 2, 1, 1, small, 64, "bf16", filled=1000, span=small)
    kb = torch.full((1, 1, C, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    vb = torch.full((1, 1, C, 64), -5.0, dtype=torch.bfloat16, device=DEV)
    kb[:, :, :small] = dev(case.k_cache)
    vb[:, :, :small] = dev(case.v_cache)
    mb = torch.zeros((1, 1, 1, C), dtype=torch.bool, device=DEV)
    mb[..., :small] = dev(case.mask)
    outs = []
    for span in (C, small):
        outs.append(mz.mzattn_decode(dev(case.q), kb, vb, span=span, mask=mb, scale=case.scale))
        torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "span truncation changed bits"
    assert_parity("bf16", outs[0], oracle_decode(case), "max cache")


def test_decode_call_set_cache():
    import masked_bidirectional_attention_amd as mz
    a = W.random_decode(32, 2, 8, 2, 1, 500, 128, "bf16", 400, 500)
    b2 = W.random_decode(33, 2, 8, 2, 1, 500, 128, "bf16", 450, 500)
    call = mz.DecodeCall(dev(a.q), dev(a.k_cache), dev(a.v_cache), span=500, mask=dev(a.mask))
    o1 = call().clone()
    call.set_cache(dev(b2.k_cache), dev(b2.v_cache))
    o2 = call().clone()
    torch.cuda.synchronize()
    assert torch.equal(o1, run_decode(a))
    ref = mzref.mzref_decode("bf16", W.to_bits(a.q), W.to_bits(b2.k_cache), W.to_bits(b2.v_cache), span=500,
                             mask=a.mask.numpy())
    assert_parity("bf16", o2, ref, "decode after set_cache")


# --------------------------------------------------------------------------
# decode: no mask, empty span, 64 rows per head group; one workspace shared
# by calls of several shapes and spans
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", [
    # B, Hq, Hkv, q_len, cache, D, span   (no mask: every key in the span)
    (2, 16, 2, 1, 8192, 128, 8192),
    (1, 32, 2, 4, 1200, 128, 1100),   # 64 rows per head group
    (2, 8, 1, 2, 700, 64, 513),
    (1, 4, 4, 1, 300, 64, 1),
    (1, 4, 2, 1, 300, 128, 0),        # empty span, no mask: output 0
], ids=lambda s: "x".join(map(str, s)))
def test_decode_no_mask(dtype, shape):
    B, Hq, Hkv, T, C, D, span = shape
    case = W.random_decode(zlib.crc32(repr(("nomask", dtype, shape)).encode()) % 10000, B, Hq, Hkv, T, C, D,
                           dtype, C, span)
    case.mask = None
    o = run_decode(case)
    if span == 0:
        assert torch.all(o == 0)
        return
    assert_parity(dtype, o, oracle_decode(case), f"decode no mask {shape}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_decode_long_cache(dtype):
    """A cache of 547 chunks (the merge folds nine super-groups of 64, the
    last ragged): parity, and the span cut past the last live key changes
    no bit."""
    case = W.random_decode(71, 2, 8, 1, 2, 70000, 64, dtype, filled=68001, span=70000, mask_heads=True)
    o = run_decode(case)
    assert_parity(dtype, o, oracle_decode(case), f"long cache {dtype}")
    o_cut = run_decode(case, span=W.ceil256(68001))
    assert np.array_equal(bits(o), bits(o_cut)), "span truncation changed bits"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_repeated_calls_share_workspace(dtype):
    """Calls of several shapes and spans (one chunk to 71 chunks, 1 to 4
    query rows per head) through one workspace that starts as all-ones
    bytes (NaN as floats), each checked against the oracle: nothing a call
    reads from the workspace may be left from before it."""
    import masked_bidirectional_attention_amd as mz
    cases = [W.random_decode(60 + i, B, Hq, Hkv, T, C, 128, dtype, fill, span)
             for i, (B, Hq, Hkv, T, C, fill, span) in enumerate([
                 (2, 16, 2, 1, 4096, 3000, 4096), (2, 16, 2, 1, 4096, 3000, 3072), (1, 8, 1, 1, 4096, 200, 256),
                 (2, 16, 2, 1, 4096, 4096, 4096), (3, 8, 1, 2, 1500, 1400, 1408), (1, 4, 4, 1, 100, 100, 100),
                 (4, 16, 4, 1, 9000, 8800, 8960), (2, 16, 2, 1, 4096, 3000, 4096)])]
    ws = torch.full((16 << 20,), 255, dtype=torch.uint8, device=DEV)
    for rep in range(2):
        for c in cases:
            call = mz.DecodeCall(dev(c.q), dev(c.k_cache), dev(c.v_cache), span=c.span, mask=dev(c.mask),
                                 workspace=ws)
            o = call()
            torch.cuda.synchronize()
            assert_parity(dtype, o, oracle_decode(c), f"{c.name} span={c.span} pass {rep}")


# --------------------------------------------------------------------------
# decode with append: the filled length is read on the device
# --------------------------------------------------------------------------

def _append_case(seed, B, Hq, Hkv, T, C, D, dtype, lens, mask_kind="none"):
    gen = torch.Generator().manual_seed(seed)
    cast = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    q = torch.randn(B, Hq, T, D, generator=gen).to(cast)
    kn = torch.randn(B, Hkv, T, D, generator=gen).to(cast)
    vn = torch.randn(B, Hkv, T, D, generator=gen).to(cast)
    kc = torch.randn(B, Hkv, C, D, generator=gen).to(cast)
    vc = torch.randn(B, Hkv, C, D, generator=gen).to(cast)
    rng = np.random.default_rng(seed + 7)
    mask = None
    if mask_kind == "bcast":
        mask = torch.from_numpy(rng.random((B, 1, 1, C)) < 0.9)
    elif mask_kind == "heads":
        mask = torch.from_numpy(rng.random((B, Hq, T, C)) < 0.8)
    return q, kn, vn, kc, vc, torch.tensor(lens, dtype=torch.int32), mask


@pytest.mark.parametrize("cfg", [
    # B, Hq, Hkv, T, C, D, dtype, lens, rope_style, mask
    (2, 16, 2, 1, 8192, 128, "bf16", [8191, 300], "interleaved", "none"),
    (2, 16, 2, 1, 8192, 128, "f16", [0, 4000], "half", "bcast"),
    (1, 32, 2, 4, 1200, 128, "bf16", [777], "interleaved", "heads"),
    (2, 8, 1, 2, 700, 64, "bf16", [127, 255], "half", "none"),
    (3, 4, 4, 3, 300, 64, "f16", [0, 10, 298], "interleaved", "bcast"),   # row 2 overflows
], ids=lambda c: "x".join(map(str, c[:6])) + f"-{c[6]}-{c[8]}-{c[9]}")
def test_decode_append(cfg):
    import masked_bidirectional_attention_amd as mz
    B, Hq, Hkv, T, C, D, dtype, lens, style, mk = cfg
    q, kn, vn, kc, vc, ln, mask = _append_case(zlib.crc32(repr(cfg).encode()) % 10000, B, Hq, Hkv, T, C, D, dtype,
                                               lens, mk)
    kc_d, vc_d = dev(kc), dev(vc)
    ovf = torch.zeros(1, dtype=torch.int32, device=DEV)
    print(f"[append] {cfg}", flush=True)
    o = mz.mzattn_decode_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, dev(ln), mask=dev(mask), rope_base=1e4,
                                rope_style=style, overflow=ovf)
    torch.cuda.synchronize()
    ref, k_rows, overflow = mzref.mzref_decode_append(
        dtype, W.to_bits(q), W.to_bits(kn), W.to_bits(vn), W.to_bits(kc), W.to_bits(vc), lens,
        mask=None if mask is None else mask.numpy(), rope_base=1e4, rope_style=style)
    assert_parity(dtype, o, ref, f"append {cfg}")
    assert int(ovf.item()) == int(overflow.any())
    kc2, vc2 = kc_d.cpu(), vc_d.cpu()
    for b in range(B):
        L = lens[b]
        if overflow[b]:
            assert torch.all(o[b] == 0)
            assert torch.equal(kc2[b], kc[b]) and torch.equal(vc2[b], vc[b]), "overflow row touched the cache"
            continue
        # untouched rows stay bit-identical; the new V rows are copied bit
        # for bit; the new K rows are the rotated keys in the storage type
        assert torch.equal(kc2[b, :, :L], kc[b, :, :L]) and torch.equal(kc2[b, :, L + T:], kc[b, :, L + T:])
        assert torch.equal(vc2[b, :, :L], vc[b, :, :L]) and torch.equal(vc2[b, :, L + T:], vc[b, :, L + T:])
        assert torch.equal(vc2[b, :, L:L + T], vn[b])
        got = kc2[b, :, L:L + T].double().numpy()
        ulp = 2.0 ** (-7 if dtype == "bf16" else -10)
        assert np.all(np.abs(got - k_rows[b]) <= ulp * np.abs(k_rows[b]) + 1e-6), "appended key rows"


def test_decode_append_equals_decode_on_updated_cache():
    """The append step gives the bits mzattn_decode gives on the updated
    cache with the mask j <= len + t and q rotated at len + t."""
    import masked_bidirectional_attention_amd as mz
    B, Hq, Hkv, T, C, D = 2, 16, 2, 3, 2048, 128
    lens = [1000, 2040]
    q, kn, vn, kc, vc, ln, _ = _append_case(91, B, Hq, Hkv, T, C, D, "bf16", lens)
    kc_d, vc_d = dev(kc), dev(vc)
    o1 = mz.mzattn_decode_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, dev(ln), rope_base=1e6)
    m = torch.zeros(B, 1, T, C, dtype=torch.bool)
    pos = torch.zeros(B, T, dtype=torch.int32)
    for b in range(B):
        for t in range(T):
            m[b, 0, t, :lens[b] + t + 1] = True
            pos[b, t] = lens[b] + t
    o2 = mz.mzattn_decode(dev(q), kc_d, vc_d, span=C, mask=dev(m), rope_base=1e6, q_pos=dev(pos))
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2))


def test_decode_append_graph_replay():
    """Recorded once in a HIP graph, replayed while the length advances on
    the device between replays: every replay equals an eager call on the
    same cache state."""
    import masked_bidirectional_attention_amd as mz
    B, Hq, Hkv, T, C, D = 2, 16, 2, 1, 4096, 128
    q, kn, vn, kc, vc, _, _ = _append_case(92, B, Hq, Hkv, T, C, D, "bf16", [0, 0])
    s = torch.cuda.Stream()
    length = torch.tensor([100, 2500], dtype=torch.int32, device=DEV)
    kc_g, vc_g = dev(kc), dev(vc)
    dq, dkn, dvn = dev(q), dev(kn), dev(vn)
    call = mz.DecodeAppendCall(dq, dkn, dvn, kc_g, vc_g, length, rope_base=1e4, stream=s)
    kc_e, vc_e = kc_g.clone(), vc_g.clone()     # the eager twin's caches
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    # capture recorded the work without running it: the caches are unchanged
    assert torch.equal(kc_g, kc_e)
    for step in range(4):
        lens_now = length.clone()
        g.replay()
        torch.cuda.synchronize()
        o_graph = call.out.clone()
        o_eager = mz.mzattn_decode_append(dq, dkn, dvn, kc_e, vc_e, lens_now, rope_base=1e4)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o_graph), bits(o_eager)), f"replay {step}"
        assert torch.equal(kc_g, kc_e) and torch.equal(vc_g, vc_e), f"caches after replay {step}"
        length += 1                                  # next position, on the device


# --------------------------------------------------------------------------
# RoPE variants: LongRoPE factors and attention factor; upstream precisions
# --------------------------------------------------------------------------

_ROPE_VARIANTS = [
    # precision, with factors, mscale
    ("fp16", False, 0.0),
    ("bf16_table", True, 1.118),
    ("exact", True, 1.25),
]


def _factors(D, seed):
    return torch.from_numpy((1.0 + 3.0 * np.random.default_rng(seed).random(D // 2)).astype(np.float32))


@pytest.mark.parametrize("variant", _ROPE_VARIANTS, ids=lambda v: f"{v[0]}-{'factors' if v[1] else 'nofactors'}")
@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_rope_variants_fwd(variant, style, dtype):
    """Forward with the RoPE options (table route for positions below the
    table size, the direct route above: segment positions are short, the
    explicit positions reach 20000)."""
    prec, with_f, mscale = variant
    import masked_bidirectional_attention_amd as mz
    case = W.random_fwd(zlib.crc32(repr(("ropev", prec, style, dtype)).encode()) % 10000, 2, 4, 2, 130, 150,
                        128 if dtype != "f32" else 64, dtype, W.MASK_BOOL, rope_base=1e4, mask_shape="key")
    D = case.q.shape[-1]
    f = _factors(D, 5) if with_f else None
    rng = np.random.default_rng(6)
    pq = torch.from_numpy(rng.integers(0, 20000, size=(2, 130)).astype(np.int32))
    pk = torch.from_numpy(rng.integers(0, 20000, size=(2, 150)).astype(np.int32))
    o = mz.mzattn_fwd(dev(case.q), dev(case.k), dev(case.v), mask=dev(case.mask), rope_base=1e4, rope_style=style,
                      pos_q=dev(pq), pos_k=dev(pk), rope_precision=prec, rope_mscale=mscale,
                      rope_factors=dev(f))
    torch.cuda.synchronize()
    ref, _ = mzref.mzref_fwd(dtype, W.to_bits(case.q), W.to_bits(case.k), W.to_bits(case.v), rope_base=1e4,
                             rope_style=style, pos_q=pq.numpy(), pos_k=pk.numpy(), mask_kind="bool",
                             mask=case.mask.numpy(), rope_precision=prec,
                             rope_factors=None if f is None else f.numpy().astype(np.float64),
                             rope_mscale=mscale if mscale > 0 else 1.0)
    assert_parity(dtype, o, ref, f"rope {variant} {style}")


@pytest.mark.parametrize("variant", _ROPE_VARIANTS, ids=lambda v: f"{v[0]}-{'factors' if v[1] else 'nofactors'}")
def test_rope_variants_decode_and_append(variant):
    prec, with_f, mscale = variant
    import masked_bidirectional_attention_amd as mz
    f = _factors(128, 7) if with_f else None
    fo = None if f is None else f.numpy().astype(np.float64)
    ms = mscale if mscale > 0 else 1.0
    case = W.random_decode(77, 2, 16, 2, 2, 3000, 128, "bf16", 2500, 2560, rope_base=1e4)
    o = mz.mzattn_decode(dev(case.q), dev(case.k_cache), dev(case.v_cache), span=case.span, mask=dev(case.mask),
                         rope_base=1e4, q_pos=dev(case.q_pos), rope_precision=prec, rope_mscale=mscale,
                         rope_factors=dev(f))
    torch.cuda.synchronize()
    ref = mzref.mzref_decode("bf16", W.to_bits(case.q), W.to_bits(case.k_cache), W.to_bits(case.v_cache),
                             span=case.span, mask=case.mask.numpy(), rope_base=1e4, q_pos=case.q_pos.numpy(),
                             rope_precision=prec, rope_factors=fo, rope_mscale=ms)
    assert_parity("bf16", o, ref, f"decode rope {variant}")
    q, kn, vn, kc, vc, ln, _ = _append_case(78, 2, 16, 2, 2, 3000, 128, "bf16", [2000, 2997])
    kc_d, vc_d = dev(kc), dev(vc)
    oa = mz.mzattn_decode_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, dev(ln), rope_base=1e4,
                                 rope_precision=prec, rope_mscale=mscale, rope_factors=dev(f))
    torch.cuda.synchronize()
    refa, k_rows, _ = mzref.mzref_decode_append("bf16", W.to_bits(q), W.to_bits(kn), W.to_bits(vn), W.to_bits(kc),
                                                W.to_bits(vc), [2000, 2997], rope_base=1e4, rope_precision=prec,
                                                rope_factors=fo, rope_mscale=ms)
    assert_parity("bf16", oa, refa, f"append rope {variant}")


# --------------------------------------------------------------------------
# q / k RMSNorm before RoPE (forward)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [
    # dtype, D, mask kind, rope_base, pe_attn_head, style, which norms
    ("bf16", 128, W.MASK_SEGMENT, 1e6, -1, "interleaved", "qk"),
    ("bf16", 128, W.MASK_BOOL, 1e6, -1, "half", "qk"),
    ("f16", 64, W.MASK_BOOL, 1e4, 1, "interleaved", "qk"),    # RoPE on head 0 only, norm on all
    ("bf16", 128, W.MASK_NONE, 0.0, -1, "interleaved", "k"),   # no RoPE: the K pass only normalises
    ("f16", 128, W.MASK_CAUSAL, 1e4, -1, "half", "q"),
    ("f32", 64, W.MASK_BOOL, 1e4, -1, "interleaved", "qk"),
    ("f32", 128, W.MASK_NONE, 0.0, -1, "half", "q"),
], ids=lambda c: "-".join(map(str, c)))
def test_qk_rms_norm(cfg):
    import masked_bidirectional_attention_amd as mz
    dtype, D, kind, base, pe, style, which = cfg
    Hq, Hkv = (4, 4) if pe >= 0 else (8, 2)
    case = W.random_fwd(zlib.crc32(repr(cfg).encode()) % 10000, 2, Hq, Hkv, 200, 200, D, dtype, kind,
                        rope_base=base, pe_attn_head=pe, mask_shape="key", n_segments=2)
    cast = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    gen = torch.Generator().manual_seed(11)
    wq = (1.0 + 0.5 * torch.randn(D, generator=gen)).to(cast) if "q" in which else None
    wk = (1.0 + 0.5 * torch.randn(D, generator=gen)).to(cast) if "k" in which else None
    # the normalised inputs far from unit scale, so a missing normalisation
    # shows (the others keep N(0,1) logits: a 4x q would make the softmax
    # sharper than the 16-bit tolerances are stated for)
    q = (case.q.float() * (4.0 if wq is not None else 1.0)).to(cast)
    k = (case.k.float() * (0.3 if wk is not None else 1.0)).to(cast)
    kw = dict(rope_base=base, pe_attn_head=pe, rope_style=style, q_norm_weight=dev(wq), k_norm_weight=dev(wk),
              norm_eps=1e-6)
    if kind == W.MASK_BOOL:
        kw["mask"] = dev(case.mask)
    elif kind == W.MASK_SEGMENT:
        kw["seg_q"], kw["seg_k"] = dev(case.seg_q), dev(case.seg_k)
    elif kind == W.MASK_CAUSAL:
        kw["causal"] = True
    o = mz.mzattn_fwd(dev(q), dev(k), dev(case.v), **kw)
    torch.cuda.synchronize()
    ref, _ = mzref.mzref_fwd(dtype, W.to_bits(q), W.to_bits(k), W.to_bits(case.v), rope_base=base,
                             pe_attn_head=pe, rope_style=style, mask_kind=case.mask_kind,
                             mask=None if case.mask is None else case.mask.numpy(),
                             seg_q=None if case.seg_q is None else case.seg_q.numpy(),
                             seg_k=None if case.seg_k is None else case.seg_k.numpy(),
                             q_norm_w=None if wq is None else W.to_bits(wq),
                             k_norm_w=None if wk is None else W.to_bits(wk), norm_eps=1e-6)
    assert_parity(dtype, o, ref, f"rms norm {cfg}")


# --------------------------------------------------------------------------
# short rows: one launch per execute (K rotated in the attention kernel)
# --------------------------------------------------------------------------

SHORT_CFGS = [
    # dtype, B, Hq, Hkv, S, D, kind, style, norms, pe_attn_head
    ("bf16", 2, 16, 2, 16, 128, W.MASK_NONE, "interleaved", "", -1),
    ("bf16", 2, 16, 2, 64, 128, W.MASK_NONE, "half", "", -1),
    ("f16", 2, 4, 4, 33, 64, W.MASK_BOOL, "interleaved", "", 1),      # RoPE on head 0 only
    ("bf16", 1, 8, 2, 50, 128, W.MASK_SEGMENT, "interleaved", "qk", -1),
    ("f16", 2, 8, 1, 64, 64, W.MASK_CAUSAL, "half", "k", -1),
    ("bf16", 3, 2, 2, 1, 128, W.MASK_BOOL, "half", "q", -1),
    ("bf16", 2, 4, 4, 40, 128, W.MASK_NONE, "interleaved", "k", 0),   # no RoPE, k normalised
]


def _short_case(cfg):
    dtype, B, Hq, Hkv, S, D, kind, style, norms, pe = cfg
    seed = zlib.crc32(repr(("short",) + cfg).encode()) % 10000
    case = W.random_fwd(seed, B, Hq, Hkv, S, S, D, dtype, kind, rope_base=1e4, pe_attn_head=pe, mask_shape="key",
                        n_segments=2)
    case.rope_style = style
    cast = W.DTYPES[dtype]
    gen = torch.Generator().manual_seed(seed + 1)
    wq = (1.0 + 0.5 * torch.randn(D, generator=gen)).to(cast) if "q" in norms else None
    wk = (1.0 + 0.5 * torch.randn(D, generator=gen)).to(cast) if "k" in norms else None
    return case, wq, wk


def _run_short(case, wq, wk, pos_k=None):
    import masked_bidirectional_attention_amd as mz
    kw = dict(rope_base=case.rope_base, pe_attn_head=case.pe_attn_head, rope_style=case.rope_style,
              q_norm_weight=dev(wq), k_norm_weight=dev(wk), pos_k=dev(pos_k))
    if case.mask_kind == W.MASK_BOOL:
        kw["mask"] = dev(case.mask)
    elif case.mask_kind == W.MASK_SEGMENT:
        kw["seg_q"], kw["seg_k"] = dev(case.seg_q), dev(case.seg_k)
    elif case.mask_kind == W.MASK_CAUSAL:
        kw["causal"] = True
    o = mz.mzattn_fwd(dev(case.q), dev(case.k), dev(case.v), **kw)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("cfg", SHORT_CFGS, ids=lambda c: "-".join(map(str, c)))
def test_short_rows_one_launch(cfg):
    """Rows of one key tile: the K heads are normalised and rotated in the
    attention kernel (no K pass).  Parity with the oracle, and the same bits
    as the K-pass path, which an explicit key position array (here the
    default positions written out) selects."""
    case, wq, wk = _short_case(cfg)
    o = _run_short(case, wq, wk)
    ref, _ = mzref.mzref_fwd(case.dtype, W.to_bits(case.q), W.to_bits(case.k), W.to_bits(case.v),
                             rope_base=case.rope_base, pe_attn_head=case.pe_attn_head, rope_style=case.rope_style,
                             mask_kind=case.mask_kind, mask=None if case.mask is None else case.mask.numpy(),
                             seg_q=None if case.seg_q is None else case.seg_q.numpy(),
                             seg_k=None if case.seg_k is None else case.seg_k.numpy(),
                             q_norm_w=None if wq is None else W.to_bits(wq),
                             k_norm_w=None if wk is None else W.to_bits(wk))
    assert_parity(case.dtype, o, ref, f"short {cfg}")
    if case.mask_kind != W.MASK_SEGMENT:   # (segment positions restart: not the default arange)
        B, S = case.q.shape[0], case.k.shape[2]
        pos_k = torch.arange(S, dtype=torch.int32)[None].repeat(B, 1)
        o_pass = _run_short(case, wq, wk, pos_k=pos_k)
        assert torch.equal(o, o_pass), "one-launch path differs from the K-pass path"


@pytest.mark.parametrize("S", [16, 64, 200])
def test_fwd_graph_replay(S):
    """FwdCall.execute recorded once in a HIP graph (plan outside) and
    replayed with new inputs written in place between replays (eager work
    in between): every replay equals an eager call on the same inputs, bit
    for bit.  16 and 64 tokens take the one-launch path, 200 the K pass."""
    import masked_bidirectional_attention_amd as mz
    B, Hq, Hkv, D = 2, 16, 2, 128
    s = torch.cuda.Stream()
    cases = [W.random_fwd(900 + S + i, B, Hq, Hkv, S, S, D, "bf16", W.MASK_NONE, rope_base=1e4) for i in range(3)]
    q, k, v = dev(cases[0].q), dev(cases[0].k), dev(cases[0].v)
    call = mz.FwdCall(q, k, v, rope_base=1e4, stream=s)
    with torch.cuda.stream(s):
        call.plan()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call.execute()
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        q.copy_(dev(c.q))
        k.copy_(dev(c.k))
        v.copy_(dev(c.v))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_graph = call.out.clone()
        o_eager = run_fwd(c)
        assert torch.equal(o_graph, o_eager), f"replay {i}"
        if i == 0:
            ref, _ = oracle_fwd(c)
            assert_parity("bf16", o_graph, ref, f"graph replay S={S}")


def test_fwd_repeated_calls_share_poisoned_workspace():
    """Forward calls of every mask kind, dtype and size class (one-launch
    short rows, the K pass, a broadcast mask, segments of one row, causal,
    fp32) through one workspace that starts as all-ones bytes, twice over in
    opposite orders, each checked against the oracle: nothing a call reads
    from its workspace (plan, positions, key bits, rotated K) may be left
    from before it."""
    import masked_bidirectional_attention_amd as mz
    cases = [
        W.random_fwd(70, 2, 16, 2, 300, 300, 128, "bf16", W.MASK_BOOL, mask_shape="full", rope_base=1e6),
        W.random_fwd(71, 1, 8, 2, 40, 40, 128, "bf16", W.MASK_NONE, rope_base=1e4),
        W.random_fwd(72, 2, 8, 8, 257, 513, 64, "f16", W.MASK_BOOL, mask_shape="key", rope_base=1e4,
                     pe_attn_head=1),
        W.random_fwd(73, 2, 4, 2, 600, 600, 128, "bf16", W.MASK_SEGMENT, rope_base=1e4, n_segments=5),
        W.random_fwd(74, 1, 4, 1, 200, 200, 128, "bf16", W.MASK_CAUSAL, rope_base=1e4),
        W.random_fwd(75, 2, 4, 2, 129, 65, 64, "f32", W.MASK_BOOL, mask_shape="blocky", rope_base=1e4),
        W.random_fwd(76, 3, 8, 1, 64, 64, 128, "f16", W.MASK_SEGMENT, rope_base=1e4, n_segments=2),
    ]
    ws = torch.full((64 << 20,), 255, dtype=torch.uint8, device=DEV)
    for rep, order in enumerate((cases, cases[::-1])):
        for c in order:
            kw = dict(scale=c.scale, rope_base=c.rope_base, pe_attn_head=c.pe_attn_head, rope_style=c.rope_style,
                      pos_q=dev(c.pos_q), pos_k=dev(c.pos_k), return_lse=True, workspace=ws)
            if c.mask_kind == W.MASK_BOOL:
                kw["mask"] = dev(c.mask)
            elif c.mask_kind == W.MASK_SEGMENT:
                kw["seg_q"], kw["seg_k"] = dev(c.seg_q), dev(c.seg_k)
            elif c.mask_kind == W.MASK_CAUSAL:
                kw["causal"] = True
            call = mz.FwdCall(dev(c.q), dev(c.k), dev(c.v), **kw)
            assert call.workspace_bytes <= ws.numel()
            o, lse = call()
            torch.cuda.synchronize()
            ref, lse_ref = oracle_fwd(c)
            assert_parity(c.dtype, o, ref, f"{c.name} pass {rep}")
            fin = np.isfinite(lse_ref)
            assert np.array_equal(np.isfinite(to64(lse)), fin)
            np.testing.assert_allclose(to64(lse)[fin], lse_ref[fin], atol=1e-4 if c.dtype == "f32" else 3e-2)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("shape", [(2, 4, 2, 100, 140, 128), (2, 16, 2, 16, 16, 128), (1, 8, 1, 40, 64, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_query_positions_past_the_table(dtype, style, shape):
    """Explicit query positions, some inside the cos/sin table (which covers
    max(Sq, Sk) positions) and some far past it, in both pairings: a wave
    whose positions all lie in the table reads it, any other wave takes the
    direct formula for its lanes past it.  Rows of one key tile (the last
    two shapes) take the one-launch path (key positions default)."""
    import masked_bidirectional_attention_amd as mz
    B, Hq, Hkv, Sq, Sk, D = shape
    seed = zlib.crc32(repr((dtype, style, shape)).encode()) % 10000
    case = W.random_fwd(seed, B, Hq, Hkv, Sq, Sk, D, dtype, W.MASK_NONE, rope_base=1e4)
    rng = np.random.default_rng(seed)
    pos_q = rng.integers(0, max(Sq, Sk), size=(B, Sq)).astype(np.int32)
    far = rng.random((B, Sq)) < 0.3
    pos_q[far] = rng.integers(5000, 60000, size=int(far.sum()))
    pos_q[0, :min(Sq, 32)] = np.arange(min(Sq, 32))   # one wave wholly inside the table
    pq = torch.from_numpy(pos_q)
    o = mz.mzattn_fwd(dev(case.q), dev(case.k), dev(case.v), rope_base=1e4, rope_style=style, pos_q=dev(pq))
    torch.cuda.synchronize()
    ref, _ = mzref.mzref_fwd(dtype, W.to_bits(case.q), W.to_bits(case.k), W.to_bits(case.v), rope_base=1e4,
                             rope_style=style, pos_q=pos_q, pos_k=np.arange(Sk, dtype=np.int32)[None].repeat(B, 0))
    assert_parity(dtype, o, ref, f"positions past the table {style} {shape}")


def test_device_info():
    """The device query names the part the measurements run on."""
    import masked_bidirectional_attention_amd as mz
    info = mz.mzattn_device_info(0)
    props = torch.cuda.get_device_properties(0)
    assert info["compute_units"] == props.multi_processor_count > 0
    assert info["arch"].split(":")[0] == props.gcnArchName.split(":")[0]
    assert info["clock_mhz"] > 0 and info["mem_clock_mhz"] > 0
    with pytest.raises(mz.MzattnError):
        mz.mzattn_device_info(torch.cuda.device_count())
    # the failed query leaves no HIP error behind for the next launch
    case = W.random_fwd(95, 1, 2, 1, 20, 30, 64, "bf16", rope_base=1e4)
    assert_parity("bf16", run_fwd(case), oracle_fwd(case)[0], "launch after a failed device query")
