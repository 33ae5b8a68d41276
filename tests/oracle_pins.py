"""Pins of the fp64 oracle to things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees
with: a library routine it does not call (numpy's float16, torch's
bfloat16 upcast, torch's CPU scaled_dot_product_attention), a closed form
of softmax attention, a complex-number form of the rotation, or an
invariant the pages state (masked keys add exact zeros; a packed
block-diagonal row equals the rows run alone; cutting the key span past
the last live key changes nothing).

``test_oracle_pins.py`` runs every pin on the oracle as written;
``test_oracle_mutants.py`` plants plausible mistakes in the oracle and
checks that some pin fails for each of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from oracle import mzref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# --------------------------------------------------------------------------
# helpers (test side only)
# --------------------------------------------------------------------------


def _bits64(x: np.ndarray):
    """fp64 values that are exact fp32 numbers -> uint32 fp32 bits."""
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32).astype(np.float64)


def _sdpa(q, k, v, mask=None, scale=None, gqa=False):
    """torch CPU SDPA in fp64 (library routine, not used by the oracle)."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    tm = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask))
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=scale, enable_gqa=gqa)
    return out.numpy()


def _close(a, b, tol=1e-12, what=""):
    a, b = np.asarray(a), np.asarray(b)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert err <= tol * scale, f"{what}: max |diff| {err:.3e} > {tol:.1e} * {scale:.3g}"


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------


def pin_fp16_decode():
    """All 65 536 binary16 patterns against numpy's float16 (a library
    routine) upcast to fp64."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = mzref.decode_fp16(bits)
    lib = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan), "fp16 NaN set differs"
    assert np.array_equal(ours[~nan], lib[~nan]), "fp16 values differ"
    # signed zero must survive
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def pin_bf16_decode():
    """All 65 536 bfloat16 patterns against torch's exact bf16 -> fp64."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = mzref.decode_bf16(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan), "bf16 NaN set differs"
    assert np.array_equal(ours[~nan], lib[~nan]), "bf16 values differ"


def pin_fp32_decode():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1000).astype(np.float32)
    assert np.array_equal(mzref.decode_fp32(x.view(np.uint32)), x.astype(np.float64))


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------


def pin_rope_complex_form():
    """Interleaved RoPE equals multiplying the complex numbers
    x_2i + 1j*x_2i+1 by exp(1j * pos * theta_i), theta_i = 1 / base^(2i/D)
    (frequencies written from the even indices 0, 2, ..., D-2)."""
    rng = np.random.default_rng(2)
    for D, base in ((8, 10000.0), (64, 1e4), (128, 1e6)):
        S = 37
        x = _rand(rng, S, D)
        pos = rng.integers(0, 5000, size=S)
        even = np.arange(0, D, 2, dtype=np.float64)
        theta = 1.0 / (base ** (even / D))
        z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * pos[:, None] * theta[None, :])
        ref = np.empty_like(x)
        ref[:, 0::2], ref[:, 1::2] = z.real, z.imag
        _close(mzref.rope_interleaved(x, pos, base), ref, 1e-12, f"rope D={D}")


def pin_rope_hand_values():
    """Worked example (tests/golden/rope_worked_example.json): D = 4 and
    base = 100 give theta = (1, 100^(-1/2)) = (1, 1/10), so at position 3
    the two pairs of x = (1, 2, 3, 4) turn by 3 rad and 0.3 rad."""
    with open(os.path.join(GOLDEN, "rope_worked_example.json")) as f:
        g = json.load(f)
    base, pos = float(g["base"]), int(g["pos"])
    theta = [1.0, 1.0 / math.sqrt(base)]
    _close(mzref.rope_inv_freq(g["D"], base), theta, 1e-15, "theta")
    x = np.array(g["x"], dtype=np.float64)
    a0, a1 = pos * theta[0], pos * theta[1]
    exp = [x[0] * math.cos(a0) - x[1] * math.sin(a0),
           x[1] * math.cos(a0) + x[0] * math.sin(a0),
           x[2] * math.cos(a1) - x[3] * math.sin(a1),
           x[3] * math.cos(a1) + x[2] * math.sin(a1)]
    got = mzref.rope_interleaved(x[None], np.array([pos]), base)[0]
    _close(got, exp, 1e-14, "rope worked example")


def pin_rope_properties():
    """p = 0 is the identity; each pair keeps its norm; scores depend only
    on the position difference (shift every position by c)."""
    rng = np.random.default_rng(3)
    D, base = 64, 1e4
    x = _rand(rng, 9, D)
    assert np.array_equal(mzref.rope_interleaved(x, np.zeros(9), base), x)
    pos = rng.integers(0, 3000, size=9)
    r = mzref.rope_interleaved(x, pos, base)
    _close(r[:, 0::2] ** 2 + r[:, 1::2] ** 2, x[:, 0::2] ** 2 + x[:, 1::2] ** 2, 1e-12, "pair norm")
    q, k = _rand(rng, 5, D), _rand(rng, 7, D)
    pq, pk = rng.integers(0, 1000, 5), rng.integers(0, 1000, 7)
    s1 = mzref.rope_interleaved(q, pq, base) @ mzref.rope_interleaved(k, pk, base).T
    s2 = mzref.rope_interleaved(q, pq + 777, base) @ mzref.rope_interleaved(k, pk + 777, base).T
    _close(s1, s2, 1e-9, "relative position")


# --------------------------------------------------------------------------
# attention core
# --------------------------------------------------------------------------


def pin_sdpa_bool_masks():
    """Oracle (no RoPE) against torch's CPU SDPA in fp64 with boolean masks
    of several broadcast shapes, GQA through enable_gqa, default and
    explicit scale; rows with at least one live key."""
    rng = np.random.default_rng(4)
    for (B, Hq, Hkv, Sq, Sk, D, mshape, scale) in (
        (2, 4, 4, 13, 17, 8, (2, 4, 13, 17), 0.0),
        (2, 6, 2, 9, 21, 16, (2, 1, 9, 21), 0.3),
        (1, 8, 1, 5, 40, 32, (1, 1, 1, 40), 0.0),
        (3, 4, 2, 16, 16, 64, (3, 4, 16, 16), 0.125),
    ):
        q, k, v = _rand(rng, B, Hq, Sq, D), _rand(rng, B, Hkv, Sk, D), _rand(rng, B, Hkv, Sk, D)
        m = rng.random(mshape) < 0.6
        m[..., 0] = True  # every row keeps a live key, so SDPA is defined
        o, _ = mzref.mzref_fwd("f32", _bits64(q), _bits64(k), _bits64(v), scale=scale,
                               mask_kind="bool", mask=m)
        ref = _sdpa(q, k, v, m, scale if scale > 0 else None, gqa=Hq != Hkv)
        _close(o, ref, 1e-12, f"sdpa {mshape}")


def _sdpa_causal(q, k, v, scale=None, gqa=False):
    """torch CPU SDPA in fp64 with is_causal (library routine)."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    return F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale, enable_gqa=gqa).numpy()


def pin_sdpa_causal():
    """Causal kind against torch's CPU SDPA is_causal in fp64, for square
    and non-square shapes (SDPA aligns the causal band at the top-left
    corner), with GQA and an explicit scale."""
    rng = np.random.default_rng(21)
    for (B, Hq, Hkv, Sq, Sk, D, scale) in ((2, 4, 4, 13, 13, 8, 0.0), (1, 6, 2, 9, 21, 16, 0.3),
                                           (2, 4, 1, 20, 7, 32, 0.0), (1, 2, 2, 1, 5, 8, 0.0)):
        q, k, v = _rand(rng, B, Hq, Sq, D), _rand(rng, B, Hkv, Sk, D), _rand(rng, B, Hkv, Sk, D)
        o, _ = mzref.mzref_fwd("f32", _bits64(q), _bits64(k), _bits64(v), scale=scale, mask_kind="causal")
        ref = _sdpa_causal(q, k, v, scale if scale > 0 else None, gqa=Hq != Hkv)
        _close(o, ref, 1e-12, f"sdpa causal {Sq}x{Sk}")


def pin_causal_first_query_is_v0():
    """Closed form: query 0 sees key 0 alone, so its output is v_0 exactly
    and its log-sum-exp is its one score."""
    rng = np.random.default_rng(22)
    q, k, v = _rand(rng, 1, 2, 6, 8), _rand(rng, 1, 2, 9, 8), _rand(rng, 1, 2, 9, 8)
    o, lse = mzref.mzref_fwd("f32", _bits64(q), _bits64(k), _bits64(v), mask_kind="causal")
    assert np.array_equal(o[0, :, 0], v[0, :, 0])
    _close(lse[0, :, 0], np.einsum("hd,hd->h", q[0, :, 0], k[0, :, 0]) / math.sqrt(8), 1e-12, "causal lse q0")


def pin_rope_half_split_vs_transformers():
    """Half-split pairing against transformers' Llama rotary helper
    (``apply_rotary_pos_emb`` with ``rotate_half``; a library routine the
    oracle does not call), in fp64, cos/sin built as that model family
    builds them: the frequency vector repeated twice."""
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    rng = np.random.default_rng(23)
    for D, base in ((8, 1e4), (64, 1e6), (128, 1e4)):
        x, y = _rand(rng, 2, 3, 7, D), _rand(rng, 2, 3, 7, D)
        pos = np.array([0, 1, 5, 77, 1000, 2047, 4095])
        inv = 1.0 / (base ** (np.arange(0, D, 2, dtype=np.float64) / D))
        emb = np.concatenate([np.outer(pos, inv)] * 2, axis=-1)
        cos, sin = torch.from_numpy(np.cos(emb))[None], torch.from_numpy(np.sin(emb))[None]
        rx, ry = apply_rotary_pos_emb(torch.from_numpy(x), torch.from_numpy(y), cos, sin)
        _close(mzref.rope_half_split(x, pos, base), rx.numpy(), 1e-12, f"half split D{D} q")
        _close(mzref.rope_half_split(y, pos, base), ry.numpy(), 1e-12, f"half split D{D} k")


def pin_rope_styles_differ_by_permutation():
    """The two pairings are one rotation seen through a fixed permutation of
    the feature axis (even features first, then odd), so attention with
    half-split RoPE equals attention with interleaved RoPE on permuted q/k."""
    rng = np.random.default_rng(24)
    B, H, S, D = 1, 2, 9, 16
    q, k, v = _rand(rng, B, H, S, D), _rand(rng, B, H, S, D), _rand(rng, B, H, S, D)
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])  # interleaved -> half-split layout
    inv = np.argsort(perm)
    o_half, _ = mzref.mzref_fwd("f32", _bits64(q), _bits64(k), _bits64(v), rope_base=1e4, rope_style="half")
    o_int, _ = mzref.mzref_fwd("f32", _bits64(q[..., inv]), _bits64(k[..., inv]), _bits64(v), rope_base=1e4)
    _close(o_half, o_int, 1e-12, "styles by permutation")


def pin_sdpa_no_mask():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 2, 4, 11, 32), _rand(rng, 2, 4, 19, 32), _rand(rng, 2, 4, 19, 32)
    o, _ = mzref.mzref_fwd("f32", _bits64(q), _bits64(k), _bits64(v))
    _close(o, _sdpa(q, k, v), 1e-12, "sdpa no mask")


def pin_drop_masked_keys():
    """Every mask pattern over 3 queries x 3 keys (2^9): the masked result
    equals unmasked SDPA over the gathered live keys of each row, and a row
    with no live key gives 0 (the library's contract)."""
    rng = np.random.default_rng(6)
    D = 4
    q, k, v = _rand(rng, 3, D), _rand(rng, 3, D), _rand(rng, 3, D)
    for code in range(512):
        m = np.array([(code >> b) & 1 for b in range(9)], dtype=bool).reshape(3, 3)
        o, lse = mzref.attend(q, k, v, m, 0.5)
        for i in range(3):
            J = np.nonzero(m[i])[0]
            if J.size == 0:
                assert np.all(o[i] == 0) and lse[i] == -np.inf, "empty row"
                continue
            ref = _sdpa(q[i:i + 1][None, None], k[J][None, None], v[J][None, None], scale=0.5)[0, 0, 0]
            _close(o[i], ref, 1e-13, f"mask {code:03x} row {i}")
            s = 0.5 * k[J] @ q[i]
            _close(lse[i], math.log(np.sum(np.exp(s))), 1e-13, "lse")


def pin_closed_forms():
    """One live key -> exactly v_j with lse = s_j; equal scores -> mean of
    the live V rows; two live keys -> sigmoid weights; large scores do not
    overflow (the max is subtracted first)."""
    rng = np.random.default_rng(7)
    D = 16
    q, k, v = _rand(rng, 4, D), _rand(rng, 10, D), _rand(rng, 10, D)
    m = np.zeros((4, 10), dtype=bool)
    m[0, 3] = m[1, 9] = m[2, 0] = m[3, 5] = True
    o, lse = mzref.attend(q, k, v, m, 0.7)
    for i, j in enumerate((3, 9, 0, 5)):
        assert np.array_equal(o[i], v[j]), "single live key must return v_j exactly"
        _close(lse[i], 0.7 * float(q[i] @ k[j]), 1e-14, "lse single")
    # equal scores
    m = rng.random((4, 10)) < 0.5
    m[:, 1] = True
    o, _ = mzref.attend(np.zeros((4, D)), k, v, m, 1.0)
    for i in range(4):
        _close(o[i], v[m[i]].mean(axis=0), 1e-14, "mean of live V")
    o, _ = mzref.attend(q, k, v, m, 0.0)
    _close(o, np.stack([v[m[i]].mean(axis=0) for i in range(4)]), 1e-14, "scale 0")
    # two keys, and large scores
    with open(os.path.join(GOLDEN, "two_key_softmax.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        qq = np.array(case["q"], dtype=np.float64)[None]
        kk = np.array(case["k"], dtype=np.float64)
        vv = np.array(case["v"], dtype=np.float64)
        o, lse = mzref.attend(qq, kk, vv, np.ones((1, 2), dtype=bool), case["scale"])
        s0, s1 = (case["scale"] * float(kk[j] @ qq[0]) for j in (0, 1))
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        _close(o[0], w0 * vv[0] + (1 - w0) * vv[1], 1e-13, case["name"])
        big = max(s0, s1)
        _close(lse[0], big + math.log1p(math.exp(min(s0, s1) - big)), 1e-13, case["name"] + " lse")


def pin_key_permutation():
    """Permuting keys (with their values and mask columns) leaves every
    output unchanged."""
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 6, 8), _rand(rng, 15, 8), _rand(rng, 15, 8)
    m = rng.random((6, 15)) < 0.6
    perm = rng.permutation(15)
    o1, l1 = mzref.attend(q, k, v, m, 0.4)
    o2, l2 = mzref.attend(q, k[perm], v[perm], m[:, perm], 0.4)
    _close(o1, o2, 1e-13, "permutation")
    _close(l1, l2, 1e-13, "permutation lse")


def pin_masked_garbage():
    """Masked positions add exact zeros (VoxCPM page, attention bullet):
    finite junk in masked K/V leaves outputs bit-identical."""
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 5, 8), _rand(rng, 12, 8), _rand(rng, 12, 8)
    m = rng.random((5, 12)) < 0.5
    m[:, 0] = True
    k2, v2 = k.copy(), v.copy()
    dead = ~m.any(axis=0)
    k2[dead] = 1e3 * _rand(rng, int(dead.sum()), 8)
    v2[dead] = -1e3 * _rand(rng, int(dead.sum()), 8)
    o1, _ = mzref.attend(q, k, v, m, 0.5)
    o2, _ = mzref.attend(q, k2, v2, m, 0.5)
    assert np.array_equal(o1, o2), "masked junk changed the output"


def pin_gqa_is_repeat():
    """GQA equals plain multi-head attention over K/V heads each repeated
    G times in a row."""
    rng = np.random.default_rng(10)
    B, Hq, Hkv, S, D = 2, 8, 2, 11, 16
    q, k, v = _rand(rng, B, Hq, S, D), _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D)
    o1, _ = mzref.mzref_fwd("f32", _bits64(q), _bits64(k), _bits64(v), rope_base=1e4)
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    o2, _ = mzref.mzref_fwd("f32", _bits64(q), _bits64(kr), _bits64(vr), rope_base=1e4)
    _close(o1, o2, 1e-13, "gqa")


def pin_partial_rope_heads():
    """pe_attn_head = n rotates exactly the first n heads; 0 equals no
    RoPE; a negative value rotates every head."""
    rng = np.random.default_rng(11)
    B, H, S, D = 1, 4, 9, 8
    q, k, v = _rand(rng, B, H, S, D), _rand(rng, B, H, S, D), _rand(rng, B, H, S, D)
    bq, bk, bv = _bits64(q), _bits64(k), _bits64(v)
    none, _ = mzref.mzref_fwd("f32", bq, bk, bv)
    allr, _ = mzref.mzref_fwd("f32", bq, bk, bv, rope_base=1e4, pe_attn_head=-1)
    one, _ = mzref.mzref_fwd("f32", bq, bk, bv, rope_base=1e4, pe_attn_head=1)
    zero, _ = mzref.mzref_fwd("f32", bq, bk, bv, rope_base=1e4, pe_attn_head=0)
    assert np.array_equal(zero, none)
    assert np.array_equal(one[:, 0], allr[:, 0]) and np.array_equal(one[:, 1:], none[:, 1:])
    assert not np.allclose(allr[:, 0], none[:, 0])
    # rotation applied to q and k heads, checked against SDPA on rotated inputs
    pos = np.arange(S)
    qr = mzref.rope_interleaved(q[0, 0], pos, 1e4)[None, None]
    kr = mzref.rope_interleaved(k[0, 0], pos, 1e4)[None, None]
    _close(one[:, :1], _sdpa(qr, kr, v[:, :1]), 1e-12, "rope head 0 vs sdpa")


def pin_packed_equals_separate():
    """OmniVoice page, 'Memory and speed': two rows packed side by side
    under a block-diagonal mask, positions restarting at 0 per block, give
    what each row gives alone (segment mode and the explicit boolean
    block-diagonal mask with explicit positions both)."""
    rng = np.random.default_rng(12)
    H, Hkv, D, A, U = 4, 2, 16, 23, 9
    q, k, v = _rand(rng, 2, H, A, D), _rand(rng, 2, Hkv, A, D), _rand(rng, 2, Hkv, A, D)
    row1_mask = np.zeros((1, 1, A, A), dtype=bool)
    row1_mask[..., :U, :U] = True
    sep0, _ = mzref.mzref_fwd("f32", _bits64(q[:1]), _bits64(k[:1]), _bits64(v[:1]), rope_base=1e6)
    sep1, _ = mzref.mzref_fwd("f32", _bits64(q[1:]), _bits64(k[1:]), _bits64(v[1:]), rope_base=1e6,
                              mask_kind="bool", mask=row1_mask)

    def pack(x):
        return np.concatenate([x[0:1], x[1:2, :, :U]], axis=2)

    pq, pk, pv = pack(q), pack(k), pack(v)
    seg = np.concatenate([np.zeros(A, np.int32), np.ones(U, np.int32)])[None]
    po, _ = mzref.mzref_fwd("f32", _bits64(pq), _bits64(pk), _bits64(pv), rope_base=1e6,
                            mask_kind="segment", seg_q=seg, seg_k=seg)
    _close(po[:, :, :A], sep0, 1e-13, "packed segment 0")
    _close(po[:, :, A:], sep1[:, :, :U], 1e-13, "packed segment 1")
    bd = np.zeros((1, 1, A + U, A + U), dtype=bool)
    bd[..., :A, :A] = True
    bd[..., A:, A:] = True
    pos = np.concatenate([np.arange(A), np.arange(U)])[None].astype(np.int32)
    po2, _ = mzref.mzref_fwd("f32", _bits64(pq), _bits64(pk), _bits64(pv), rope_base=1e6,
                             mask_kind="bool", mask=bd, pos_q=pos, pos_k=pos)
    _close(po2, po, 1e-13, "bool block-diagonal vs segment")


def pin_segment_positions():
    seg = np.array([-1, -1, 0, 0, 0, 3, 7, 7, 7, 7])
    assert list(mzref.segment_positions(seg)) == [0, 1, 0, 1, 2, 0, 0, 1, 2, 3]


def pin_segment_padding():
    """Padding ids (< 0) never attend and are never attended to."""
    seg = np.array([[-1, -1, 0, 0, 1, 1, 1]])
    live = mzref.live_set_fwd(1, 1, 7, 7, "segment", seg_q=seg, seg_k=seg)[0, 0]
    exp = np.zeros((7, 7), dtype=bool)
    exp[2:4, 2:4] = True
    exp[4:, 4:] = True
    assert np.array_equal(live, exp)


# --------------------------------------------------------------------------
# static-cache decode
# --------------------------------------------------------------------------


def pin_decode_vs_sdpa_truncated():
    """A decode step equals SDPA (GQA) over the first ``span`` keys with the
    mask's live columns; span cutting through live keys drops exactly those
    keys."""
    rng = np.random.default_rng(13)
    B, Hq, Hkv, T, C, D = 2, 8, 2, 3, 300, 32
    q, k, v = _rand(rng, B, Hq, T, D), _rand(rng, B, Hkv, C, D), _rand(rng, B, Hkv, C, D)
    m = rng.random((B, 1, T, C)) < 0.8
    m[..., 0] = True
    for span in (1, 77, 256, 300):
        o = mzref.mzref_decode("f32", _bits64(q), _bits64(k), _bits64(v), span=span, mask=m)
        ref = _sdpa(q, k[:, :, :span], v[:, :, :span], m[..., :span], gqa=True)
        _close(o, ref, 1e-12, f"decode span {span}")


def pin_decode_span_invariance():
    """VoxCPM page, attention bullet: with every key at or past L masked,
    any span >= L gives the same result (the full cache, the next multiple
    of 256, or L itself); in the oracle this holds bit for bit."""
    rng = np.random.default_rng(14)
    B, Hq, Hkv, C, D, L = 1, 4, 1, 1024, 16, 300
    q, k, v = _rand(rng, B, Hq, 1, D), _rand(rng, B, Hkv, C, D), _rand(rng, B, Hkv, C, D)
    m = np.zeros((B, 1, 1, C), dtype=bool)
    m[..., :L] = True
    outs = [mzref.mzref_decode("f32", _bits64(q), _bits64(k), _bits64(v), span=s, mask=m)
            for s in (L, 512, 1024)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def pin_decode_rope_q():
    """Decode with q RoPE at q_pos equals decode of the pre-rotated q."""
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 1, 2, 2, 16), _rand(rng, 1, 1, 64, 16), _rand(rng, 1, 1, 64, 16)
    pos = np.array([[5, 900]])
    o = mzref.mzref_decode("f32", _bits64(q), _bits64(k), _bits64(v), span=64, rope_base=1e4, q_pos=pos)
    qr = np.stack([mzref.rope_interleaved(q[0, h], pos[0], 1e4) for h in range(2)])[None]
    ref = _sdpa(qr, np.repeat(k, 2, 1), np.repeat(v, 2, 1))
    _close(o, ref, 1e-12, "decode rope")


def _rope_complex(x, pos, base):
    """Interleaved rotation as complex multiplication (test-side, written
    from the definition; x [..., S, D], pos [S])."""
    D = x.shape[-1]
    theta = 1.0 / (base ** (np.arange(0, D, 2, dtype=np.float64) / D))
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * np.asarray(pos, dtype=np.float64)[:, None] * theta)
    out = np.empty_like(x)
    out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


def pin_append_empty_cache_is_causal_sdpa():
    """Appending q_len tokens to an empty cache (len 0) is causal attention
    over the new tokens: torch SDPA is_causal (GQA) over q and k rotated at
    positions 0 .. q_len-1 (complex form); the rows written are those
    rotated keys."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, T, C, D = 2, 4, 2, 5, 40, 16
    q, kn, vn = _rand(rng, B, Hq, T, D), _rand(rng, B, Hkv, T, D), _rand(rng, B, Hkv, T, D)
    kc, vc = _rand(rng, B, Hkv, C, D), _rand(rng, B, Hkv, C, D)   # junk past the filled rows
    o, k_rows, ovf = mzref.mzref_decode_append("f32", _bits64(q), _bits64(kn), _bits64(vn), _bits64(kc),
                                               _bits64(vc), [0, 0], rope_base=1e4)
    pos = np.arange(T)
    qr, kr = _rope_complex(q, pos, 1e4), _rope_complex(kn, pos, 1e4)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)) for a in (qr, kr, vn))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True).numpy()
    _close(o, ref, 1e-12, "append on empty cache")
    _close(k_rows, kr, 1e-12, "appended key rows")
    assert not ovf.any()


def pin_append_single_token_first_row():
    """One new token on an empty cache is the only live key of its query:
    the output is its value exactly (p = 1, l = 1)."""
    rng = np.random.default_rng(32)
    q, kn, vn = _rand(rng, 1, 4, 1, 8), _rand(rng, 1, 2, 1, 8), _rand(rng, 1, 2, 1, 8)
    kc, vc = _rand(rng, 1, 2, 20, 8), _rand(rng, 1, 2, 20, 8)
    o, _, _ = mzref.mzref_decode_append("f32", _bits64(q), _bits64(kn), _bits64(vn), _bits64(kc), _bits64(vc),
                                        [0], rope_base=1e4)
    assert np.array_equal(o[0, :, 0], np.repeat(vn[0, :, 0], 2, axis=0))


def pin_append_equals_sdpa_on_updated_cache():
    """Rows of different filled lengths with a user mask: equals SDPA (GQA)
    with the bool mask (j <= len + t) & mask over a cache whose rows
    len .. len+T-1 hold the new keys rotated at those positions (complex
    form) and the new values."""
    rng = np.random.default_rng(33)
    B, Hq, Hkv, T, C, D = 3, 6, 2, 3, 50, 16
    lens = np.array([0, 17, 47])
    q, kn, vn = _rand(rng, B, Hq, T, D), _rand(rng, B, Hkv, T, D), _rand(rng, B, Hkv, T, D)
    kc, vc = _rand(rng, B, Hkv, C, D), _rand(rng, B, Hkv, C, D)
    um = rng.random((B, Hq, T, C)) < 0.7
    for b in range(B):
        for t in range(T):
            um[b, :, t, lens[b] + t] = True
    o, _, ovf = mzref.mzref_decode_append("f32", _bits64(q), _bits64(kn), _bits64(vn), _bits64(kc), _bits64(vc),
                                          lens, mask=um, rope_base=1e4)
    assert not ovf.any()
    k2, v2 = kc.copy(), vc.copy()
    qr = np.empty_like(q)
    live = np.zeros((B, Hq, T, C), dtype=bool)
    for b in range(B):
        pos = lens[b] + np.arange(T)
        k2[b, :, lens[b]:lens[b] + T] = _rope_complex(kn[b], pos, 1e4)
        v2[b, :, lens[b]:lens[b] + T] = vn[b]
        qr[b] = _rope_complex(q[b], pos, 1e4)
        live[b] = um[b] & (np.arange(C)[None, None, :] <= pos[None, :, None])
    _close(o, _sdpa(qr, k2, v2, live, gqa=True), 1e-12, "append vs SDPA on the updated cache")


def pin_append_overflow():
    """A row whose new tokens would run past the cache end writes nothing
    and gives 0; the last row that fits is computed."""
    rng = np.random.default_rng(34)
    T, C = 2, 10
    q, kn, vn = _rand(rng, 2, 2, T, 8), _rand(rng, 2, 1, T, 8), _rand(rng, 2, 1, T, 8)
    kc, vc = _rand(rng, 2, 1, C, 8), _rand(rng, 2, 1, C, 8)
    o, _, ovf = mzref.mzref_decode_append("f32", _bits64(q), _bits64(kn), _bits64(vn), _bits64(kc), _bits64(vc),
                                          [C - T, C - T + 1])
    assert list(ovf) == [False, True]
    assert np.all(o[1] == 0) and np.all(np.abs(o[0]) > 0)


def pin_longrope_vs_transformers():
    """LongRoPE factors and attention factor: cos / sin of the oracle with
    factors and mscale equal transformers' longrope inverse frequencies
    (short and long factor lists) and attention factor applied to
    cos / sin (library routine, not used by the oracle)."""
    import warnings
    from transformers import LlamaConfig
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    D, base = 128, 1e4
    rng = np.random.default_rng(41)
    sf = list(1.0 + rng.random(D // 2))
    lf = list(1.0 + 8.0 * rng.random(D // 2))
    cfg = LlamaConfig(hidden_size=4 * D, num_attention_heads=4, head_dim=D, max_position_embeddings=32768,
                      rope_parameters={"rope_type": "longrope", "rope_theta": base, "long_factor": lf,
                                       "short_factor": sf, "original_max_position_embeddings": 4096})
    pos = rng.integers(0, 30000, size=50)
    for seq_len, fac in ((None, sf), (10000, lf)):
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            inv, att = ROPE_INIT_FUNCTIONS["longrope"](cfg, device="cpu", seq_len=seq_len)
        inv = inv.double().numpy()
        c, s_ = mzref.rope_cos_sin(pos, D, base, "exact", np.array(fac), att)
        ang = pos[:, None].astype(np.float64) * inv[None, :]
        # transformers forms inv_freq in fp32: compare at fp32 resolution of the angle
        _close(c, np.cos(ang) * att, 2e-7 * 30000, "longrope cos")
        _close(s_, np.sin(ang) * att, 2e-7 * 30000, "longrope sin")
        assert att > 1.0


def pin_rope_fp16_angles_vs_torch():
    """fp16 angles: torch half tensors (inv_freq cast to fp16, positions as
    fp16, their product and its cos / sin in fp16) give the oracle's
    cos / sin; positions past 2048 round in fp16, so they differ from the
    exact angles."""
    D, base = 64, 1e4
    pos = np.arange(0, 4000, 7)
    inv = torch.from_numpy(mzref.rope_inv_freq(D, base)).half()
    t = torch.from_numpy(pos.astype(np.float64)).half()
    freqs = t[:, None] * inv[None, :]
    c_ref, s_ref = freqs.cos().double().numpy(), freqs.sin().double().numpy()
    c, s_ = mzref.rope_cos_sin(pos, D, base, "fp16")
    ulp = 2.0 ** -10
    assert np.all(np.abs(c - c_ref) <= ulp) and np.all(np.abs(s_ - s_ref) <= ulp)
    assert np.mean(c == c_ref) > 0.99 and np.mean(s_ == s_ref) > 0.99
    ce, _ = mzref.rope_cos_sin(pos, D, base, "exact")
    assert np.max(np.abs(ce - c)) > 0.05   # the fp16 angles are far off at large positions


def pin_rope_bf16_table_vs_torch():
    """bf16 table: fp32 angles, fp32 cos / sin times mscale, rounded to
    bf16 by torch equal the oracle's table."""
    D, base, mscale = 128, 1e6, 1.25
    pos = np.arange(0, 8192, 3)
    inv = torch.from_numpy(mzref.rope_inv_freq(D, base)).float()
    t = torch.from_numpy(pos.astype(np.float32))
    ang = t[:, None] * inv[None, :]
    c_ref = (ang.double().cos().float() * mscale).to(torch.bfloat16).double().numpy()
    s_ref = (ang.double().sin().float() * mscale).to(torch.bfloat16).double().numpy()
    c, s_ = mzref.rope_cos_sin(pos, D, base, "bf16_table", None, mscale)
    assert np.array_equal(c, c_ref) and np.array_equal(s_, s_ref)
    assert np.array_equal(mzref.round_bf16(c_ref), c_ref)


def pin_qk_rms_norm():
    """q / k RMSNorm before RoPE: the forward with norm weights equals SDPA
    over q and k normalised by torch's rms_norm (library routine) and then
    rotated (complex form)."""
    rng = np.random.default_rng(51)
    B, Hq, Hkv, S, D = 1, 4, 2, 20, 16
    f32 = lambda a: a.astype(np.float32).astype(np.float64)   # inputs exact in fp32
    q, k, v = f32(_rand(rng, B, Hq, S, D) * 3.0), f32(_rand(rng, B, Hkv, S, D) * 0.2), _rand(rng, B, Hkv, S, D)
    wq, wk = _rand(rng, D), _rand(rng, D)
    o, _ = mzref.mzref_fwd("f32", _bits64(q), _bits64(k), _bits64(v), rope_base=1e4, q_norm_w=_bits64(wq),
                           k_norm_w=_bits64(wk), norm_eps=1e-6)
    qn = F.rms_norm(torch.from_numpy(q), (D,), torch.from_numpy(wq), eps=1e-6).numpy()
    kn = F.rms_norm(torch.from_numpy(k), (D,), torch.from_numpy(wk), eps=1e-6).numpy()
    pos = np.arange(S)
    ref = _sdpa(_rope_complex(qn, pos, 1e4), _rope_complex(kn, pos, 1e4), v, gqa=True)
    _close(o, ref, 1e-12, "q/k rms norm")
    # the scale of q or k then does not matter
    o2, _ = mzref.mzref_fwd("f32", _bits64(q * 4.0), _bits64(k * 0.25), _bits64(v), rope_base=1e4,
                            q_norm_w=_bits64(wq), k_norm_w=_bits64(wk), norm_eps=0.0)
    o3, _ = mzref.mzref_fwd("f32", _bits64(q), _bits64(k), _bits64(v), rope_base=1e4,
                            q_norm_w=_bits64(wq), k_norm_w=_bits64(wk), norm_eps=0.0)
    _close(o2, o3, 1e-12, "rms norm scale invariance")


# --------------------------------------------------------------------------
# the comparison that decides every GPU parity check
# --------------------------------------------------------------------------


def pin_parity_checker():
    """``parity_stats`` / ``within_tolerance`` on synthetic outputs placed
    just inside and just outside each bound the GPU path is held to: fp32
    max |d| <= 1e-5; fp16 / bf16 relative L2 <= 4e-3 and max |d| <=
    2e-2 * max |ref| (both must hold); non-finite outputs fail; an
    all-zero reference admits only an all-zero output.  The bounds are the
    stated tolerances, so the margins here (a few tenths of a percent) are
    what a slip in the checker (an ``or`` for the ``and``, the norm or the
    maximum taken from the output instead of the reference, a bound off by
    a factor) has to survive."""
    rng = np.random.default_rng(97)
    ok = lambda dt, out, ref: mzref.within_tolerance(dt, mzref.parity_stats(out, ref))
    ref = rng.standard_normal(4096)
    # fp32: one element off by just under / just over 1e-5 (max |d| only)
    for d, want in ((0.99e-5, True), (1.01e-5, False), (-1.01e-5, False)):
        out = ref.copy()
        out[17] += d
        assert ok("f32", out, ref) is want, f"f32 bump {d}"
    # fp32: a rel-L2 far above 4e-3 with max |d| below 1e-5 still passes
    small = rng.standard_normal(64) * 1e-3
    out = small + 0.9e-5
    st = mzref.parity_stats(out, small)
    assert st["rel_l2"] > 4e-3 and ok("f32", out, small), "f32 holds max |d| only"
    for dt in ("bf16", "f16"):
        # relative L2 just under / just over 4e-3 (max |d| well inside)
        for eps, want in ((3.99e-3, True), (4.005e-3, False)):
            out = ref * (1.0 + eps)
            st = mzref.parity_stats(out, ref)
            assert abs(st["rel_l2"] - eps) < 1e-9, f"rel_l2 {st['rel_l2']} != {eps}"
            assert ok(dt, out, ref) is want, f"{dt} rel-L2 {eps}"
        # max |d| just under / just over 2e-2 * max |ref| at the largest
        # element, rel-L2 well inside (a long all-ones reference)
        big = np.ones(200000)
        big[5] = 2.0
        for frac, want in ((0.0198, True), (0.0202, False)):
            out = big.copy()
            out[5] += frac * 2.0
            st = mzref.parity_stats(out, big)
            assert st["rel_l2"] < 1e-3 and st["max_ref"] == 2.0
            assert ok(dt, out, big) is want, f"{dt} max-abs {frac}"
        # the same bump on an ordinary element is measured against max |ref|
        out = big.copy()
        out[9] += 0.0202 * 2.0
        assert not ok(dt, out, big), f"{dt} max-abs on a non-maximal element"
        # non-finite outputs fail however small the rest of the error
        for bad in (np.nan, np.inf, -np.inf):
            out = ref.copy()
            out[3] = bad
            assert not ok(dt, out, ref), f"{dt} output {bad}"
        # an all-zero reference: zero passes, anything else fails
        z = np.zeros(256)
        assert ok(dt, z.copy(), z)
        out = z.copy()
        out[0] = 1e-6
        assert not ok(dt, out, z), f"{dt} nonzero output for a zero reference"
    for bad in (np.nan, np.inf):
        out = ref.copy()
        out[3] = bad
        assert not ok("f32", out, ref), f"f32 output {bad}"
    # empty outputs (no queries) pass
    assert ok("bf16", np.zeros(0), np.zeros(0)) and ok("f32", np.zeros(0), np.zeros(0))
    # the statistics themselves, on a hand-checked case
    st = mzref.parity_stats(np.array([3.0, 4.0, 0.0]), np.array([0.0, 0.0, -2.0]))
    assert st["max_abs"] == 4.0 and st["max_ref"] == 2.0 and abs(st["rel_l2"] - math.sqrt(29.0) / 2.0) < 1e-15


ALL_PINS = [
    pin_fp16_decode, pin_bf16_decode, pin_fp32_decode,
    pin_rope_complex_form, pin_rope_hand_values, pin_rope_properties,
    pin_sdpa_bool_masks, pin_sdpa_no_mask, pin_drop_masked_keys, pin_closed_forms,
    pin_key_permutation, pin_masked_garbage, pin_gqa_is_repeat, pin_partial_rope_heads,
    pin_packed_equals_separate, pin_segment_positions, pin_segment_padding,
    pin_decode_vs_sdpa_truncated, pin_decode_span_invariance, pin_decode_rope_q,
    pin_sdpa_causal, pin_causal_first_query_is_v0,
    pin_rope_half_split_vs_transformers, pin_rope_styles_differ_by_permutation,
    pin_append_empty_cache_is_causal_sdpa, pin_append_single_token_first_row,
    pin_append_equals_sdpa_on_updated_cache, pin_append_overflow,
    pin_longrope_vs_transformers, pin_rope_fp16_angles_vs_torch, pin_rope_bf16_table_vs_torch,
    pin_qk_rms_norm, pin_parity_checker,
]
