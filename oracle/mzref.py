"""fp64 CPU oracle for masked bidirectional attention (test infrastructure).

This module is test infrastructure.  Only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it.  The HIP library never calls it and shares no code with it: this file
does its own fp16/bf16 decoding, its own RoPE and its own softmax.

What it computes, and where the pages state it
----------------------------------------------
The method on the pages is ordinary scaled-dot-product attention run
without a causal mask, under a boolean mask, inside every transformer
forward of three speech engines:

* F5-TTS page, "How it works": classifier-free guidance is a batch of
  two rows; the DiT uses interleaved rotary embedding (x-transformers
  style), and the v0 base variant ("Variants" table) rotates only the
  first ``pe_attn_head`` = 1 heads.
* OmniVoice page, "What matches upstream" (attention mask): the
  bidirectional LM gets a full 4-D boolean mask, not causal, with the K/V
  heads repeated to the query heads (GQA).
* OmniVoice page, "Memory and speed" (packed_guidance): the conditional
  row and the target-only unconditional row sit side by side in one row
  under a block-diagonal mask, each block with positions from 0, and each
  block computes what it would compute alone.
* VoxCPM page, "What matches upstream" (attention): each generation step
  attends to a static KV cache under an explicit boolean mask; masked
  positions add exact zeros, so cutting the key span anywhere past the
  last live key leaves the result unchanged.  The same bullet runs the
  prefill through SDPA with a causal mask (the ``causal`` kind here).

The oracle is the plain definition, written out in fp64 (tiling and an
online softmax are exact reformulations of it, so there is no algorithm
to follow step by step):

    live(i, j)  from the mask / segment ids / span
    s_ij = scale * <rope(q_i), rope(k_j)>          for live j only
    m_i  = max_j s_ij,  p_ij = exp(s_ij - m_i),  l_i = sum_j p_ij
    o_i  = sum_j p_ij v_j / l_i,  lse_i = m_i + ln l_i
    no live key: o_i = 0, lse_i = -inf

Readings where the pages are silent:
True in a mask means "takes part"; a query with no live key gives 0;
interleaved RoPE rotates adjacent pairs (2i, 2i+1) by pos * base^(-2i/D);
with GQA, query head h reads K/V head floor(h / G); causal follows SDPA's
is_causal, key j live for query i iff j <= i (aligned at the top-left
corner also when Sq != Sk).

Inputs are raw storage bits (uint16 for fp16/bf16, uint32 for fp32); the
oracle decodes them exactly to fp64 and never rounds afterwards.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

# --------------------------------------------------------------------------
# Storage formats
# --------------------------------------------------------------------------


def decode_fp16(bits: np.ndarray) -> np.ndarray:
    """IEEE 754 binary16 -> fp64, from the format's definition: 1 sign bit,
    5 exponent bits (bias 15), 10 fraction bits; exponent 0 is subnormal
    (fraction * 2^-24), exponent 31 is inf (fraction 0) or NaN."""
    b = np.asarray(bits).astype(np.uint32)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = ((b >> 10) & 0x1F).astype(np.int64)
    f = (b & 0x3FF).astype(np.float64)
    normal = np.ldexp(1.0 + f / 1024.0, (e - 15).astype(np.int32))
    sub = np.ldexp(f, -24)
    special = np.where(f == 0, np.inf, np.nan)
    out = np.where(e == 0, sub, np.where(e == 31, special, normal))
    return sign * out


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 -> fp64: a bf16 value is the upper half of an IEEE binary32,
    so widen the bits to 32 and read them as fp32 (exact in fp64)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def decode_fp32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits).astype(np.uint32).view(np.float32).astype(np.float64)


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return decode_fp16(bits)
    if dtype == "bf16":
        return decode_bf16(bits)
    if dtype == "f32":
        return decode_fp32(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# Rotary position embedding, interleaved pairs
# --------------------------------------------------------------------------


def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/D), i = 0 .. D/2-1 (F5-TTS page, 'How it works'
    and 'What matches upstream': the interleaved rotary embedding of
    x-transformers; frequencies as in the standard RoPE definition)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / head_dim)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to fp32 and then to bf16 (round to nearest even on
    the upper 16 bits of the fp32 pattern), returned as fp64."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def rope_cos_sin(pos, head_dim: int, base: float, precision: str = "exact", factors=None, mscale: float = 1.0):
    """cos and sin of the rotation angles, [..., S, D/2] for pos [..., S].

    theta_i = base^(-2i/D) / factors[i] (LongRoPE's per-dimension factors,
    the MiniCPM-4 LM of the VoxCPM page, 'How it works'; factors None = 1);
    mscale multiplies cos and sin (LongRoPE's attention factor).
    precision 'exact': the angle pos * theta_i and its cos / sin in fp64.
    'fp16' (F5-TTS page, 'What matches upstream': on GPU inv_freq and the
    angles are fp16): theta_i and pos rounded to fp16, their product rounded
    to fp16, cos / sin of it rounded to fp16, then times mscale (reading:
    the rounding is taken from the fp64 cos / sin; torch rounds an fp32
    one, which lands one fp16 ulp away in rare cases).
    'bf16_table' (VoxCPM page, 'What matches upstream': the LongRoPE table
    is built in fp32 and rounded with the model to bf16): the fp32 product
    of fp32 pos and fp32 theta_i, cos / sin rounded to fp32, times mscale
    in fp32, rounded to bf16."""
    theta = rope_inv_freq(head_dim, base)
    if factors is not None:
        theta = theta / np.asarray(factors, dtype=np.float64)
    p = np.asarray(pos, dtype=np.float64)[..., None]
    if precision == "exact":
        ang = p * theta
        return np.cos(ang) * mscale, np.sin(ang) * mscale
    if precision == "fp16":
        th16 = theta.astype(np.float16).astype(np.float64)
        p16 = p.astype(np.float16).astype(np.float64)
        a16 = (p16 * th16).astype(np.float16).astype(np.float64)
        c = np.cos(a16).astype(np.float16).astype(np.float64)
        s_ = np.sin(a16).astype(np.float16).astype(np.float64)
        return c * mscale, s_ * mscale
    if precision == "bf16_table":
        a32 = p.astype(np.float32) * theta.astype(np.float32)
        m32 = np.float32(mscale)
        c = np.cos(a32.astype(np.float64)).astype(np.float32) * m32
        s_ = np.sin(a32.astype(np.float64)).astype(np.float32) * m32
        return round_bf16(c), round_bf16(s_)
    raise ValueError(precision)


def rope_interleaved(x: np.ndarray, pos: np.ndarray, base: float, precision: str = "exact", factors=None,
                     mscale: float = 1.0) -> np.ndarray:
    """Rotate adjacent pairs (x_2i, x_2i+1) of every row of x [..., S, D]
    by the angle pos * theta_i, pos [S] (or broadcastable to x[..., 0])."""
    D = x.shape[-1]
    if precision == "exact" and factors is None and mscale == 1.0:
        ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(D, base)
        c, s = np.cos(ang), np.sin(ang)
    else:
        c, s = rope_cos_sin(pos, D, base, precision, factors, mscale)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x1 * c + x0 * s
    return out


def rope_half_split(x: np.ndarray, pos: np.ndarray, base: float, precision: str = "exact", factors=None,
                    mscale: float = 1.0) -> np.ndarray:
    """Rotate the pairs (x_i, x_i+D/2) of every row of x [..., S, D] by the
    angle pos * theta_i: the "rotate half" pairing of GPT-NeoX / Llama-style
    models, offered beside the interleaved one for the pages' other models.
    Same frequencies and rotation sense."""
    D = x.shape[-1]
    c, s = rope_cos_sin(pos, D, base, precision, factors, mscale)
    x0, x1 = x[..., :D // 2], x[..., D // 2:]
    out = np.empty_like(x)
    out[..., :D // 2] = x0 * c - x1 * s
    out[..., D // 2:] = x1 * c + x0 * s
    return out


def rope(x: np.ndarray, pos: np.ndarray, base: float, style: str = "interleaved", precision: str = "exact",
         factors=None, mscale: float = 1.0) -> np.ndarray:
    """The rotation of one pairing: 'interleaved' (default) or 'half', with
    the cos / sin of rope_cos_sin."""
    if style == "interleaved":
        return rope_interleaved(x, pos, base, precision, factors, mscale)
    if style == "half":
        return rope_half_split(x, pos, base, precision, factors, mscale)
    raise ValueError(style)


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis (the q / k
    normalisation of the Qwen3 LM, OmniVoice page, 'What matches upstream':
    q and k are normalised separately, as transformers does, before RoPE)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def segment_positions(seg: np.ndarray) -> np.ndarray:
    """Positions that restart at 0 at the start of every run of equal ids
    (OmniVoice page, 'Memory and speed': each packed block has its own
    positions from 0).  seg: [S] -> [S] int64."""
    seg = np.asarray(seg)
    S = seg.shape[0]
    pos = np.zeros(S, dtype=np.int64)
    start = 0
    for i in range(1, S):
        if seg[i] != seg[i - 1]:
            start = i
        pos[i] = i - start
    return pos


# --------------------------------------------------------------------------
# Attention over the live set
# --------------------------------------------------------------------------


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, live: np.ndarray, scale: float):
    """Softmax attention of q [Sq, D] over k, v [Sk, D] restricted to the
    live keys, live [Sq, Sk] bool.  Two passes: the max over live scores,
    then exponentials, their sum and the weighted sum of V.  Non-live keys
    are excluded (their weight is set to 0, never exp of a large negative
    bias), so finite values in masked K/V cannot change the result.

    Returns o [Sq, D] and lse [Sq] (natural log); a row with no live key
    gives o = 0 and lse = -inf."""
    live = np.broadcast_to(live, (q.shape[0], k.shape[0]))
    s = scale * (q @ k.T)
    any_live = live.any(axis=1)
    m = np.where(live, s, -np.inf).max(axis=1, initial=-np.inf)
    m_safe = np.where(any_live, m, 0.0)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(s - m_safe[:, None])
    p = np.where(live, e, 0.0)
    l = p.sum(axis=1)
    o = np.zeros((q.shape[0], v.shape[1]))
    o[any_live] = (p[any_live] @ v) / l[any_live, None]
    with np.errstate(divide="ignore"):
        lse = np.where(any_live, m_safe + np.log(np.where(any_live, l, 1.0)), -np.inf)
    return o, lse


def _rot_heads(n_heads_q: int, pe_attn_head: int) -> int:
    """Number of leading query heads that get RoPE: all when
    pe_attn_head < 0, else min(pe_attn_head, Hq) (F5-TTS page, 'Variants'
    table: RoPE on only the first head for the v0 base model)."""
    return n_heads_q if pe_attn_head < 0 else min(pe_attn_head, n_heads_q)


def live_set_fwd(B, Hq, Sq, Sk, mask_kind, mask=None, seg_q=None, seg_k=None):
    """The live set [B, Hq|1, Sq, Sk] of the forward call.

    'none': every key.  'bool': the mask itself (True = takes part;
    OmniVoice page, attention-mask bullet), broadcast over size-1 dims.
    'segment': query i and key j of one row are live together iff both
    carry the same non-negative id (the block-diagonal mask of the
    OmniVoice page's packed_guidance mode).  'causal': key j is live for
    query i iff j <= i (the prefill of the VoxCPM page's attention bullet,
    SDPA's is_causal convention)."""
    if mask_kind == "none":
        return np.ones((B, 1, Sq, Sk), dtype=bool)
    if mask_kind == "bool":
        m = np.asarray(mask, dtype=bool)
        assert m.ndim == 4 and m.shape[3] == Sk
        return np.broadcast_to(m, (B, m.shape[1], Sq, Sk))
    if mask_kind == "causal":
        live = np.arange(Sk)[None, :] <= np.arange(Sq)[:, None]
        return np.broadcast_to(live, (B, 1, Sq, Sk))
    if mask_kind == "segment":
        sq = np.broadcast_to(np.asarray(seg_q), (B, Sq))
        sk = np.broadcast_to(np.asarray(seg_k), (B, Sk))
        live = (sq[:, :, None] >= 0) & (sq[:, :, None] == sk[:, None, :])
        return live[:, None]
    raise ValueError(mask_kind)


def mzref_fwd(dtype: str, q_bits, k_bits, v_bits, *, scale: float = 0.0,
              rope_base: float = 0.0, pe_attn_head: int = -1,
              pos_q=None, pos_k=None, mask_kind: str = "none", mask=None,
              seg_q=None, seg_k=None, heads=None, rope_style: str = "interleaved",
              rope_precision: str = "exact", rope_factors=None, rope_mscale: float = 1.0,
              q_norm_w=None, k_norm_w=None, norm_eps: float = 1e-6):
    """Oracle of the bidirectional forward.

    q_bits [B, Hq, Sq, D], k_bits / v_bits [B, Hkv, Sk, D] (storage bits
    of ``dtype``).  GQA: query head h reads K/V head h // (Hq / Hkv), i.e.
    each K/V head repeated G times in a row (OmniVoice page, attention
    mask bullet; VoxCPM page, attention bullet: SDPA with enable_gqa).
    RoPE (rope_base > 0) on the first pe_attn_head query heads and the
    K/V heads they read; positions default to 0..S-1, or in segment mode
    to the index within the segment.  ``heads``: optional list of query
    heads to evaluate (others are left 0), for sampling large shapes.
    ``rope_style``: 'interleaved' (adjacent pairs) or 'half' (x_i, x_i+D/2).

    Returns (o [B, Hq, Sq, D], lse [B, Hq, Sq]) in fp64.
    """
    q = decode(q_bits, dtype)
    k = decode(k_bits, dtype)
    v = decode(v_bits, dtype)
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if scale <= 0:
        scale = 1.0 / math.sqrt(D)
    n_rot = _rot_heads(Hq, pe_attn_head) if rope_base > 0 else 0
    if G > 1 and n_rot not in (0, Hq):
        raise ValueError("partial-head RoPE is defined only without GQA")

    def positions(pos, seg, S):
        if pos is not None:
            return np.broadcast_to(np.asarray(pos, dtype=np.int64), (B, S))
        if mask_kind == "segment":
            sg = np.broadcast_to(np.asarray(seg), (B, S))
            return np.stack([segment_positions(sg[b]) for b in range(B)])
        return np.broadcast_to(np.arange(S, dtype=np.int64), (B, S))

    live = live_set_fwd(B, Hq, Sq, Sk, mask_kind, mask, seg_q, seg_k)
    o = np.zeros((B, Hq, Sq, D))
    lse = np.full((B, Hq, Sq), -np.inf)
    if n_rot:
        pq = positions(pos_q, seg_q, Sq)
        pk = positions(pos_k, seg_k, Sk)
    for b in range(B):
        for h in range(Hq):
            if heads is not None and h not in heads:
                continue
            hk = h // G
            qh, kh, vh = q[b, h], k[b, hk], v[b, hk]
            if q_norm_w is not None:
                qh = rms_norm(qh, decode(q_norm_w, dtype), norm_eps)
            if k_norm_w is not None:
                kh = rms_norm(kh, decode(k_norm_w, dtype), norm_eps)
            if h < n_rot:
                qh = rope(qh, pq[b], rope_base, rope_style, rope_precision, rope_factors, rope_mscale)
                kh = rope(kh, pk[b], rope_base, rope_style, rope_precision, rope_factors, rope_mscale)
            lv = live[b, h if live.shape[1] > 1 else 0]
            o[b, h], lse[b, h] = attend(qh, kh, vh, lv, scale)
    return o, lse


def mzref_decode(dtype: str, q_bits, k_bits, v_bits, *, span: int, mask=None,
                 scale: float = 0.0, rope_base: float = 0.0, q_pos=None, rope_style: str = "interleaved",
                 rope_precision: str = "exact", rope_factors=None, rope_mscale: float = 1.0):
    """Oracle of one static-cache step (VoxCPM page, 'What matches
    upstream', attention bullet, and 'Memory and speed', attention_span).

    q_bits [B, Hq, q_len, D]; k_bits / v_bits [B, Hkv, cache_len, D] with
    K already rotated (a static cache stores rotated keys).  Key j is live
    for (b, h, t) iff j < span and mask[b, h, t, j] (mask broadcast over
    size-1 dims; None = all).  Optional RoPE on q at positions q_pos
    [B, q_len] on every head.  Returns o [B, Hq, q_len, D] in fp64.
    """
    q = decode(q_bits, dtype)
    k = decode(k_bits, dtype)
    v = decode(v_bits, dtype)
    B, Hq, T, D = q.shape
    Hkv, C = k.shape[1], k.shape[2]
    G = Hq // Hkv
    if scale <= 0:
        scale = 1.0 / math.sqrt(D)
    in_span = np.arange(C) < span
    if mask is None:
        m = np.ones((1, 1, 1, C), dtype=bool)
    else:
        m = np.asarray(mask, dtype=bool)
    live = np.broadcast_to(m, (B, Hq, T, C)) & in_span
    o = np.zeros((B, Hq, T, D))
    for b in range(B):
        for h in range(Hq):
            qh = q[b, h]
            if rope_base > 0:
                qh = rope(qh, np.asarray(q_pos)[b], rope_base, rope_style, rope_precision, rope_factors, rope_mscale)
            o[b, h], _ = attend(qh, k[b, h // G], v[b, h // G], live[b, h], scale)
    return o


def mzref_decode_append(dtype: str, q_bits, k_new_bits, v_new_bits, k_cache_bits, v_cache_bits, lens, *,
                        mask=None, scale: float = 0.0, rope_base: float = 0.0, rope_style: str = "interleaved",
                        rope_precision: str = "exact", rope_factors=None, rope_mscale: float = 1.0):
    """Oracle of one generation step that appends its own keys and values
    to the static cache and reads the filled length from the cache state
    instead of the host (VoxCPM page, 'Memory and speed': every patch waits
    on the device for the language models' positions, copied from Python
    integers, and CUDA graphs attend over the whole cache; 'What matches
    upstream', attention bullet: the step attends to the static cache under
    an explicit boolean mask, past the current length zero and masked).

    Reading: the q_len new tokens of row b take cache rows and positions
    lens[b] + t (t = 0 .. q_len-1); their keys are rotated at that position
    (the cache stores rotated keys) and, with the values, written into the
    cache; query t rotated at the same position attends to keys
    j <= lens[b] + t (the filled rows and the new tokens up to itself),
    further restricted by mask[b, h, t, j] when a mask is given.  A row with
    lens[b] < 0 or lens[b] + q_len > cache_len overflows: nothing is
    written and its output is 0.

    q_bits [B, Hq, T, D], k_new_bits / v_new_bits [B, Hkv, T, D] (keys not
    rotated), k_cache_bits / v_cache_bits [B, Hkv, C, D].  Returns
    (o [B, Hq, T, D] fp64, k_rows [B, Hkv, T, D] fp64 (the rotated new
    keys, unrounded), overflow [B] bool)."""
    q = decode(q_bits, dtype)
    kn = decode(k_new_bits, dtype)
    vn = decode(v_new_bits, dtype)
    k = decode(k_cache_bits, dtype).copy()
    v = decode(v_cache_bits, dtype).copy()
    B, Hq, T, D = q.shape
    Hkv, C = k.shape[1], k.shape[2]
    G = Hq // Hkv
    if scale <= 0:
        scale = 1.0 / math.sqrt(D)
    lens = np.asarray(lens, dtype=np.int64)
    o = np.zeros((B, Hq, T, D))
    k_rows = np.zeros((B, Hkv, T, D))
    overflow = np.zeros(B, dtype=bool)
    m = np.ones((1, 1, 1, C), dtype=bool) if mask is None else np.asarray(mask, dtype=bool)
    m = np.broadcast_to(m, (B, Hq, T, C))
    for b in range(B):
        L = int(lens[b])
        if L < 0 or L + T > C:
            overflow[b] = True
            continue
        pos = L + np.arange(T)
        for hk in range(Hkv):
            kr = rope(kn[b, hk], pos, rope_base, rope_style, rope_precision, rope_factors, rope_mscale) if rope_base > 0 else kn[b, hk]
            k_rows[b, hk] = kr
            k[b, hk, L:L + T] = kr
            v[b, hk, L:L + T] = vn[b, hk]
        causal = np.arange(C)[None, :] <= pos[:, None]          # [T, C]
        for h in range(Hq):
            qh = rope(q[b, h], pos, rope_base, rope_style, rope_precision, rope_factors, rope_mscale) if rope_base > 0 else q[b, h]
            o[b, h], _ = attend(qh, k[b, h // G], v[b, h // G], causal & m[b, h], scale)
    return o, k_rows, overflow


# --------------------------------------------------------------------------
# Comparison helpers (the tolerances the GPU path is held to)
# --------------------------------------------------------------------------

def parity_stats(out: np.ndarray, ref: np.ndarray) -> dict:
    """max |d|, relative L2 and max |ref| of an output against the oracle."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = out - ref
    nref = float(np.linalg.norm(ref))
    return {
        "max_abs": float(np.abs(d).max()) if d.size else 0.0,
        "rel_l2": float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d)),
        "max_ref": float(np.abs(ref).max()) if ref.size else 0.0,
        "finite": bool(np.isfinite(out).all()),
    }


def within_tolerance(dtype: str, stats: dict) -> bool:
    """fp32: max |d| <= 1e-5.  fp16 / bf16: relative L2 <= 4e-3 and
    max |d| <= 2e-2 * max |ref|."""
    if not stats["finite"]:
        return False
    if dtype == "f32":
        return stats["max_abs"] <= 1e-5
    return stats["rel_l2"] <= 4e-3 and stats["max_abs"] <= 2e-2 * max(stats["max_ref"], 1e-30)
