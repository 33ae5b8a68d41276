"""Seeded synthetic inputs for masked bidirectional attention.

This module only *builds inputs*: shapes, random values, boolean masks,
segment ids.  It holds none of the attention arithmetic (no RoPE, no
scores, no softmax), so both the fp64 oracle under ``oracle/`` and the
HIP path can take their inputs from it without sharing any of the
method's computation.

The workloads mirror the shapes the source pages describe:

* F5-TTS page, "How it works": the DiT runs classifier-free guidance as a
  batch of two rows (conditional, unconditional); the v0 base variant
  rotates only head 0 (``pe_attn_head = 1``) and padded text is masked.
* OmniVoice page, "What matches upstream" (attention-mask bullet): a
  bidirectional Qwen3-0.6B forward over a conditional row and an
  unconditional row under a full 4-D boolean mask, K/V heads shared by
  query-head groups.
* OmniVoice page, "Memory and speed" (packed_guidance fast mode): the two
  rows packed side by side in one row under a block-diagonal mask, with
  positions restarting at 0 in each block.
* VoxCPM page, "What matches upstream" (attention bullet) and "Memory and
  speed" (attention_span fast mode): one query per step against a static
  8192-position KV cache, unfilled positions zero and masked, key span cut
  at the next multiple of 256.

Values are drawn with a CPU ``torch.Generator`` seeded per workload, as
fp32 ``randn`` in the order q, k, v, then rounded to the storage dtype
with round-to-nearest-even (torch's ``.to``).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
DTYPE_NAME = {v: k for k, v in DTYPES.items()}

MASK_NONE, MASK_BOOL, MASK_SEGMENT, MASK_CAUSAL = "none", "bool", "segment", "causal"


@dataclasses.dataclass
class FwdCase:
    """One call of the bidirectional forward: tensors live on the host.

    q: [B, Hq, Sq, D]; k, v: [B, Hkv, Sk, D], all in ``dtype``.
    mask: bool, broadcastable to [B, Hq, Sq, Sk] with size-1 dims
    (True = the key takes part).  seg_q / seg_k: int32 [B, S],
    non-decreasing per row, negative = padding.  pos_q / pos_k: int32
    [B, S] or None (None = default positions).
    """

    name: str
    dtype: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    scale: float = 0.0          # <= 0 means 1/sqrt(D)
    rope_base: float = 0.0      # 0 means no RoPE
    pe_attn_head: int = -1      # < 0 means all heads
    rope_style: str = "interleaved"  # or "half" (pairs (i, i + D/2))
    mask_kind: str = MASK_NONE
    mask: Optional[torch.Tensor] = None
    seg_q: Optional[torch.Tensor] = None
    seg_k: Optional[torch.Tensor] = None
    pos_q: Optional[torch.Tensor] = None
    pos_k: Optional[torch.Tensor] = None

    @property
    def shape(self):
        B, Hq, Sq, D = self.q.shape
        return B, Hq, self.k.shape[1], Sq, self.k.shape[2], D


@dataclasses.dataclass
class DecodeCase:
    """One static-cache step.

    q: [B, Hq, q_len, D]; k_cache / v_cache: [B, Hkv, cache_len, D];
    mask: bool broadcastable to [B, Hq, q_len, cache_len] or None;
    keys [0, span) are considered.
    """

    name: str
    dtype: str
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    span: int
    mask: Optional[torch.Tensor] = None
    scale: float = 0.0
    rope_base: float = 0.0
    q_pos: Optional[torch.Tensor] = None
    filled: int = 0             # informational: number of filled cache rows
    rope_style: str = "interleaved"


def _randn(gen: torch.Generator, shape, dtype: str, mult: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if mult != 1.0:
        x = x * mult
    return x.to(DTYPES[dtype])


def _qkv(seed, B, Hq, Hkv, Sq, Sk, D, dtype, mult=1.0):
    gen = torch.Generator().manual_seed(seed)
    q = _randn(gen, (B, Hq, Sq, D), dtype, mult)
    k = _randn(gen, (B, Hkv, Sk, D), dtype, mult)
    v = _randn(gen, (B, Hkv, Sk, D), dtype, mult)
    return q, k, v


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------

def tiny_cfg(materialized: bool = False) -> FwdCase:
    """fp32 CFG pair: B 2, H 4, S 64, D 64, RoPE base 1e4 on all heads;
    row 1's last 8 keys masked.  Seed 0."""
    q, k, v = _qkv(0, 2, 4, 4, 64, 64, 64, "f32")
    if materialized:
        mask = torch.ones(2, 1, 64, 64, dtype=torch.bool)
        mask[1, :, :, 56:] = False
    else:
        mask = torch.ones(2, 1, 1, 64, dtype=torch.bool)
        mask[1, :, :, 56:] = False
    return FwdCase("tiny_cfg_f32", "f32", q, k, v, scale=1.0 / 8.0, rope_base=1e4,
                   pe_attn_head=-1, mask_kind=MASK_BOOL, mask=mask)


def f5_dit_layer() -> FwdCase:
    """fp16 F5-style DiT layer: B 2 (CFG), H 16, D 64, S 1500 mel frames,
    values N(0,1)*0.5, RoPE (base 1e4) on head 0 only, row 1 pads its last
    300 keys.  Seed 1."""
    q, k, v = _qkv(1, 2, 16, 16, 1500, 1500, 64, "f16", mult=0.5)
    mask = torch.ones(2, 1, 1, 1500, dtype=torch.bool)
    mask[1, :, :, 1200:] = False
    return FwdCase("f5_dit_f16", "f16", q, k, v, scale=1.0 / 8.0, rope_base=1e4,
                   pe_attn_head=1, mask_kind=MASK_BOOL, mask=mask)


QWEN_S, QWEN_UNCOND = 2048, 800


def qwen_cfg_padded() -> FwdCase:
    """bf16 Qwen3-0.6B-shaped step: B 2 rows (cond 2048 tokens; uncond
    target-only 800 tokens right-padded to 2048), Hq 16 / Hkv 8, D 128,
    RoPE base 1e6 on all heads, materialized [2,1,2048,2048] mask.
    Seed 2."""
    S, U = QWEN_S, QWEN_UNCOND
    q, k, v = _qkv(2, 2, 16, 8, S, S, 128, "bf16")
    mask = torch.ones(2, 1, S, S, dtype=torch.bool)
    mask[1] = False
    mask[1, :, :U, :U] = True
    return FwdCase("qwen_cfg_padded_bf16", "bf16", q, k, v, scale=1.0 / math.sqrt(128),
                   rope_base=1e6, pe_attn_head=-1, mask_kind=MASK_BOOL, mask=mask)


def qwen_cfg_packed(as_bool_mask: bool = False, padded: Optional[FwdCase] = None) -> FwdCase:
    """The same two rows packed into one row of 2848 tokens: segment 0 is
    row 0 (2048 tokens), segment 1 is row 1's first 800 tokens.  Segment
    mode (positions derived from the segments), or, with
    ``as_bool_mask``, the equivalent materialized block-diagonal mask with
    explicit restarting positions."""
    p = padded if padded is not None else qwen_cfg_padded()
    S, U = QWEN_S, QWEN_UNCOND
    T = S + U

    def pack(x):
        return torch.cat([x[0:1], x[1:2, :, :U]], dim=2).contiguous()

    q, k, v = pack(p.q), pack(p.k), pack(p.v)
    seg = torch.cat([torch.zeros(S, dtype=torch.int32), torch.ones(U, dtype=torch.int32)])[None]
    if not as_bool_mask:
        return FwdCase("qwen_cfg_packed_bf16", "bf16", q, k, v, scale=p.scale,
                       rope_base=p.rope_base, pe_attn_head=-1, mask_kind=MASK_SEGMENT,
                       seg_q=seg, seg_k=seg)
    mask = torch.zeros(1, 1, T, T, dtype=torch.bool)
    mask[0, 0, :S, :S] = True
    mask[0, 0, S:, S:] = True
    pos = torch.cat([torch.arange(S, dtype=torch.int32), torch.arange(U, dtype=torch.int32)])[None]
    return FwdCase("qwen_cfg_packed_boolmask_bf16", "bf16", q, k, v, scale=p.scale,
                   rope_base=p.rope_base, pe_attn_head=-1, mask_kind=MASK_BOOL, mask=mask,
                   pos_q=pos, pos_k=pos)


VOX_CACHE = 8192
VOX_FILLED = (257, 1024, 3100, 8192)


def ceil256(n: int) -> int:
    """Span rounding for the static cache: the first multiple of 256 at or
    after the current length (VoxCPM page, 'What matches upstream')."""
    return -(-n // 256) * 256


VOX_PREFILL = 2048


def vox_prefill_causal(seed: int = 5) -> FwdCase:
    """bf16 causal prefill in the VoxCPM text-semantic LM's head layout
    (the decode step's: Hq 16 / Hkv 2, D 128): B 2 (guidance pair), 2048
    tokens, N(0,1) q/k/v, interleaved RoPE base 1e4 (the LM's LongRoPE
    factors are not modelled)."""
    B, Hq, Hkv, S, D = 2, 16, 2, VOX_PREFILL, 128
    gen = torch.Generator().manual_seed(seed)
    q = _randn(gen, (B, Hq, S, D), "bf16")
    k = _randn(gen, (B, Hkv, S, D), "bf16")
    v = _randn(gen, (B, Hkv, S, D), "bf16")
    return FwdCase("vox_prefill_causal_bf16", "bf16", q, k, v, scale=1.0 / math.sqrt(D),
                   rope_base=1e4, pe_attn_head=-1, mask_kind=MASK_CAUSAL)


def vox_decode(filled: int, span: Optional[int] = None, seed: int = 4) -> DecodeCase:
    """bf16 VoxCPM-style step: B 2 (CFG), 1 query, Hq 16 / Hkv 2, D 128,
    static cache of 8192 positions; the cache is drawn N(0,1) for every
    position and then zeroed from ``filled`` on, so the prefix is the same
    for every ``filled``; mask True iff j < filled.  ``span`` defaults to
    the full cache."""
    B, Hq, Hkv, D, C = 2, 16, 2, 128, VOX_CACHE
    gen = torch.Generator().manual_seed(seed)
    q = _randn(gen, (B, Hq, 1, D), "bf16")
    kc = _randn(gen, (B, Hkv, C, D), "bf16")
    vc = _randn(gen, (B, Hkv, C, D), "bf16")
    kc[:, :, filled:] = 0
    vc[:, :, filled:] = 0
    mask = torch.zeros(B, 1, 1, C, dtype=torch.bool)
    mask[..., :filled] = True
    return DecodeCase(f"vox_decode_L{filled}_bf16", "bf16", q, kc, vc,
                      span=C if span is None else span, mask=mask,
                      scale=1.0 / math.sqrt(D), filled=filled)


# --------------------------------------------------------------------------
# Random small cases for parity sweeps
# --------------------------------------------------------------------------

def random_fwd(seed: int, B: int, Hq: int, Hkv: int, Sq: int, Sk: int, D: int, dtype: str,
               mask_kind: str = MASK_NONE, *, rope_base: float = 0.0, pe_attn_head: int = -1,
               mask_shape: str = "full", live_p: float = 0.7, n_segments: int = 2,
               explicit_pos: bool = False, scale: float = 0.0, mult: float = 1.0) -> FwdCase:
    """A seeded random forward case.

    mask_shape (bool mode): 'full' [B,Hq,Sq,Sk], 'bcast_h' [B,1,Sq,Sk],
    'key' [B,1,1,Sk] or 'blocky' (a [B,1,Sq,Sk] mask with whole blocks of
    True/False and a few random holes, so that tile classification sees
    all-true, all-false and mixed tiles).
    Segment mode: ``n_segments`` contiguous runs per row (random lengths),
    with a trailing padding run of id -1 in row 0 when there is room;
    requires Sq == Sk.
    """
    q, k, v = _qkv(seed, B, Hq, Hkv, Sq, Sk, D, dtype, mult)
    rng = np.random.default_rng(seed + 1000)
    case = FwdCase(f"rand{seed}_{dtype}_{mask_kind}", dtype, q, k, v, scale=scale,
                   rope_base=rope_base, pe_attn_head=pe_attn_head, mask_kind=mask_kind)
    if mask_kind == MASK_BOOL:
        if mask_shape == "full":
            m = rng.random((B, Hq, Sq, Sk)) < live_p
        elif mask_shape == "bcast_h":
            m = rng.random((B, 1, Sq, Sk)) < live_p
        elif mask_shape == "key":
            m = rng.random((B, 1, 1, Sk)) < live_p
        elif mask_shape == "blocky":
            bq, bk = 48, 40
            blocks = rng.random((B, 1, -(-Sq // bq), -(-Sk // bk))) < 0.5
            m = np.repeat(np.repeat(blocks, bq, axis=2), bk, axis=3)[:, :, :Sq, :Sk].copy()
            holes = rng.random(m.shape) < 0.01
            m ^= holes
        else:
            raise ValueError(mask_shape)
        case.mask = torch.from_numpy(np.ascontiguousarray(m))
    elif mask_kind == MASK_SEGMENT:
        assert Sq == Sk
        segs = []
        for b in range(B):
            cuts = np.sort(rng.choice(np.arange(1, Sq), size=min(n_segments, Sq) - 1, replace=False)) \
                if n_segments > 1 and Sq > 1 else np.array([], dtype=np.int64)
            ids = np.zeros(Sq, dtype=np.int32)
            for c in cuts:
                ids[c:] += 1
            if b == 0 and Sq >= 8:
                pad = int(rng.integers(1, max(2, Sq // 8)))
                ids[Sq - pad:] = -1
                # keep ids non-decreasing: the padding run moves to the front
                ids = np.concatenate([ids[Sq - pad:], ids[:Sq - pad]])
            segs.append(ids)
        seg = torch.from_numpy(np.stack(segs).astype(np.int32))
        case.seg_q, case.seg_k = seg, seg.clone()
    if explicit_pos:
        case.pos_q = torch.from_numpy(rng.integers(0, 4096, size=(B, Sq)).astype(np.int32))
        case.pos_k = torch.from_numpy(rng.integers(0, 4096, size=(B, Sk)).astype(np.int32))
    return case


def random_decode(seed: int, B: int, Hq: int, Hkv: int, q_len: int, cache_len: int, D: int,
                  dtype: str, filled: int, span: int, *, rope_base: float = 0.0,
                  mask_heads: bool = False, garbage: float = 0.0) -> DecodeCase:
    """A seeded random decode case; keys at or past ``filled`` are masked
    and hold zeros, or N(0,1)*``garbage`` when ``garbage`` > 0 (finite
    junk that must not change the result)."""
    gen = torch.Generator().manual_seed(seed)
    q = _randn(gen, (B, Hq, q_len, D), dtype)
    kc = _randn(gen, (B, Hkv, cache_len, D), dtype)
    vc = _randn(gen, (B, Hkv, cache_len, D), dtype)
    if garbage > 0:
        kc[:, :, filled:] = (kc[:, :, filled:].float() * garbage).to(kc.dtype)
        vc[:, :, filled:] = (vc[:, :, filled:].float() * garbage).to(vc.dtype)
    else:
        kc[:, :, filled:] = 0
        vc[:, :, filled:] = 0
    rng = np.random.default_rng(seed + 2000)
    if mask_heads:
        m = rng.random((B, Hq, q_len, cache_len)) < 0.8
    else:
        m = np.ones((B, 1, 1, cache_len), dtype=bool)
    m[..., filled:] = False
    q_pos = None
    if rope_base > 0:
        q_pos = torch.from_numpy(rng.integers(0, 8192, size=(B, q_len)).astype(np.int32))
    return DecodeCase(f"rdec{seed}_{dtype}", dtype, q, kc, vc, span=span,
                      mask=torch.from_numpy(np.ascontiguousarray(m)), rope_base=rope_base,
                      q_pos=q_pos, filled=filled)


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits of a host tensor: uint16 for fp16/bf16, uint32 for
    fp32.  The oracle decodes these itself."""
    t = t.contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(t.dtype)
