"""Shared helpers of the GPU parity tests: run a workload through the HIP
library (via the C-ABI binding) and through the fp64 oracle."""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import masked_bidirectional_attention_amd as mz
from masked_bidirectional_attention_amd import workloads as W
from oracle import mzref

DEV = torch.device("cuda:0")


def dev(t):
    return None if t is None else t.to(DEV)


def run_fwd(case: W.FwdCase, return_lse=False, q=None, k=None, v=None, key_streams=0):
    q = dev(case.q) if q is None else q
    k = dev(case.k) if k is None else k
    v = dev(case.v) if v is None else v
    kw = dict(scale=case.scale, rope_base=case.rope_base, pe_attn_head=case.pe_attn_head,
              rope_style=case.rope_style, pos_q=dev(case.pos_q), pos_k=dev(case.pos_k), return_lse=return_lse,
              key_streams=key_streams)
    if case.mask_kind == W.MASK_BOOL:
        kw["mask"] = dev(case.mask)
    elif case.mask_kind == W.MASK_SEGMENT:
        kw["seg_q"], kw["seg_k"] = dev(case.seg_q), dev(case.seg_k)
    elif case.mask_kind == W.MASK_CAUSAL:
        kw["causal"] = True
    out = mz.mzattn_fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    return out


def oracle_fwd(case: W.FwdCase, heads=None):
    return mzref.mzref_fwd(
        case.dtype, W.to_bits(case.q), W.to_bits(case.k), W.to_bits(case.v),
        scale=case.scale, rope_base=case.rope_base, pe_attn_head=case.pe_attn_head,
        pos_q=None if case.pos_q is None else case.pos_q.numpy(),
        pos_k=None if case.pos_k is None else case.pos_k.numpy(),
        mask_kind=case.mask_kind, mask=None if case.mask is None else case.mask.numpy(),
        seg_q=None if case.seg_q is None else case.seg_q.numpy(),
        seg_k=None if case.seg_k is None else case.seg_k.numpy(), heads=heads, rope_style=case.rope_style)


def run_decode(case: W.DecodeCase, span=None, k=None, v=None):
    o = mz.mzattn_decode(dev(case.q), dev(case.k_cache) if k is None else k,
                         dev(case.v_cache) if v is None else v,
                         span=case.span if span is None else span, mask=dev(case.mask),
                         scale=case.scale, rope_base=case.rope_base, q_pos=dev(case.q_pos),
                         rope_style=case.rope_style)
    torch.cuda.synchronize()
    return o


def oracle_decode(case: W.DecodeCase, span=None):
    return mzref.mzref_decode(
        case.dtype, W.to_bits(case.q), W.to_bits(case.k_cache), W.to_bits(case.v_cache),
        span=case.span if span is None else span,
        mask=None if case.mask is None else case.mask.numpy(), scale=case.scale,
        rope_base=case.rope_base, q_pos=None if case.q_pos is None else case.q_pos.numpy(),
        rope_style=case.rope_style)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def log_parity(record: dict):
    """Append one JSON line to the file named by MZATTN_PARITY_LOG (if set):
    the achieved error of a parity check, kept beside the pass/fail."""
    path = os.environ.get("MZATTN_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(record) + "\n")


def assert_parity(dtype, out, ref, what=""):
    st = mzref.parity_stats(to64(out), ref)
    print(f"[parity] {what} {dtype} max_abs={st['max_abs']:.3e} rel_l2={st['rel_l2']:.3e} "
          f"max_ref={st['max_ref']:.3g}", flush=True)
    ok = mzref.within_tolerance(dtype, st)
    log_parity({"what": what, "dtype": dtype, "ok": ok, **st})
    assert ok, f"{what}: out of tolerance {st}"
    return st


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy()
    return t.view(torch.int32).numpy()
