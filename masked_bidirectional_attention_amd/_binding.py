"""ctypes binding of libmzattn.so (argument marshalling only).

Every computation runs in the HIP library; this module turns torch tensors
into the C argument structs of ``include/mzattn.h``, allocates outputs and
workspaces with torch (device memory is torch's), and passes torch's
current HIP stream.  There is no fallback: if the library is missing,
every call raises ``MzattnNotBuilt``.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmzattn.so")

# status codes (include/mzattn.h)
MZ_OK = 0
MZ_ERR_NULL = -1
MZ_ERR_SHAPE = -2
MZ_ERR_DTYPE = -3
MZ_ERR_STRIDE = -4
MZ_ERR_ALIGN = -5
MZ_ERR_UNSUPPORTED = -6
MZ_ERR_WORKSPACE = -7
MZ_ERR_ABI = -8
MZ_ERR_HIP = -9
MZ_ERR_VALUE = -10

MZ_F32, MZ_F16, MZ_BF16 = 0, 1, 2
MZ_MASK_NONE, MZ_MASK_BOOL, MZ_MASK_SEGMENT, MZ_MASK_CAUSAL = 0, 1, 2, 3
ROPE_STYLES = {"interleaved": 0, "half": 1}


def _rope_style(style) -> int:
    if style not in ROPE_STYLES:
        raise MzattnError(MZ_ERR_VALUE, f"rope_style must be one of {sorted(ROPE_STYLES)}")
    return ROPE_STYLES[style]


ROPE_PRECISIONS = {"exact": 0, "fp16": 1, "bf16_table": 2}


def _set_rope_extra(a, keep, precision, mscale, factors):
    """rope_precision ('exact' | 'fp16' | 'bf16_table'), rope_mscale and
    the optional fp32 device tensor of LongRoPE factors [head_dim / 2]."""
    if precision not in ROPE_PRECISIONS:
        raise MzattnError(MZ_ERR_VALUE, f"rope_precision must be one of {sorted(ROPE_PRECISIONS)}")
    a.rope_precision = ROPE_PRECISIONS[precision]
    a.rope_mscale = float(mscale)
    if factors is not None:
        torch = _torch()
        if factors.dtype != torch.float32 or factors.dim() != 1 or factors.shape[0] != a.head_dim // 2 \
                or not factors.is_contiguous():
            raise MzattnError(MZ_ERR_SHAPE, "rope_factors must be a contiguous float32 tensor [head_dim / 2]")
        a.rope_factors = factors.data_ptr()
        keep.append(factors)

_i64x3 = ctypes.c_int64 * 3
_i64x4 = ctypes.c_int64 * 4


class MzattnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"mzattn status {status}: {msg}")
        self.status = status


class MzattnNotBuilt(RuntimeError):
    pass


class FwdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("seq_q", ctypes.c_int32),
        ("seq_k", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("pe_attn_head", ctypes.c_int32),
        ("mask_kind", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("rope_style", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("rope_precision", ctypes.c_int32),
        ("rope_mscale", ctypes.c_float),
        ("rope_factors", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("q_stride", _i64x3),
        ("k_stride", _i64x3),
        ("v_stride", _i64x3),
        ("o_stride", _i64x3),
        ("pos_q", ctypes.c_void_p),
        ("pos_k", ctypes.c_void_p),
        ("pos_q_stride_b", ctypes.c_int64),
        ("pos_k_stride_b", ctypes.c_int64),
        ("mask", ctypes.c_void_p),
        ("mask_stride", _i64x4),
        ("seg_q", ctypes.c_void_p),
        ("seg_k", ctypes.c_void_p),
        ("seg_q_stride_b", ctypes.c_int64),
        ("seg_k_stride_b", ctypes.c_int64),
        ("q_norm_w", ctypes.c_void_p),
        ("k_norm_w", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
        ("lse", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("key_streams", ctypes.c_int32),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("cache_len", ctypes.c_int32),
        ("span", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("rope_style", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("rope_precision", ctypes.c_int32),
        ("rope_mscale", ctypes.c_float),
        ("rope_factors", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("q_stride", _i64x3),
        ("k_cache", ctypes.c_void_p),
        ("k_stride", _i64x3),
        ("v_cache", ctypes.c_void_p),
        ("v_stride", _i64x3),
        ("o", ctypes.c_void_p),
        ("o_stride", _i64x3),
        ("q_pos", ctypes.c_void_p),
        ("q_pos_stride_b", ctypes.c_int64),
        ("mask", ctypes.c_void_p),
        ("mask_stride", _i64x4),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class DecodeAppendArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("cache_len", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("rope_style", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("rope_precision", ctypes.c_int32),
        ("rope_mscale", ctypes.c_float),
        ("rope_factors", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("q_stride", _i64x3),
        ("k_new", ctypes.c_void_p),
        ("k_new_stride", _i64x3),
        ("v_new", ctypes.c_void_p),
        ("v_new_stride", _i64x3),
        ("k_cache", ctypes.c_void_p),
        ("k_stride", _i64x3),
        ("v_cache", ctypes.c_void_p),
        ("v_stride", _i64x3),
        ("len", ctypes.c_void_p),
        ("len_stride_b", ctypes.c_int64),
        ("o", ctypes.c_void_p),
        ("o_stride", _i64x3),
        ("mask", ctypes.c_void_p),
        ("mask_stride", _i64x4),
        ("overflow", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


# exported C symbols and their signatures
_SIGNATURES = {
    "mzattn_fwd": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "mzattn_fwd_plan": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "mzattn_fwd_execute": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "mzattn_fwd_rotate_k": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "mzattn_fwd_attend": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.c_void_p]),
    "mzattn_fwd_workspace_size": (ctypes.c_int, [ctypes.POINTER(FwdArgs), ctypes.POINTER(ctypes.c_size_t)]),
    "mzattn_validate_fwd": (ctypes.c_int, [ctypes.POINTER(FwdArgs)]),
    "mzattn_decode": (ctypes.c_int, [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]),
    "mzattn_decode_workspace_size": (ctypes.c_int, [ctypes.POINTER(DecodeArgs), ctypes.POINTER(ctypes.c_size_t)]),
    "mzattn_validate_decode": (ctypes.c_int, [ctypes.POINTER(DecodeArgs)]),
    "mzattn_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]),
    "mzattn_decode_append": (ctypes.c_int, [ctypes.POINTER(DecodeAppendArgs), ctypes.c_void_p]),
    "mzattn_decode_append_workspace_size": (ctypes.c_int, [ctypes.POINTER(DecodeAppendArgs),
                                                           ctypes.POINTER(ctypes.c_size_t)]),
    "mzattn_validate_decode_append": (ctypes.c_int, [ctypes.POINTER(DecodeAppendArgs)]),
    "mzattn_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "mzattn_last_error": (ctypes.c_char_p, []),
    "mzattn_version": (ctypes.c_int, []),
    "mzattn_device_info": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                          ctypes.POINTER(ctypes.c_int), ctypes.c_char_p, ctypes.c_int]),
}

_lib = None
_lib_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use)."""
    global _lib
    if _lib is None:
        with _lib_lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise MzattnNotBuilt(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m masked_bidirectional_attention_amd.build`")
                l = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in _SIGNATURES.items():
                    fn = getattr(l, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = l
    return _lib


def _check(status: int):
    if status != MZ_OK:
        L = lib()
        detail = L.mzattn_last_error().decode()
        raise MzattnError(status, f"{L.mzattn_strerror(status).decode()}: {detail}")


def new_fwd_args() -> FwdArgs:
    a = FwdArgs()
    a.struct_size = ctypes.sizeof(FwdArgs)
    return a


def new_decode_args() -> DecodeArgs:
    a = DecodeArgs()
    a.struct_size = ctypes.sizeof(DecodeArgs)
    return a


def new_decode_append_args() -> DecodeAppendArgs:
    a = DecodeAppendArgs()
    a.struct_size = ctypes.sizeof(DecodeAppendArgs)
    return a


# --------------------------------------------------------------------------
# torch marshalling
# --------------------------------------------------------------------------

def _torch():
    import torch  # noqa: WPS433 - torch is only needed for tensors
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: MZ_F32, torch.float16: MZ_F16, torch.bfloat16: MZ_BF16}
    if t.dtype not in codes:
        raise MzattnError(MZ_ERR_DTYPE, f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _strides3(t, name):
    if t.dim() != 4:
        raise MzattnError(MZ_ERR_SHAPE, f"{name} must be 4-D [B, H, S, D]")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise MzattnError(MZ_ERR_STRIDE, f"{name} head_dim must be contiguous")
    return _i64x3(*(t.stride(i) if t.shape[i] > 1 else 0 for i in range(3)))


def _mask_strides(m, B, H, Sq, Sk, name="mask"):
    torch = _torch()
    if m.dtype == torch.bool:
        m = m.view(torch.uint8)
    if m.dtype != torch.uint8:
        raise MzattnError(MZ_ERR_DTYPE, f"{name} must be bool or uint8")
    if m.dim() != 4:
        raise MzattnError(MZ_ERR_SHAPE, f"{name} must be 4-D")
    want = (B, H, Sq, Sk)
    st = []
    for i in range(4):
        if m.shape[i] == want[i] and want[i] != 1:
            st.append(m.stride(i))
        elif m.shape[i] == 1:
            st.append(0 if i < 3 else m.stride(i))
        else:
            raise MzattnError(MZ_ERR_SHAPE, f"{name} dim {i} is {m.shape[i]}, expected {want[i]} or 1")
    if Sk <= 1:
        st[3] = 1
    return m, _i64x4(*st)


class _Workspaces:
    """Per (device, stream) scratch buffers, grown on demand (contents need
    no initialisation)."""

    def __init__(self):
        self._bufs = {}
        self._lock = threading.Lock()

    def get(self, kind: str, device, stream_ptr: int, nbytes: int, zero: bool):
        torch = _torch()
        key = (kind, device.index, stream_ptr)
        with self._lock:
            buf = self._bufs.get(key)
            if buf is None or buf.numel() < nbytes:
                n = max(nbytes, 1 << 20)
                buf = (torch.zeros if zero else torch.empty)(n, dtype=torch.uint8, device=device)
                self._bufs[key] = buf
            return buf


_WS = _Workspaces()


class FwdCall:
    """A marshalled forward call: the C argument struct plus the tensors it
    points to (kept alive here).  ``plan()`` launches the layout prepasses,
    ``execute()`` the per-input work (``rotate_k()`` then ``attend()``), all
    on the call's stream; ``__call__`` launches everything.

    The plan lives in the workspace, so every FwdCall owns one (allocated
    here unless ``workspace`` is given): a plan is never overwritten by
    another call's.  A caller-supplied workspace must not be shared with
    another call between its plan and its executes."""

    def __init__(self, q, k, v, *, mask=None, seg_q=None, seg_k=None, causal: bool = False, pos_q=None, pos_k=None,
                 scale: float = 0.0, rope_base: float = 0.0, pe_attn_head: int = -1,
                 rope_style: str = "interleaved", rope_precision: str = "exact", rope_mscale: float = 0.0,
                 rope_factors=None, q_norm_weight=None, k_norm_weight=None, norm_eps: float = 1e-6,
                 out=None, return_lse: bool = False, workspace=None, stream=None, key_streams: int = 0,
                 _shared_workspace=False):
        torch = _torch()
        L = lib()
        B, Hq, Sq, D = q.shape
        Hkv, Sk = k.shape[1], k.shape[2]
        a = new_fwd_args()
        a.dtype = _dtype_code(q)
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise MzattnError(MZ_ERR_DTYPE, "q, k, v must share one dtype")
        a.batch, a.heads_q, a.heads_kv, a.seq_q, a.seq_k, a.head_dim = B, Hq, Hkv, Sq, Sk, D
        a.pe_attn_head = pe_attn_head
        a.scale = float(scale)
        a.rope_base = float(rope_base)
        a.rope_style = _rope_style(rope_style)
        o = out if out is not None else torch.empty(B, Hq, Sq, D, dtype=q.dtype, device=q.device)
        a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
        a.q_stride, a.k_stride = _strides3(q, "q"), _strides3(k, "k")
        a.v_stride, a.o_stride = _strides3(v, "v"), _strides3(o, "o")
        keep = [q, k, v, o]
        _set_rope_extra(a, keep, rope_precision, rope_mscale, rope_factors)
        for name, w in (("q_norm_w", q_norm_weight), ("k_norm_w", k_norm_weight)):
            if w is not None:
                if w.dtype != q.dtype or w.dim() != 1 or w.shape[0] != D or not w.is_contiguous():
                    raise MzattnError(MZ_ERR_SHAPE, f"{name} must be a contiguous [head_dim] tensor of q's dtype")
                setattr(a, name, w.data_ptr())
                keep.append(w)
        a.norm_eps = float(norm_eps)
        a.key_streams = int(key_streams)
        if (mask is not None) + (seg_q is not None) + bool(causal) > 1:
            raise MzattnError(MZ_ERR_UNSUPPORTED, "give at most one of mask, segment ids, causal")
        if causal:
            a.mask_kind = MZ_MASK_CAUSAL
        elif mask is not None:
            a.mask_kind = MZ_MASK_BOOL
            m, st = _mask_strides(mask, B, Hq, Sq, Sk)
            a.mask, a.mask_stride = m.data_ptr(), st
            keep.append(m)
        elif seg_q is not None:
            a.mask_kind = MZ_MASK_SEGMENT
            seg_k = seg_q if seg_k is None else seg_k
            for s_ in (seg_q, seg_k):
                if s_.dtype != torch.int32 or s_.dim() != 2:
                    raise MzattnError(MZ_ERR_DTYPE, "segment ids must be int32 [B, S]")
            a.seg_q, a.seg_k = seg_q.data_ptr(), seg_k.data_ptr()
            a.seg_q_stride_b = seg_q.stride(0) if seg_q.shape[0] > 1 else 0
            a.seg_k_stride_b = seg_k.stride(0) if seg_k.shape[0] > 1 else 0
            keep += [seg_q, seg_k]
        for name, pos in (("pos_q", pos_q), ("pos_k", pos_k)):
            if pos is not None:
                if pos.dtype != torch.int32 or pos.dim() != 2:
                    raise MzattnError(MZ_ERR_DTYPE, f"{name} must be int32 [B, S]")
                setattr(a, name, pos.data_ptr())
                setattr(a, name + "_stride_b", pos.stride(0) if pos.shape[0] > 1 else 0)
                keep.append(pos)
        self.lse = None
        if return_lse:
            self.lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device=q.device)
            a.lse = self.lse.data_ptr()
        need = ctypes.c_size_t(0)
        _check(L.mzattn_fwd_workspace_size(ctypes.byref(a), ctypes.byref(need)))
        self.stream = torch.cuda.current_stream(q.device) if stream is None else stream
        if need.value > 0:
            if workspace is None and _shared_workspace:
                # one-shot calls (plan and execute launched back to back on
                # one stream) share a per-stream buffer: stream order keeps
                # a later call from overwriting it before this one is done
                workspace = _WS.get("fwd", q.device, self.stream.cuda_stream, need.value, zero=False)
            elif workspace is None:
                workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
            a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
            keep.append(workspace)
        self.args, self.out, self._keep, self._lib = a, o, keep, L
        self.workspace_bytes = need.value
        self._qkv_shape = [(tuple(x.shape), tuple(x.stride()), x.dtype) for x in (q, k, v)]

    def set_inputs(self, q, k, v):
        """Point the call at other Q, K, V of the same shapes, strides and
        dtype (the plan stays valid: it depends on the layout only)."""
        for x, want in zip((q, k, v), self._qkv_shape):
            if (tuple(x.shape), tuple(x.stride()), x.dtype) != want:
                raise MzattnError(MZ_ERR_SHAPE, "replacement input differs in shape, strides or dtype")
        self.args.q, self.args.k, self.args.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
        self._keep[0], self._keep[1], self._keep[2] = q, k, v

    def _launch(self, fn):
        _check(fn(ctypes.byref(self.args), ctypes.c_void_p(self.stream.cuda_stream)))

    def plan(self):
        self._launch(self._lib.mzattn_fwd_plan)

    def execute(self):
        self._launch(self._lib.mzattn_fwd_execute)

    def rotate_k(self):
        self._launch(self._lib.mzattn_fwd_rotate_k)

    def attend(self):
        self._launch(self._lib.mzattn_fwd_attend)

    def __call__(self):
        self._launch(self._lib.mzattn_fwd)
        return (self.out, self.lse) if self.lse is not None else self.out


def mzattn_fwd(q, k, v, *, mask=None, seg_q=None, seg_k=None, causal: bool = False, pos_q=None, pos_k=None,
               scale: float = 0.0, rope_base: float = 0.0, pe_attn_head: int = -1,
               rope_style: str = "interleaved", rope_precision: str = "exact", rope_mscale: float = 0.0,
               rope_factors=None, q_norm_weight=None, k_norm_weight=None, norm_eps: float = 1e-6, out=None,
               return_lse: bool = False, workspace=None, stream=None, key_streams: int = 0):
    """Masked bidirectional attention forward (see ``mzattn_fwd`` in
    include/mzattn.h).  q [B, Hq, Sq, D], k / v [B, Hkv, Sk, D] on one GPU,
    same dtype; mask: bool [B|1, Hq|1, Sq|1, Sk]; seg_q / seg_k: int32
    [B, S] (segment mode); causal: key j live for query i iff j <= i.
    Returns o (and lse when ``return_lse``)."""
    return FwdCall(q, k, v, mask=mask, seg_q=seg_q, seg_k=seg_k, causal=causal, pos_q=pos_q, pos_k=pos_k,
                   scale=scale, rope_base=rope_base, pe_attn_head=pe_attn_head, rope_style=rope_style, rope_precision=rope_precision,
                   rope_mscale=rope_mscale, rope_factors=rope_factors, q_norm_weight=q_norm_weight,
                   k_norm_weight=k_norm_weight, norm_eps=norm_eps, out=out,
                   return_lse=return_lse, workspace=workspace, stream=stream, key_streams=key_streams,
                   _shared_workspace=True)()


class DecodeCall:
    """A marshalled static-cache step: the C argument struct plus the
    tensors it points to.  ``set_cache`` swaps in other caches of the same
    shape, strides and dtype; ``__call__`` launches on the call's stream.
    With ``noalloc`` the call goes to ``mzattn_decode_noalloc`` (the
    library's own per-GPU scratch; no workspace is allocated here)."""

    def __init__(self, q, k_cache, v_cache, *, span: Optional[int] = None, mask=None,
                 scale: float = 0.0, rope_base: float = 0.0, q_pos=None, rope_style: str = "interleaved",
                 rope_precision: str = "exact", rope_mscale: float = 0.0, rope_factors=None, out=None,
                 workspace=None, stream=None, noalloc: bool = False):
        torch = _torch()
        L = lib()
        B, Hq, T, D = q.shape
        Hkv, C = k_cache.shape[1], k_cache.shape[2]
        a = new_decode_args()
        a.dtype = _dtype_code(q)
        if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
            raise MzattnError(MZ_ERR_DTYPE, "q and the caches must share one dtype")
        a.batch, a.heads_q, a.heads_kv, a.q_len, a.head_dim, a.cache_len = B, Hq, Hkv, T, D, C
        a.span = C if span is None else int(span)
        a.scale = float(scale)
        a.rope_base = float(rope_base)
        a.rope_style = _rope_style(rope_style)
        o = out if out is not None else torch.empty(B, Hq, T, D, dtype=q.dtype, device=q.device)
        a.q, a.k_cache, a.v_cache, a.o = q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr()
        a.q_stride, a.k_stride = _strides3(q, "q"), _strides3(k_cache, "k_cache")
        a.v_stride, a.o_stride = _strides3(v_cache, "v_cache"), _strides3(o, "o")
        keep = [q, k_cache, v_cache, o]
        _set_rope_extra(a, keep, rope_precision, rope_mscale, rope_factors)
        if mask is not None:
            m, st = _mask_strides(mask, B, Hq, T, C)
            a.mask, a.mask_stride = m.data_ptr(), st
            keep.append(m)
        if q_pos is not None:
            if q_pos.dtype != torch.int32 or q_pos.dim() != 2:
                raise MzattnError(MZ_ERR_DTYPE, "q_pos must be int32 [B, q_len]")
            a.q_pos = q_pos.data_ptr()
            a.q_pos_stride_b = q_pos.stride(0) if q_pos.shape[0] > 1 else 0
            keep.append(q_pos)
        need = ctypes.c_size_t(0)
        _check(L.mzattn_decode_workspace_size(ctypes.byref(a), ctypes.byref(need)))
        self.stream = torch.cuda.current_stream(q.device) if stream is None else stream
        self._fn = L.mzattn_decode_noalloc if noalloc else L.mzattn_decode
        if not noalloc:
            if workspace is None:
                workspace = _WS.get("decode", q.device, self.stream.cuda_stream, need.value, zero=False)
            a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
            keep.append(workspace)
        self.args, self.out, self._keep, self._lib = a, o, keep, L
        self._cache_shape = (tuple(k_cache.shape), tuple(k_cache.stride()), k_cache.dtype)

    def set_cache(self, k_cache, v_cache):
        for c in (k_cache, v_cache):
            if (tuple(c.shape), tuple(c.stride()), c.dtype) != self._cache_shape:
                raise MzattnError(MZ_ERR_SHAPE, "replacement cache differs in shape, strides or dtype")
        self.args.k_cache, self.args.v_cache = k_cache.data_ptr(), v_cache.data_ptr()
        self._keep[1], self._keep[2] = k_cache, v_cache

    def __call__(self):
        _check(self._fn(ctypes.byref(self.args), ctypes.c_void_p(self.stream.cuda_stream)))
        return self.out


def mzattn_decode(q, k_cache, v_cache, *, span: Optional[int] = None, mask=None,
                  scale: float = 0.0, rope_base: float = 0.0, q_pos=None, rope_style: str = "interleaved",
                  rope_precision: str = "exact", rope_mscale: float = 0.0, rope_factors=None, out=None, workspace=None, stream=None):
    """One static-cache step (see ``mzattn_decode`` in include/mzattn.h).
    q [B, Hq, q_len, D]; k_cache / v_cache [B, Hkv, cache_len, D]; keys
    [0, span) considered (default: the whole cache); mask: bool
    [B|1, Hq|1, q_len|1, cache_len] or None."""
    return DecodeCall(q, k_cache, v_cache, span=span, mask=mask, scale=scale, rope_base=rope_base,
                      q_pos=q_pos, rope_style=rope_style, rope_precision=rope_precision,
                      rope_mscale=rope_mscale, rope_factors=rope_factors, out=out, workspace=workspace, stream=stream)()


def mzattn_decode_noalloc(q, k_cache, v_cache, *, span: Optional[int] = None, mask=None,
                          scale: float = 0.0, rope_base: float = 0.0, q_pos=None, rope_style: str = "interleaved",
                          rope_precision: str = "exact", rope_mscale: float = 0.0, rope_factors=None, out=None,
                          stream=None):
    """``mzattn_decode`` through ``mzattn_decode_noalloc``: the library's
    fixed per-GPU scratch replaces the workspace (include/mzattn.h).  Calls
    on one GPU must not overlap in time."""
    return DecodeCall(q, k_cache, v_cache, span=span, mask=mask, scale=scale, rope_base=rope_base,
                      q_pos=q_pos, rope_style=rope_style, rope_precision=rope_precision,
                      rope_mscale=rope_mscale, rope_factors=rope_factors, out=out, stream=stream, noalloc=True)()


class DecodeAppendCall:
    """A marshalled append step (see ``mzattn_decode_append`` in
    include/mzattn.h): q [B, Hq, q_len, D] and k_new / v_new
    [B, Hkv, q_len, D], not rotated; the caches [B, Hkv, cache_len, D] get
    the new rows at len[b] + t; ``length`` is an int32 device tensor [B]
    (or [1]) holding the filled rows before the step.  Nothing here reads
    ``length`` on the host, so a call can be captured in a HIP graph and
    replayed after the caller updates ``length`` on the device.
    ``overflow`` (optional int32 device tensor [1]) is set to 1 when a row
    does not fit."""

    def __init__(self, q, k_new, v_new, k_cache, v_cache, length, *, mask=None, scale: float = 0.0,
                 rope_base: float = 0.0, rope_style: str = "interleaved", rope_precision: str = "exact",
                 rope_mscale: float = 0.0, rope_factors=None, overflow=None, out=None,
                 workspace=None, stream=None):
        torch = _torch()
        L = lib()
        B, Hq, T, D = q.shape
        Hkv, C = k_cache.shape[1], k_cache.shape[2]
        a = new_decode_append_args()
        a.dtype = _dtype_code(q)
        for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
            if t.dtype != q.dtype:
                raise MzattnError(MZ_ERR_DTYPE, f"{name} must have q's dtype")
        a.batch, a.heads_q, a.heads_kv, a.q_len, a.head_dim, a.cache_len = B, Hq, Hkv, T, D, C
        a.scale = float(scale)
        a.rope_base = float(rope_base)
        a.rope_style = _rope_style(rope_style)
        o = out if out is not None else torch.empty(B, Hq, T, D, dtype=q.dtype, device=q.device)
        a.q, a.k_new, a.v_new = q.data_ptr(), k_new.data_ptr(), v_new.data_ptr()
        a.k_cache, a.v_cache, a.o = k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr()
        a.q_stride, a.k_new_stride, a.v_new_stride = _strides3(q, "q"), _strides3(k_new, "k_new"), _strides3(v_new, "v_new")
        a.k_stride, a.v_stride, a.o_stride = _strides3(k_cache, "k_cache"), _strides3(v_cache, "v_cache"), _strides3(o, "o")
        if length.dtype != torch.int32 or length.dim() != 1 or length.shape[0] not in (1, B):
            raise MzattnError(MZ_ERR_DTYPE, "length must be an int32 tensor [B] or [1]")
        a.len = length.data_ptr()
        a.len_stride_b = length.stride(0) if length.shape[0] > 1 else 0
        keep = [q, k_new, v_new, k_cache, v_cache, length, o]
        _set_rope_extra(a, keep, rope_precision, rope_mscale, rope_factors)
        if mask is not None:
            m, st = _mask_strides(mask, B, Hq, T, C)
            a.mask, a.mask_stride = m.data_ptr(), st
            keep.append(m)
        if overflow is not None:
            if overflow.dtype != torch.int32 or overflow.numel() < 1:
                raise MzattnError(MZ_ERR_DTYPE, "overflow must be an int32 tensor")
            a.overflow = overflow.data_ptr()
            keep.append(overflow)
        need = ctypes.c_size_t(0)
        _check(L.mzattn_decode_append_workspace_size(ctypes.byref(a), ctypes.byref(need)))
        self.stream = torch.cuda.current_stream(q.device) if stream is None else stream
        if workspace is None:
            workspace = _WS.get("decode", q.device, self.stream.cuda_stream, need.value, zero=False)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        keep.append(workspace)
        self.args, self.out, self._keep, self._lib = a, o, keep, L

    def __call__(self):
        _check(self._lib.mzattn_decode_append(ctypes.byref(self.args), ctypes.c_void_p(self.stream.cuda_stream)))
        return self.out


def mzattn_decode_append(q, k_new, v_new, k_cache, v_cache, length, *, mask=None, scale: float = 0.0,
                         rope_base: float = 0.0, rope_style: str = "interleaved", rope_precision: str = "exact",
                         rope_mscale: float = 0.0, rope_factors=None, overflow=None, out=None,
                         workspace=None, stream=None):
    """One append step (see ``DecodeAppendCall``): writes the new rows into
    the caches and returns o [B, Hq, q_len, D]."""
    return DecodeAppendCall(q, k_new, v_new, k_cache, v_cache, length, mask=mask, scale=scale,
                            rope_base=rope_base, rope_style=rope_style, rope_precision=rope_precision,
                            rope_mscale=rope_mscale, rope_factors=rope_factors, overflow=overflow, out=out,
                            workspace=workspace, stream=stream)()


def mzattn_device_info(device: int = 0) -> dict:
    """What the HIP runtime reports for ``device`` (``mzattn_device_info``
    in include/mzattn.h): compute units, peak engine and memory clocks in
    MHz, and the gfx target name."""
    L = lib()
    cu, clk, mclk = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    arch = ctypes.create_string_buffer(64)
    _check(L.mzattn_device_info(int(device), ctypes.byref(cu), ctypes.byref(clk), ctypes.byref(mclk), arch, 64))
    return {"compute_units": cu.value, "clock_mhz": clk.value / 1000.0, "mem_clock_mhz": mclk.value / 1000.0,
            "arch": arch.value.decode()}
