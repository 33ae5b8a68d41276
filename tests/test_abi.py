"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/mzattn.h declares, agrees with the binding's struct layout, and
reports every invalid argument from the host-only validators."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from masked_bidirectional_attention_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mzattn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libmzattn.so not built")
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(mzattn_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
        assert n in B._SIGNATURES, f"{n} has no binding signature"


def test_version_and_strerror(lib):
    assert lib.mzattn_version() == 400
    for code in range(0, -11, -1):
        msg = lib.mzattn_strerror(code).decode()
        assert msg and msg != "unknown status", code
    assert lib.mzattn_strerror(-99).decode() == "unknown status"


def _c_layout(struct, fields):
    """sizeof and offsetof of a header struct, compiled with gcc."""
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"mzattn.h\"\nint main(void){\n"
    src += f'printf("%zu\\n", sizeof({struct}));\n'
    for f in fields:
        src += f'printf("%zu\\n", offsetof({struct}, {f}));\n'
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "probe.c")
        exe = os.path.join(d, "probe")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", f"-I{os.path.dirname(HEADER)}", c, "-o", exe],
                       check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    return [int(x) for x in out]


@pytest.mark.parametrize("cls,cname", [(B.FwdArgs, "mzattn_fwd_args"), (B.DecodeArgs, "mzattn_decode_args"),
                                      (B.DecodeAppendArgs, "mzattn_decode_append_args")])
def test_struct_layout_matches_header(cls, cname):
    fields = [f for f, _ in cls._fields_]
    got = _c_layout(cname, fields)
    assert got[0] == ctypes.sizeof(cls), "sizeof differs"
    for f, off in zip(fields, got[1:]):
        assert getattr(cls, f).offset == off, f"offset of {f} differs"


def test_header_compiles_as_cxx():
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "probe.cc")
        open(c, "w").write('#include "mzattn.h"\nint main(){ mzattn_fwd_args a{}; (void)a; return 0; }\n')
        subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", f"-I{os.path.dirname(HEADER)}", "-c", c,
                        "-o", os.path.join(d, "probe.o")], check=True)


# --------------------------------------------------------------------------
# forward argument checks (fake, aligned device addresses: nothing is read)
# --------------------------------------------------------------------------

FAKE = 0x7F0000000000


def good_fwd(dtype=B.MZ_BF16, B_=2, Hq=16, Hkv=8, Sq=300, Sk=300, D=128):
    a = B.new_fwd_args()
    a.dtype = dtype
    a.batch, a.heads_q, a.heads_kv, a.seq_q, a.seq_k, a.head_dim = B_, Hq, Hkv, Sq, Sk, D
    a.pe_attn_head = -1
    a.q, a.k, a.v, a.o = FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000
    for name, H, S in (("q", Hq, Sq), ("k", Hkv, Sk), ("v", Hkv, Sk), ("o", Hq, Sq)):
        setattr(a, name + "_stride", B._i64x3(H * S * D, S * D, D))
    return a


def with_workspace(L, a):
    need = ctypes.c_size_t(0)
    st = L.mzattn_fwd_workspace_size(ctypes.byref(a), ctypes.byref(need))
    assert st == 0, L.mzattn_last_error()
    a.workspace, a.workspace_bytes = (FAKE + 0x4000000 if need.value else None), need.value
    return need.value


def vfwd(L, a):
    return L.mzattn_validate_fwd(ctypes.byref(a))


def test_fwd_valid_variants(lib):
    L = lib
    a = good_fwd()
    with_workspace(L, a)
    assert vfwd(L, a) == 0
    # RoPE + segment mode
    a = good_fwd()
    a.rope_base, a.mask_kind = 1e6, B.MZ_MASK_SEGMENT
    a.seg_q = a.seg_k = FAKE + 0x5000000
    assert with_workspace(L, a) > 0
    assert vfwd(L, a) == 0
    # bool mask, broadcast over heads and queries
    a = good_fwd(dtype=B.MZ_F16, Hkv=16)
    a.mask_kind, a.mask = B.MZ_MASK_BOOL, FAKE + 0x6000000
    a.mask_stride = B._i64x4(300, 0, 0, 1)
    with_workspace(L, a)
    assert vfwd(L, a) == 0
    # causal: no mask or segment pointers needed, no extra workspace
    a = good_fwd()
    a.mask_kind = B.MZ_MASK_CAUSAL
    with_workspace(L, a)
    assert vfwd(L, a) == 0
    # empty problems are legal no-ops even with NULL tensors
    e = good_fwd(Sq=0)
    e.q = e.o = None
    assert vfwd(L, e) == 0
    z = good_fwd(B_=0)
    z.q = z.k = z.v = z.o = None
    assert vfwd(L, z) == 0


def mutate(field, value):
    def f(a):
        setattr(a, field, value)
    return f


def fwd_cases():
    def stride(name, i, v):
        def f(a):
            s = getattr(a, name + "_stride")
            s[i] = v
        return f

    def bool_mask(st3=1, st0=300):
        def f(a):
            a.mask_kind, a.mask = B.MZ_MASK_BOOL, FAKE + 0x6000000
            a.mask_stride = B._i64x4(st0, 0, 300, st3)
        return f

    def mask_null(a):
        a.mask_kind, a.mask = B.MZ_MASK_BOOL, None
        a.mask_stride = B._i64x4(300, 0, 300, 1)

    def seg(q=True, k=True):
        def f(a):
            a.mask_kind = B.MZ_MASK_SEGMENT
            a.seg_q = FAKE if q else None
            a.seg_k = FAKE if k else None
        return f

    return [
        ("struct_size", mutate("struct_size", 12), B.MZ_ERR_ABI),
        ("rope_style", mutate("rope_style", 3), B.MZ_ERR_VALUE),
        ("dtype", mutate("dtype", 7), B.MZ_ERR_DTYPE),
        ("batch<0", mutate("batch", -1), B.MZ_ERR_SHAPE),
        ("heads_q=0", mutate("heads_q", 0), B.MZ_ERR_SHAPE),
        ("gqa_ratio", mutate("heads_kv", 5), B.MZ_ERR_SHAPE),
        ("seq_q<0", mutate("seq_q", -3), B.MZ_ERR_SHAPE),
        ("seq_k_huge", mutate("seq_k", (1 << 20) + 1), B.MZ_ERR_SHAPE),
        ("head_dim", mutate("head_dim", 96), B.MZ_ERR_UNSUPPORTED),
        ("mask_kind", mutate("mask_kind", 9), B.MZ_ERR_UNSUPPORTED),
        ("scale_nan", mutate("scale", float("nan")), B.MZ_ERR_VALUE),
        ("rope_neg", mutate("rope_base", -1.0), B.MZ_ERR_VALUE),
        ("rope_one", mutate("rope_base", 1.0), B.MZ_ERR_VALUE),
        ("key_streams_3", mutate("key_streams", 3), B.MZ_ERR_VALUE),
        ("key_streams_neg", mutate("key_streams", -1), B.MZ_ERR_VALUE),
        ("q_null", mutate("q", None), B.MZ_ERR_NULL),
        ("o_null", mutate("o", None), B.MZ_ERR_NULL),
        ("k_null", mutate("k", None), B.MZ_ERR_NULL),
        ("q_misaligned", mutate("q", FAKE + 8), B.MZ_ERR_ALIGN),
        ("stride_neg", stride("k", 2, -128), B.MZ_ERR_STRIDE),
        ("stride_odd", stride("v", 2, 130), B.MZ_ERR_ALIGN),
        ("mask_null", mask_null, B.MZ_ERR_NULL),
        ("mask_key_stride", bool_mask(st3=2), B.MZ_ERR_STRIDE),
        ("mask_neg_stride", bool_mask(st0=-300), B.MZ_ERR_STRIDE),
        ("seg_null", seg(k=False), B.MZ_ERR_NULL),
        ("pos_stride", mutate("pos_q_stride_b", -1), B.MZ_ERR_STRIDE),
        ("lse_misaligned", mutate("lse", FAKE + 2), B.MZ_ERR_ALIGN),
    ]


@pytest.mark.parametrize("name,edit,code", fwd_cases(), ids=[c[0] for c in fwd_cases()])
def test_fwd_rejects(lib, name, edit, code):
    a = good_fwd()
    with_workspace(lib, a)
    edit(a)
    st = vfwd(lib, a)
    assert st == code, (name, st, lib.mzattn_last_error())
    assert lib.mzattn_last_error().decode()


def test_fwd_partial_rope_with_gqa_unsupported(lib):
    a = good_fwd()
    a.rope_base, a.pe_attn_head = 1e4, 1
    need = ctypes.c_size_t(0)
    assert lib.mzattn_fwd_workspace_size(ctypes.byref(a), ctypes.byref(need)) == B.MZ_ERR_UNSUPPORTED
    m = good_fwd(Hkv=16)
    m.rope_base, m.pe_attn_head = 1e4, 1
    with_workspace(lib, m)
    assert vfwd(lib, m) == 0


def test_fwd_workspace_checks(lib):
    a = good_fwd()
    a.rope_base = 1e4
    need = with_workspace(lib, a)
    assert need > 0
    a.workspace_bytes = need - 1
    assert vfwd(lib, a) == B.MZ_ERR_WORKSPACE
    a.workspace_bytes = need
    a.workspace = FAKE + 0x4000000 + 64
    assert vfwd(lib, a) == B.MZ_ERR_WORKSPACE
    a.workspace = None
    assert vfwd(lib, a) == B.MZ_ERR_WORKSPACE
    # no RoPE and no mask: no workspace at all
    b = good_fwd()
    assert with_workspace(lib, b) == 0
    assert vfwd(lib, b) == 0


def test_fwd_workspace_grows_with_shape(lib):
    sizes = []
    for S in (64, 1000, 4000):
        a = good_fwd(Sq=S, Sk=S)
        a.rope_base, a.mask_kind = 1e6, B.MZ_MASK_SEGMENT
        sizes.append(with_workspace(lib, a))
    assert sizes[0] < sizes[1] < sizes[2]


# --------------------------------------------------------------------------
# decode argument checks
# --------------------------------------------------------------------------

def good_dec(dtype=B.MZ_BF16, B_=2, Hq=16, Hkv=2, T=1, C=8192, D=128, span=8192):
    a = B.new_decode_args()
    a.dtype = dtype
    a.batch, a.heads_q, a.heads_kv, a.q_len, a.head_dim, a.cache_len, a.span = B_, Hq, Hkv, T, D, C, span
    a.q, a.k_cache, a.v_cache, a.o = FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000
    a.q_stride = B._i64x3(Hq * T * D, T * D, D)
    a.o_stride = B._i64x3(Hq * T * D, T * D, D)
    a.k_stride = B._i64x3(Hkv * C * D, C * D, D)
    a.v_stride = B._i64x3(Hkv * C * D, C * D, D)
    need = ctypes.c_size_t(0)
    return a, need


def vdec(L, a):
    need = ctypes.c_size_t(0)
    st = L.mzattn_decode_workspace_size(ctypes.byref(a), ctypes.byref(need))
    if st == 0:
        a.workspace, a.workspace_bytes = FAKE + 0x8000000, need.value
    return L.mzattn_validate_decode(ctypes.byref(a))


def test_decode_valid(lib):
    a, _ = good_dec()
    assert vdec(lib, a) == 0
    a, _ = good_dec(span=0)
    assert vdec(lib, a) == 0
    a, _ = good_dec(T=4, Hq=32, Hkv=2)
    a.mask, a.mask_stride = FAKE, B._i64x4(8192, 0, 0, 1)
    assert vdec(lib, a) == 0


def test_decode_workspace_independent_of_span(lib):
    sizes = set()
    for span in (0, 1, 257, 8192):
        a, need = good_dec(span=span)
        assert lib.mzattn_decode_workspace_size(ctypes.byref(a), ctypes.byref(need)) == 0
        sizes.add(need.value)
    assert len(sizes) == 1


def dec_cases():
    return [
        ("struct_size", mutate("struct_size", 1), B.MZ_ERR_ABI),
        ("dtype", mutate("dtype", -1), B.MZ_ERR_DTYPE),
        ("gqa_ratio", mutate("heads_kv", 3), B.MZ_ERR_SHAPE),
        ("q_len0", mutate("q_len", 0), B.MZ_ERR_SHAPE),
        ("q_len17", mutate("q_len", 17), B.MZ_ERR_SHAPE),
        ("rope_style", mutate("rope_style", 2), B.MZ_ERR_VALUE),
        ("head_dim", mutate("head_dim", 256), B.MZ_ERR_UNSUPPORTED),
        ("span_big", mutate("span", 8193), B.MZ_ERR_VALUE),
        ("span_neg", mutate("span", -1), B.MZ_ERR_VALUE),
        ("rows_too_many", mutate("heads_q", 160), B.MZ_ERR_UNSUPPORTED),
        ("rope_no_pos", mutate("rope_base", 1e4), B.MZ_ERR_NULL),
        ("cache_null", mutate("k_cache", None), B.MZ_ERR_NULL),
        ("o_misaligned", mutate("o", FAKE + 4), B.MZ_ERR_ALIGN),
        ("scale_inf", mutate("scale", float("inf")), B.MZ_ERR_VALUE),
    ]


@pytest.mark.parametrize("name,edit,code", dec_cases(), ids=[c[0] for c in dec_cases()])
def test_decode_rejects(lib, name, edit, code):
    a, _ = good_dec()
    edit(a)
    assert vdec(lib, a) == code, (name, lib.mzattn_last_error())


def test_decode_workspace_too_small(lib):
    a, need = good_dec()
    assert lib.mzattn_decode_workspace_size(ctypes.byref(a), ctypes.byref(need)) == 0
    a.workspace, a.workspace_bytes = FAKE, need.value - 256
    assert lib.mzattn_validate_decode(ctypes.byref(a)) == B.MZ_ERR_WORKSPACE


def test_no_gpu_needed_for_validation(lib):
    """The validators and size queries run here, where no GPU exists."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("this machine has a GPU")
    a = good_fwd()
    assert vfwd(lib, a) == 0


def test_compute_without_library_fails_loudly(monkeypatch):
    """No fallback: with the library missing, a compute call raises."""
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libmzattn.so")
    with pytest.raises(B.MzattnNotBuilt):
        B.lib()


# --------------------------------------------------------------------------
# mzattn_decode_append (host checks only)
# --------------------------------------------------------------------------

def good_app(B_=2, Hq=16, Hkv=2, T=1, C=8192, D=128):
    a = B.new_decode_append_args()
    a.dtype = B.MZ_BF16
    a.batch, a.heads_q, a.heads_kv, a.q_len, a.head_dim, a.cache_len = B_, Hq, Hkv, T, D, C
    a.q, a.k_new, a.v_new = FAKE, FAKE + 0x100000, FAKE + 0x200000
    a.k_cache, a.v_cache, a.o = FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000
    a.q_stride = a.o_stride = B._i64x3(Hq * T * D, T * D, D)
    a.k_new_stride = a.v_new_stride = B._i64x3(Hkv * T * D, T * D, D)
    a.k_stride = a.v_stride = B._i64x3(Hkv * C * D, C * D, D)
    a.len, a.len_stride_b = FAKE + 0x4000000, 1
    a.rope_base = 1e4
    return a


def vapp(L, a):
    need = ctypes.c_size_t(0)
    st = L.mzattn_decode_append_workspace_size(ctypes.byref(a), ctypes.byref(need))
    if st == 0:
        a.workspace, a.workspace_bytes = FAKE + 0x8000000, need.value
    return L.mzattn_validate_decode_append(ctypes.byref(a))


def test_decode_append_valid(lib):
    assert vapp(lib, good_app()) == 0
    a = good_app(T=4, Hq=32, Hkv=2)
    a.mask, a.mask_stride = FAKE, B._i64x4(8192, 0, 0, 1)
    a.overflow = FAKE + 0x5000000
    a.len_stride_b = 0
    assert vapp(lib, a) == 0


def test_decode_append_workspace_matches_decode(lib):
    """The append step needs the decode step's workspace for the whole
    cache (no rotated-q copy: q rotates in the chunk kernel)."""
    a = good_app()
    need = ctypes.c_size_t(0)
    assert lib.mzattn_decode_append_workspace_size(ctypes.byref(a), ctypes.byref(need)) == 0
    d, nd = good_dec(span=8192)
    assert lib.mzattn_decode_workspace_size(ctypes.byref(d), ctypes.byref(nd)) == 0
    assert need.value == nd.value


def app_cases():
    def m(field, value):
        return lambda a: setattr(a, field, value)
    return [
        ("struct_size", m("struct_size", 4), B.MZ_ERR_ABI),
        ("fp32", m("dtype", B.MZ_F32), B.MZ_ERR_UNSUPPORTED),
        ("len_null", m("len", None), B.MZ_ERR_NULL),
        ("len_stride_neg", m("len_stride_b", -1), B.MZ_ERR_STRIDE),
        ("k_new_null", m("k_new", None), B.MZ_ERR_NULL),
        ("v_new_misaligned", m("v_new", FAKE + 0x200000 + 2), B.MZ_ERR_ALIGN),
        ("k_new_stride", m("k_new_stride", B._i64x3(2 * 128, 128, 129)), B.MZ_ERR_ALIGN),
        ("rope_base_one", m("rope_base", 1.0), B.MZ_ERR_VALUE),
        ("cache_empty", m("cache_len", 0), B.MZ_ERR_SHAPE),
        ("q_len17", m("q_len", 17), B.MZ_ERR_SHAPE),
        ("gqa_ratio", m("heads_kv", 3), B.MZ_ERR_SHAPE),
    ]


@pytest.mark.parametrize("name,edit,code", app_cases(), ids=[c[0] for c in app_cases()])
def test_decode_append_rejects(lib, name, edit, code):
    a = good_app()
    edit(a)
    assert vapp(lib, a) == code, (name, lib.mzattn_last_error())


@pytest.mark.parametrize("field,value,code", [
    ("rope_precision", 3, B.MZ_ERR_VALUE),
    ("rope_precision", -1, B.MZ_ERR_VALUE),
    ("rope_mscale", -1.0, B.MZ_ERR_VALUE),
    ("rope_mscale", float("nan"), B.MZ_ERR_VALUE),
    ("rope_factors", FAKE + 2, B.MZ_ERR_ALIGN),
])
def test_rope_options_checked_everywhere(lib, field, value, code):
    """The RoPE precision, scale and factors are checked by all three entry
    points."""
    a = good_fwd()
    setattr(a, field, value)
    assert vfwd(lib, a) == code, lib.mzattn_last_error()
    d, _ = good_dec()
    setattr(d, field, value)
    assert vdec(lib, d) == code, lib.mzattn_last_error()
    p = good_app()
    setattr(p, field, value)
    assert vapp(lib, p) == code, lib.mzattn_last_error()


def test_rope_options_valid(lib):
    for prec in (0, 1, 2):
        a = good_fwd()
        a.rope_precision, a.rope_mscale, a.rope_factors = prec, 1.118, FAKE + 0x6000000
        assert vfwd(lib, a) == 0, lib.mzattn_last_error()


def test_norm_options_checked(lib):
    a = good_fwd()
    a.q_norm_w, a.k_norm_w, a.norm_eps = FAKE + 0x7000000, FAKE + 0x7001000, 1e-6
    with_workspace(lib, a)
    assert vfwd(lib, a) == 0, lib.mzattn_last_error()
    a.k_norm_w = FAKE + 0x7001000 + 8
    assert vfwd(lib, a) == B.MZ_ERR_ALIGN
    a.k_norm_w = None
    a.norm_eps = -1.0
    assert vfwd(lib, a) == B.MZ_ERR_VALUE
    a.norm_eps = float("inf")
    assert vfwd(lib, a) == B.MZ_ERR_VALUE


def test_k_norm_needs_the_k_pass_workspace(lib):
    """With k normalised every K head passes through the workspace, RoPE or
    not, so the workspace grows."""
    a = good_fwd()
    a.rope_base = 0.0
    need0 = ctypes.c_size_t(0)
    assert lib.mzattn_fwd_workspace_size(ctypes.byref(a), ctypes.byref(need0)) == 0
    a.k_norm_w = FAKE + 0x7000000
    need1 = ctypes.c_size_t(0)
    assert lib.mzattn_fwd_workspace_size(ctypes.byref(a), ctypes.byref(need1)) == 0
    assert need1.value >= need0.value + a.batch * a.heads_kv * a.seq_k * a.head_dim * 2
