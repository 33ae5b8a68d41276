// mzattn C ABI: host-side argument checks, workspace carving and dispatch.
// The checks make no HIP call, so mzattn_validate_* runs on machines
// without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "mzattn.h"
#include "mz_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return MZ_OK;
}

constexpr int64_t kMaxSeq = int64_t(1) << 20;
constexpr int kMaxBatch = 65535;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t elem_size(int dtype) { return dtype == MZ_F32 ? 4 : 2; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// rope_precision, rope_mscale and rope_factors (checked whether or not
// rotation is on, so a bad value never passes silently)
int check_rope_extra(int32_t precision, float mscale, const float* factors) {
  if (precision < 0 || precision > 2) return fail(MZ_ERR_VALUE, "rope_precision must be 0, 1 or 2 (got %d)", precision);
  if (!isfinite(mscale) || mscale < 0.f) return fail(MZ_ERR_VALUE, "rope_mscale must be finite and >= 0");
  if (factors != nullptr && !aligned(factors, 4)) return fail(MZ_ERR_ALIGN, "rope_factors is not 4-byte aligned");
  return MZ_OK;
}

mz::RopeSpec rope_spec(double base, int32_t precision, float mscale, const float* factors) {
  mz::RopeSpec r;
  r.log2_base = base > 0.0 ? log2(base) : 0.0;
  r.factors = factors;
  r.mscale = mscale > 0.f ? mscale : 1.f;
  r.precision = precision;
  return r;
}

// ---------------------------------------------------------------------------
// forward plan
// ---------------------------------------------------------------------------
struct FwdPlan {
  bool empty = false;
  int n_qt = 0, n_kt = 0, bm = 0;
  int n_rot = 0, n_rot_kv = 0, n_rotk = 0, tab_len = 0;
  int Bm = 1, Hm = 1;
  size_t off_tab = 0, off_krot = 0, off_qrange = 0, off_qtrange = 0, off_qpos = 0, off_kpos = 0, off_cls = 0;
  size_t off_bits = 0, off_qrows = 0, off_krows = 0, off_qcst = 0;
  int q_rows_b = 0, k_rows_b = 0;  // batch rows of the cos / sin row arrays (0: none)
  int q_cst_b = 0;                 // batch rows of the chunk-major query cos / sin (0: none)
  int mask_rows = 0;
  bool need_qpos = false;
  size_t bytes = 0;
};

int check_strides3(const int64_t* s, int vec, const char* name) {
  for (int i = 0; i < 3; ++i) {
    if (s[i] < 0) return fail(MZ_ERR_STRIDE, "%s_stride[%d] = %lld is negative", name, i, (long long)s[i]);
    if (s[i] % vec != 0)
      return fail(MZ_ERR_ALIGN, "%s_stride[%d] = %lld is not a multiple of %d elements", name, i,
                  (long long)s[i], vec);
  }
  return MZ_OK;
}

// Shape-only part of the forward checks and the workspace plan.
int plan_fwd(const mzattn_fwd_args* a, FwdPlan* pl) {
  if (a == nullptr) return fail(MZ_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(mzattn_fwd_args))
    return fail(MZ_ERR_ABI, "struct_size %u != sizeof(mzattn_fwd_args) %zu", a->struct_size,
                sizeof(mzattn_fwd_args));
  if (a->rope_style != 0 && a->rope_style != 1) return fail(MZ_ERR_VALUE, "rope_style must be 0 or 1 (got %d)", a->rope_style);
  if (a->dtype != MZ_F32 && a->dtype != MZ_F16 && a->dtype != MZ_BF16)
    return fail(MZ_ERR_DTYPE, "unknown dtype %d", a->dtype);
  if (a->batch < 0 || a->batch > kMaxBatch) return fail(MZ_ERR_SHAPE, "batch %d outside [0, %d]", a->batch, kMaxBatch);
  if (a->heads_q < 1 || a->heads_kv < 1 || a->heads_q > 65535 || a->heads_kv > 65535)
    return fail(MZ_ERR_SHAPE, "heads_q %d / heads_kv %d must be in [1, 65535]", a->heads_q, a->heads_kv);
  if (a->heads_q % a->heads_kv != 0)
    return fail(MZ_ERR_SHAPE, "heads_q %d is not a multiple of heads_kv %d", a->heads_q, a->heads_kv);
  if (a->seq_q < 0 || a->seq_k < 0 || a->seq_q > kMaxSeq || a->seq_k > kMaxSeq)
    return fail(MZ_ERR_SHAPE, "seq_q %d / seq_k %d outside [0, %lld]", a->seq_q, a->seq_k, (long long)kMaxSeq);
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(MZ_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", a->head_dim);
  if (a->mask_kind != MZ_MASK_NONE && a->mask_kind != MZ_MASK_BOOL && a->mask_kind != MZ_MASK_SEGMENT &&
      a->mask_kind != MZ_MASK_CAUSAL)
    return fail(MZ_ERR_UNSUPPORTED, "unknown mask_kind %d", a->mask_kind);
  if (!isfinite(a->scale)) return fail(MZ_ERR_VALUE, "scale is not finite");
  if (a->key_streams < 0 || a->key_streams > 2)
    return fail(MZ_ERR_VALUE, "key_streams %d (0 automatic, 1 or 2)", a->key_streams);
  if (!isfinite(a->rope_base) || a->rope_base < 0.0)
    return fail(MZ_ERR_VALUE, "rope_base must be finite and >= 0");
  if (a->rope_base > 0.0 && a->rope_base == 1.0)
    return fail(MZ_ERR_VALUE, "rope_base 1 gives no frequencies");
  {
    const int st = check_rope_extra(a->rope_precision, a->rope_mscale, a->rope_factors);
    if (st != MZ_OK) return st;
  }

  const int Hq = a->heads_q, Hkv = a->heads_kv, G = Hq / Hkv;
  int n_rot = 0;
  if (a->rope_base > 0.0) n_rot = a->pe_attn_head < 0 ? Hq : (a->pe_attn_head < Hq ? a->pe_attn_head : Hq);
  if (G > 1 && n_rot != 0 && n_rot != Hq)
    return fail(MZ_ERR_UNSUPPORTED, "pe_attn_head %d with GQA (G = %d): only 0 or all heads", a->pe_attn_head, G);
  pl->n_rot = n_rot;
  pl->n_rotk = G > 1 ? (n_rot ? Hkv : 0) : n_rot;
  // K heads that pass through the workspace: the rotated ones, or all when
  // k is normalised
  pl->n_rot_kv = a->k_norm_w != nullptr ? Hkv : pl->n_rotk;
  if (!isfinite(a->norm_eps) || a->norm_eps < 0.f) return fail(MZ_ERR_VALUE, "norm_eps must be finite and >= 0");
  if ((a->q_norm_w && !aligned(a->q_norm_w, 16)) || (a->k_norm_w && !aligned(a->k_norm_w, 16)))
    return fail(MZ_ERR_ALIGN, "q_norm_w / k_norm_w must be 16-byte aligned");

  pl->bm = a->dtype == MZ_F32 ? mz::F32_BM : mz::FWD_BM;
  pl->n_qt = (a->seq_q + pl->bm - 1) / pl->bm;
  pl->n_kt = (a->seq_k + mz::FWD_BN - 1) / mz::FWD_BN;
  pl->empty = a->batch == 0 || a->seq_q == 0;

  if (a->mask_kind == MZ_MASK_BOOL) {
    // (with no keys the mask is never read)
    if (a->mask_stride[3] != 1 && a->seq_k > 0)
      return fail(MZ_ERR_STRIDE, "mask_stride[3] must be 1 (got %lld)", (long long)a->mask_stride[3]);
    for (int i = 0; i < 3; ++i)
      if (a->mask_stride[i] < 0) return fail(MZ_ERR_STRIDE, "mask_stride[%d] is negative", i);
    pl->Bm = a->mask_stride[0] == 0 ? 1 : a->batch;
    pl->Hm = a->mask_stride[1] == 0 ? 1 : Hq;
  }
  if ((int64_t)a->batch * Hq * pl->n_qt >= (int64_t(1) << 31))
    return fail(MZ_ERR_SHAPE, "too many query tiles");
  if (a->mask_kind == MZ_MASK_BOOL && (int64_t)pl->Bm * pl->Hm * pl->n_qt * pl->n_kt >= (int64_t(1) << 31))
    return fail(MZ_ERR_SHAPE, "too many mask tiles");

  // workspace carve-up
  size_t off = 0;
  auto carve = [&](size_t bytes) {
    const size_t o = align256(off);
    off = o + bytes;
    return o;
  };
  const int D = a->head_dim;
  if (n_rot > 0) {
    // Index positions read the table (positions 0 .. seq - 1 of that side);
    // explicit or segment-derived positions get per-row arrays, so that no
    // kernel after the plan needs a position or the direct formula.
    const bool q_rows = a->pos_q != nullptr || a->mask_kind == MZ_MASK_SEGMENT;
    const bool k_rows = a->pos_k != nullptr || a->mask_kind == MZ_MASK_SEGMENT;
    int len = 0;
    if (!q_rows && a->seq_q > len) len = a->seq_q;
    if (!k_rows && a->seq_k > len) len = a->seq_k;
    pl->tab_len = len;
    if (len > 0) pl->off_tab = carve((size_t)len * (D / 2) * sizeof(float) * 2);
    if (q_rows) {
      pl->q_rows_b = (a->pos_q != nullptr && a->pos_q_stride_b == 0) ? 1 : a->batch;
      pl->off_qrows = carve((size_t)pl->q_rows_b * a->seq_q * (D / 2) * sizeof(float) * 2);
    }
    if (k_rows) {
      pl->k_rows_b = (a->pos_k != nullptr && a->pos_k_stride_b == 0) ? 1 : a->batch;
      pl->off_krows = carve((size_t)pl->k_rows_b * a->seq_k * (D / 2) * sizeof(float) * 2);
    }
    if (a->dtype != MZ_F32 && a->seq_q > 0) {
      pl->q_cst_b = q_rows ? pl->q_rows_b : 1;
      pl->off_qcst = carve((size_t)pl->q_cst_b * a->seq_q * (D / 2) * sizeof(float) * 2);
    }
  }
  if (pl->n_rot_kv > 0) pl->off_krot = carve((size_t)a->batch * pl->n_rot_kv * a->seq_k * D * elem_size(a->dtype));
  if (a->mask_kind == MZ_MASK_SEGMENT) {
    pl->off_qrange = carve((size_t)a->batch * a->seq_q * 8);
    pl->off_qtrange = carve((size_t)a->batch * pl->n_qt * 16);
    if (n_rot > 0) {
      pl->need_qpos = true;
      pl->off_qpos = carve((size_t)a->batch * a->seq_q * 4);
      pl->off_kpos = carve((size_t)a->batch * a->seq_k * 4);
    }
  }
  if (a->mask_kind == MZ_MASK_BOOL) {
    pl->off_cls = carve((size_t)pl->Bm * pl->Hm * pl->n_qt * pl->n_kt);
    if (a->dtype != MZ_F32) {
      pl->mask_rows = a->mask_stride[2] == 0 ? 1 : a->seq_q;
      pl->off_bits = carve((size_t)pl->Bm * pl->Hm * pl->mask_rows * pl->n_kt * 8);
    }
  }
  pl->bytes = off == 0 ? 0 : align256(off);
  return MZ_OK;
}

int validate_fwd_full(const mzattn_fwd_args* a, FwdPlan* pl) {
  int st = plan_fwd(a, pl);
  if (st != MZ_OK) return st;
  if (pl->empty) return MZ_OK;
  const int vec = a->dtype == MZ_F32 ? 4 : 8;
  if (a->q == nullptr || a->o == nullptr) return fail(MZ_ERR_NULL, "q and o must not be NULL");
  if (a->seq_k > 0 && (a->k == nullptr || a->v == nullptr)) return fail(MZ_ERR_NULL, "k and v must not be NULL");
  const void* ptrs[4] = {a->q, a->k, a->v, a->o};
  const char* names[4] = {"q", "k", "v", "o"};
  for (int i = 0; i < 4; ++i)
    if (ptrs[i] && !aligned(ptrs[i], 16)) return fail(MZ_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  if ((st = check_strides3(a->q_stride, vec, "q")) != MZ_OK) return st;
  if ((st = check_strides3(a->k_stride, vec, "k")) != MZ_OK) return st;
  if ((st = check_strides3(a->v_stride, vec, "v")) != MZ_OK) return st;
  if ((st = check_strides3(a->o_stride, vec, "o")) != MZ_OK) return st;
  if (a->k_stride[2] >= (int64_t(1) << 24) || a->v_stride[2] >= (int64_t(1) << 24))
    return fail(MZ_ERR_UNSUPPORTED, "k / v row strides must be below 2^24 elements");
  if (a->pos_q_stride_b < 0 || a->pos_k_stride_b < 0) return fail(MZ_ERR_STRIDE, "position strides must be >= 0");
  if (a->mask_kind == MZ_MASK_BOOL && a->mask == nullptr && a->seq_k > 0)
    return fail(MZ_ERR_NULL, "mask_kind BOOL needs mask");
  if (a->mask_kind == MZ_MASK_SEGMENT) {
    if (a->seg_q == nullptr || (a->seg_k == nullptr && a->seq_k > 0))
      return fail(MZ_ERR_NULL, "mask_kind SEGMENT needs seg_q and seg_k");
    if (a->seg_q_stride_b < 0 || a->seg_k_stride_b < 0) return fail(MZ_ERR_STRIDE, "segment strides must be >= 0");
  }
  if (a->lse && !aligned(a->lse, 4)) return fail(MZ_ERR_ALIGN, "lse is not 4-byte aligned");
  if (pl->bytes > 0) {
    if (a->workspace == nullptr) return fail(MZ_ERR_WORKSPACE, "workspace of %zu bytes required", pl->bytes);
    if (a->workspace_bytes < pl->bytes)
      return fail(MZ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", a->workspace_bytes, pl->bytes);
    if (!aligned(a->workspace, 256)) return fail(MZ_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  }
  return MZ_OK;
}

// ---------------------------------------------------------------------------
// decode plan
// ---------------------------------------------------------------------------
struct DecPlan {
  bool empty = false;
  int n_chunks = 0, n_chunks_max = 0, R = 0;
  size_t off_ml = 0, off_acc = 0, off_qrot = 0;
  size_t bytes = 0;
};

int plan_decode(const mzattn_decode_args* a, DecPlan* pl) {
  if (a == nullptr) return fail(MZ_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(mzattn_decode_args))
    return fail(MZ_ERR_ABI, "struct_size %u != sizeof(mzattn_decode_args) %zu", a->struct_size,
                sizeof(mzattn_decode_args));
  if (a->dtype != MZ_F32 && a->dtype != MZ_F16 && a->dtype != MZ_BF16)
    return fail(MZ_ERR_DTYPE, "unknown dtype %d", a->dtype);
  if (a->batch < 0 || a->batch > kMaxBatch) return fail(MZ_ERR_SHAPE, "batch %d outside [0, %d]", a->batch, kMaxBatch);
  if (a->heads_q < 1 || a->heads_kv < 1 || a->heads_q > 65535 || a->heads_kv > 65535)
    return fail(MZ_ERR_SHAPE, "heads_q %d / heads_kv %d must be in [1, 65535]", a->heads_q, a->heads_kv);
  if (a->heads_q % a->heads_kv != 0)
    return fail(MZ_ERR_SHAPE, "heads_q %d is not a multiple of heads_kv %d", a->heads_q, a->heads_kv);
  if (a->q_len < 1 || a->q_len > 16) return fail(MZ_ERR_SHAPE, "q_len %d outside [1, 16]", a->q_len);
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(MZ_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", a->head_dim);
  if (a->cache_len < 0 || a->cache_len > (1 << 24)) return fail(MZ_ERR_SHAPE, "cache_len %d outside [0, 2^24]", a->cache_len);
  if (a->span < 0 || a->span > a->cache_len)
    return fail(MZ_ERR_VALUE, "span %d outside [0, cache_len %d]", a->span, a->cache_len);
  const int G = a->heads_q / a->heads_kv;
  if ((int64_t)G * a->q_len > 64)
    return fail(MZ_ERR_UNSUPPORTED, "heads_q / heads_kv * q_len = %lld exceeds 64", (long long)G * a->q_len);
  if (!isfinite(a->scale)) return fail(MZ_ERR_VALUE, "scale is not finite");
  if (!isfinite(a->rope_base) || a->rope_base < 0.0 || a->rope_base == 1.0)
    return fail(MZ_ERR_VALUE, "rope_base must be finite, >= 0 and != 1");
  {
    const int st = check_rope_extra(a->rope_precision, a->rope_mscale, a->rope_factors);
    if (st != MZ_OK) return st;
  }
  if (a->rope_style != 0 && a->rope_style != 1)
    return fail(MZ_ERR_VALUE, "rope_style must be 0 or 1 (got %d)", a->rope_style);
  pl->R = G * a->q_len;
  pl->n_chunks = a->span > 0 ? (a->span + mz::DEC_CHUNK - 1) / mz::DEC_CHUNK : 1;
  pl->n_chunks_max = a->cache_len > 0 ? (a->cache_len + mz::DEC_CHUNK - 1) / mz::DEC_CHUNK : 1;
  pl->empty = a->batch == 0;
  if ((int64_t)a->batch * a->heads_kv * pl->n_chunks >= (int64_t(1) << 31)) return fail(MZ_ERR_SHAPE, "grid too large");
  size_t off = 0;
  auto carve = [&](size_t bytes) {
    const size_t o = align256(off);
    off = o + bytes;
    return o;
  };
  const size_t units = (size_t)a->batch * a->heads_kv;
  pl->off_ml = carve(units * pl->n_chunks_max * pl->R * sizeof(float) * 2);
  pl->off_acc = carve(units * pl->n_chunks_max * pl->R * a->head_dim * sizeof(float));
  if (a->rope_base > 0.0)
    pl->off_qrot = carve((size_t)a->batch * a->heads_q * a->q_len * a->head_dim * elem_size(a->dtype));
  pl->bytes = align256(off);
  return MZ_OK;
}

int validate_decode_full(const mzattn_decode_args* a, DecPlan* pl) {
  int st = plan_decode(a, pl);
  if (st != MZ_OK) return st;
  if (pl->empty) return MZ_OK;
  const int vec = a->dtype == MZ_F32 ? 4 : 8;
  if (a->q == nullptr || a->o == nullptr) return fail(MZ_ERR_NULL, "q and o must not be NULL");
  if (a->cache_len > 0 && (a->k_cache == nullptr || a->v_cache == nullptr))
    return fail(MZ_ERR_NULL, "k_cache and v_cache must not be NULL");
  const void* ptrs[4] = {a->q, a->k_cache, a->v_cache, a->o};
  const char* names[4] = {"q", "k_cache", "v_cache", "o"};
  for (int i = 0; i < 4; ++i)
    if (ptrs[i] && !aligned(ptrs[i], 16)) return fail(MZ_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  if ((st = check_strides3(a->q_stride, vec, "q")) != MZ_OK) return st;
  if ((st = check_strides3(a->k_stride, vec, "k")) != MZ_OK) return st;
  if ((st = check_strides3(a->v_stride, vec, "v")) != MZ_OK) return st;
  if ((st = check_strides3(a->o_stride, vec, "o")) != MZ_OK) return st;
  if (a->mask) {
    if (a->mask_stride[3] != 1) return fail(MZ_ERR_STRIDE, "mask_stride[3] must be 1 (got %lld)", (long long)a->mask_stride[3]);
    for (int i = 0; i < 3; ++i)
      if (a->mask_stride[i] < 0) return fail(MZ_ERR_STRIDE, "mask_stride[%d] is negative", i);
  }
  if (a->rope_base > 0.0) {
    if (a->q_pos == nullptr) return fail(MZ_ERR_NULL, "rope_base > 0 needs q_pos");
    if (a->q_pos_stride_b < 0) return fail(MZ_ERR_STRIDE, "q_pos_stride_b must be >= 0");
  }
  if (a->workspace == nullptr) return fail(MZ_ERR_WORKSPACE, "workspace of %zu bytes required", pl->bytes);
  if (a->workspace_bytes < pl->bytes)
    return fail(MZ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", a->workspace_bytes, pl->bytes);
  if (!aligned(a->workspace, 256)) return fail(MZ_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  return MZ_OK;
}

float scale_log2(float scale, int D) {
  const double s = scale > 0.f ? (double)scale : 1.0 / sqrt((double)D);
  return (float)(s * 1.4426950408889634074);  // log2(e)
}

// Fill the kernel parameter block of a validated call.
void fill_fwd_params(const mzattn_fwd_args* a, const FwdPlan& pl, mz::FwdParams& p) {
  memset(&p, 0, sizeof(p));
  p.dtype = a->dtype;
  p.B = a->batch; p.Hq = a->heads_q; p.Hkv = a->heads_kv; p.G = a->heads_q / a->heads_kv;
  p.Sq = a->seq_q; p.Sk = a->seq_k; p.D = a->head_dim;
  p.n_qt = pl.n_qt; p.n_kt = pl.n_kt;
  p.mask_kind = a->mask_kind;
  p.key_streams = a->key_streams;
  p.scale_log2 = scale_log2(a->scale, a->head_dim);
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o;
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = a->q_stride[i]; p.ks[i] = a->k_stride[i]; p.vs[i] = a->v_stride[i]; p.os[i] = a->o_stride[i];
  }
  char* ws = static_cast<char*>(a->workspace);
  p.n_rot = pl.n_rot; p.n_rot_kv = pl.n_rot_kv; p.n_rotk = pl.n_rotk;
  p.q_norm_w = a->q_norm_w; p.k_norm_w = a->k_norm_w; p.norm_eps = a->norm_eps;
  if (pl.n_rot_kv > 0) p.k_rot = ws + pl.off_krot;
  p.rope_style = a->rope_style;
  if (pl.n_rot > 0) {
    p.rs = rope_spec(a->rope_base, a->rope_precision, a->rope_mscale, a->rope_factors);
    p.rope_tab = pl.tab_len > 0 ? reinterpret_cast<float2*>(ws + pl.off_tab) : nullptr;
    p.rope_tab_len = pl.tab_len;
    if (pl.q_rows_b > 0) {
      p.q_rows = reinterpret_cast<float2*>(ws + pl.off_qrows);
      p.q_rows_b = pl.q_rows_b;
      p.q_cs = p.q_rows;
      p.q_cs_sb = pl.q_rows_b == 1 ? 0 : a->seq_q;
    } else {
      p.q_cs = p.rope_tab;
    }
    if (pl.q_cst_b > 0) {
      p.q_cst = reinterpret_cast<float4*>(ws + pl.off_qcst);
      p.q_cst_b = pl.q_cst_b;
      p.q_cst_sb = pl.q_cst_b == 1 ? 0 : (int64_t)(a->head_dim / 4) * a->seq_q;
    }
    if (pl.k_rows_b > 0) {
      p.k_rows = reinterpret_cast<float2*>(ws + pl.off_krows);
      p.k_rows_b = pl.k_rows_b;
      p.k_cs = p.k_rows;
      p.k_cs_sb = pl.k_rows_b == 1 ? 0 : a->seq_k;
    } else {
      p.k_cs = p.rope_tab;
    }
    if (a->pos_q) { p.pos_q_mode = mz::POS_ARRAY; p.pos_q = a->pos_q; p.pos_q_sb = a->pos_q_stride_b; }
    else if (a->mask_kind == MZ_MASK_SEGMENT) {
      p.pos_q_mode = mz::POS_SEGMENT; p.pos_q = reinterpret_cast<int32_t*>(ws + pl.off_qpos); p.pos_q_sb = a->seq_q;
    } else p.pos_q_mode = mz::POS_ARANGE;
    if (a->pos_k) { p.pos_k_mode = mz::POS_ARRAY; p.pos_k = a->pos_k; p.pos_k_sb = a->pos_k_stride_b; }
    else if (a->mask_kind == MZ_MASK_SEGMENT) {
      p.pos_k_mode = mz::POS_SEGMENT; p.pos_k = reinterpret_cast<int32_t*>(ws + pl.off_kpos); p.pos_k_sb = a->seq_k;
    } else p.pos_k_mode = mz::POS_ARANGE;
  }
  p.Bm = pl.Bm; p.Hm = pl.Hm;
  if (a->mask_kind == MZ_MASK_BOOL) {
    p.mask = a->mask;
    for (int i = 0; i < 4; ++i) p.ms[i] = a->mask_stride[i];
    p.tile_cls = reinterpret_cast<uint8_t*>(ws + pl.off_cls);
    if (a->dtype != MZ_F32) {
      p.mask_bits = reinterpret_cast<uint64_t*>(ws + pl.off_bits);
      p.mask_rows = pl.mask_rows;
    }
    p.mask_vec16 = aligned(a->mask, 16) && a->mask_stride[0] % 16 == 0 && a->mask_stride[1] % 16 == 0 &&
                   a->mask_stride[2] % 16 == 0;
  }
  if (a->mask_kind == MZ_MASK_SEGMENT) {
    p.seg_q = a->seg_q; p.seg_k = a->seg_k;
    p.seg_q_sb = a->seg_q_stride_b; p.seg_k_sb = a->seg_k_stride_b;
    p.q_range = reinterpret_cast<int2*>(ws + pl.off_qrange);
    p.qt_range = reinterpret_cast<int4*>(ws + pl.off_qtrange);
    p.qpos_ws = (pl.need_qpos && a->pos_q == nullptr) ? reinterpret_cast<int32_t*>(ws + pl.off_qpos) : nullptr;
    p.kpos_ws = (pl.need_qpos && a->pos_k == nullptr) ? reinterpret_cast<int32_t*>(ws + pl.off_kpos) : nullptr;
  }
  p.lse = a->lse;
}

int run_decode(const mzattn_decode_args* a, void* stream);

enum { FWD_PLAN = 1, FWD_ROT = 2, FWD_MAIN = 4 };

int run_fwd(const mzattn_fwd_args* a, void* stream, int parts) {
  FwdPlan pl;
  const int st = validate_fwd_full(a, &pl);
  if (st != MZ_OK) return st;
  if (pl.empty) return ok();
  mz::FwdParams p;
  fill_fwd_params(a, pl, p);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (parts & FWD_PLAN) e = mz::launch_fwd_plan(p, s);
  if (e == hipSuccess && (parts & FWD_ROT)) e = mz::launch_fwd_rotate(p, s);
  if (e == hipSuccess && (parts & FWD_MAIN)) e = mz::launch_fwd_main(p, s);
  if (e != hipSuccess) return fail(MZ_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}


}  // namespace

extern "C" {

int mzattn_version(void) { return MZATTN_VERSION; }

int mzattn_device_info(int device, int* compute_units, int* clock_khz, int* mem_clock_khz, char* arch, int arch_len) {
  hipDeviceProp_t prop;
  const hipError_t e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) {
    // the failed query leaves its error as the thread's last HIP error;
    // take it back so that the next launch check does not report it
    (void)hipGetLastError();
    return fail(MZ_ERR_HIP, "hipGetDeviceProperties(%d): %s", device, hipGetErrorString(e));
  }
  if (compute_units) *compute_units = prop.multiProcessorCount;
  if (clock_khz) *clock_khz = prop.clockRate;
  if (mem_clock_khz) *mem_clock_khz = prop.memoryClockRate;
  if (arch != nullptr && arch_len > 0) {
    snprintf(arch, (size_t)arch_len, "%s", prop.gcnArchName);
  }
  return MZ_OK;
}

const char* mzattn_strerror(int status) {
  switch (status) {
    case MZ_OK: return "ok";
    case MZ_ERR_NULL: return "a required pointer is NULL";
    case MZ_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case MZ_ERR_DTYPE: return "unknown element type";
    case MZ_ERR_STRIDE: return "invalid stride";
    case MZ_ERR_ALIGN: return "misaligned pointer or stride";
    case MZ_ERR_UNSUPPORTED: return "unsupported configuration";
    case MZ_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case MZ_ERR_ABI: return "argument struct does not match this library";
    case MZ_ERR_HIP: return "HIP launch failed";
    case MZ_ERR_VALUE: return "invalid scalar argument";
    default: return "unknown status";
  }
}

const char* mzattn_last_error(void) { return g_last_error.c_str(); }

int mzattn_fwd_workspace_size(const mzattn_fwd_args* args, size_t* bytes) {
  if (bytes == nullptr) return fail(MZ_ERR_NULL, "bytes is NULL");
  FwdPlan pl;
  const int st = plan_fwd(args, &pl);
  if (st != MZ_OK) return st;
  *bytes = pl.bytes;
  return ok();
}

int mzattn_validate_fwd(const mzattn_fwd_args* args) {
  FwdPlan pl;
  const int st = validate_fwd_full(args, &pl);
  return st == MZ_OK ? ok() : st;
}

int mzattn_fwd(const mzattn_fwd_args* a, void* stream) { return run_fwd(a, stream, FWD_PLAN | FWD_ROT | FWD_MAIN); }

int mzattn_fwd_plan(const mzattn_fwd_args* a, void* stream) { return run_fwd(a, stream, FWD_PLAN); }

int mzattn_fwd_execute(const mzattn_fwd_args* a, void* stream) { return run_fwd(a, stream, FWD_ROT | FWD_MAIN); }

int mzattn_fwd_rotate_k(const mzattn_fwd_args* a, void* stream) { return run_fwd(a, stream, FWD_ROT); }

int mzattn_fwd_attend(const mzattn_fwd_args* a, void* stream) { return run_fwd(a, stream, FWD_MAIN); }

int mzattn_decode_workspace_size(const mzattn_decode_args* args, size_t* bytes) {
  if (bytes == nullptr) return fail(MZ_ERR_NULL, "bytes is NULL");
  DecPlan pl;
  const int st = plan_decode(args, &pl);
  if (st != MZ_OK) return st;
  *bytes = pl.bytes;
  return ok();
}

int mzattn_validate_decode(const mzattn_decode_args* args) {
  DecPlan pl;
  const int st = validate_decode_full(args, &pl);
  return st == MZ_OK ? ok() : st;
}

int mzattn_decode(const mzattn_decode_args* a, void* stream) { return run_decode(a, stream); }

}  // extern "C"

// ---- the decode step without allocation --------------------------------
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): mzattn_decode with the
// workspace taken from a fixed device array of this library instead of the
// caller.  Each GPU holds its own copy of the array until the process ends;
// its device address is looked up once per device and kept, and only that
// address is handed to the kernels.
namespace {

constexpr size_t kScratchBytes = size_t(MZATTN_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on the first
// call on the device, with that device current).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MZ_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MZ_ERR_UNSUPPORTED, "device index %d above %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(MZ_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MZ_OK;
}

}  // namespace

extern "C" {

int mzattn_decode_noalloc(const mzattn_decode_args* a, void* stream) {
  if (a == nullptr) return fail(MZ_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(mzattn_decode_args))
    return fail(MZ_ERR_ABI, "struct_size %u != sizeof(mzattn_decode_args) %zu", a->struct_size,
                sizeof(mzattn_decode_args));
  DecPlan pl;
  const int st = plan_decode(a, &pl);
  if (st != MZ_OK) return st;
  if (pl.bytes > kScratchBytes)
    return fail(MZ_ERR_WORKSPACE, "the step needs %zu bytes of scratch, above the %zu this entry point holds",
                pl.bytes, kScratchBytes);
  mzattn_decode_args d = *a;
  const int sa = scratch_address(&d.workspace);
  if (sa != MZ_OK) return sa;
  d.workspace_bytes = kScratchBytes;
  return run_decode(&d, stream);
}

}  // extern "C"

namespace {

int run_decode(const mzattn_decode_args* a, void* stream) {
  DecPlan pl;
  const int st = validate_decode_full(a, &pl);
  if (st != MZ_OK) return st;
  if (pl.empty) return ok();
  mz::DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.dtype = a->dtype;
  p.B = a->batch; p.Hq = a->heads_q; p.Hkv = a->heads_kv; p.G = a->heads_q / a->heads_kv;
  p.T = a->q_len; p.R = pl.R; p.C = a->cache_len; p.span = a->span; p.D = a->head_dim;
  p.n_chunks = pl.n_chunks;
  p.scale_log2 = scale_log2(a->scale, a->head_dim);
  char* ws = static_cast<char*>(a->workspace);
  if (a->rope_base > 0.0) {
    p.rope = 1;
    p.rope_style = a->rope_style;
    p.rs = rope_spec(a->rope_base, a->rope_precision, a->rope_mscale, a->rope_factors);
    p.q_in = a->q;
    for (int i = 0; i < 3; ++i) p.q_in_s[i] = a->q_stride[i];
    p.q_pos = a->q_pos; p.q_pos_sb = a->q_pos_stride_b;
    p.q = ws + pl.off_qrot;
    p.qs[0] = (int64_t)a->heads_q * a->q_len * a->head_dim;
    p.qs[1] = (int64_t)a->q_len * a->head_dim;
    p.qs[2] = a->head_dim;
  } else {
    p.q = a->q;
    for (int i = 0; i < 3; ++i) p.qs[i] = a->q_stride[i];
  }
  p.k = a->k_cache; p.v = a->v_cache; p.o = a->o;
  for (int i = 0; i < 3; ++i) { p.ks[i] = a->k_stride[i]; p.vs[i] = a->v_stride[i]; p.os[i] = a->o_stride[i]; }
  p.mask = a->mask;
  if (a->mask)
    for (int i = 0; i < 4; ++i) p.ms[i] = a->mask_stride[i];
  p.part_ml = reinterpret_cast<float2*>(ws + pl.off_ml);
  p.part_acc = reinterpret_cast<float*>(ws + pl.off_acc);
  const hipError_t e = mz::launch_decode(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MZ_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

// ---- decode with append ---------------------------------------------------
namespace {

// The shared checks of mzattn_decode on the equivalent call (whole-cache
// span, no q_pos rotation), then the append step's own.
int validate_append_full(const mzattn_decode_append_args* a, mzattn_decode_args* d, DecPlan* pl) {
  if (a == nullptr) return fail(MZ_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(mzattn_decode_append_args))
    return fail(MZ_ERR_ABI, "struct_size %u != sizeof(mzattn_decode_append_args) %zu", a->struct_size,
                sizeof(mzattn_decode_append_args));
  memset(d, 0, sizeof(*d));
  d->struct_size = sizeof(mzattn_decode_args);
  d->dtype = a->dtype;
  d->batch = a->batch; d->heads_q = a->heads_q; d->heads_kv = a->heads_kv; d->q_len = a->q_len;
  d->head_dim = a->head_dim; d->cache_len = a->cache_len; d->span = a->cache_len;
  d->scale = a->scale; d->rope_style = a->rope_style; d->rope_base = 0.0;
  d->q = a->q; d->k_cache = a->k_cache; d->v_cache = a->v_cache; d->o = a->o;
  for (int i = 0; i < 3; ++i) {
    d->q_stride[i] = a->q_stride[i]; d->k_stride[i] = a->k_stride[i];
    d->v_stride[i] = a->v_stride[i]; d->o_stride[i] = a->o_stride[i];
  }
  d->mask = a->mask;
  for (int i = 0; i < 4; ++i) d->mask_stride[i] = a->mask_stride[i];
  d->workspace = a->workspace; d->workspace_bytes = a->workspace_bytes;
  if (a->dtype == MZ_F32) return fail(MZ_ERR_UNSUPPORTED, "mzattn_decode_append supports bf16 and fp16");
  if (!isfinite(a->rope_base) || a->rope_base < 0.0 || a->rope_base == 1.0)
    return fail(MZ_ERR_VALUE, "rope_base must be finite, >= 0 and != 1");
  int st = check_rope_extra(a->rope_precision, a->rope_mscale, a->rope_factors);
  if (st != MZ_OK) return st;
  st = validate_decode_full(d, pl);
  if (st != MZ_OK || pl->empty) return st;
  if (a->cache_len < 1) return fail(MZ_ERR_SHAPE, "cache_len must be >= 1 to append");
  if (a->k_new == nullptr || a->v_new == nullptr) return fail(MZ_ERR_NULL, "k_new and v_new must not be NULL");
  if (!aligned(a->k_new, 16) || !aligned(a->v_new, 16)) return fail(MZ_ERR_ALIGN, "k_new / v_new not 16-byte aligned");
  if ((st = check_strides3(a->k_new_stride, 8, "k_new")) != MZ_OK) return st;
  if ((st = check_strides3(a->v_new_stride, 8, "v_new")) != MZ_OK) return st;
  if (a->len == nullptr) return fail(MZ_ERR_NULL, "len must not be NULL");
  if (a->len_stride_b < 0) return fail(MZ_ERR_STRIDE, "len_stride_b must be >= 0");
  return MZ_OK;
}

}  // namespace

extern "C" {

int mzattn_decode_append_workspace_size(const mzattn_decode_append_args* args, size_t* bytes) {
  if (bytes == nullptr) return fail(MZ_ERR_NULL, "bytes is NULL");
  if (args == nullptr) return fail(MZ_ERR_NULL, "args is NULL");
  if (args->struct_size != sizeof(mzattn_decode_append_args))
    return fail(MZ_ERR_ABI, "struct_size %u != sizeof(mzattn_decode_append_args) %zu", args->struct_size,
                sizeof(mzattn_decode_append_args));
  mzattn_decode_args d;
  memset(&d, 0, sizeof(d));
  d.struct_size = sizeof(d);
  d.dtype = args->dtype; d.batch = args->batch; d.heads_q = args->heads_q; d.heads_kv = args->heads_kv;
  d.q_len = args->q_len; d.head_dim = args->head_dim; d.cache_len = args->cache_len; d.span = args->cache_len;
  d.scale = args->scale; d.rope_style = args->rope_style;
  DecPlan pl;
  const int st = plan_decode(&d, &pl);
  if (st != MZ_OK) return st;
  *bytes = pl.bytes;
  return ok();
}

int mzattn_validate_decode_append(const mzattn_decode_append_args* args) {
  mzattn_decode_args d;
  DecPlan pl;
  const int st = validate_append_full(args, &d, &pl);
  return st == MZ_OK ? ok() : st;
}

int mzattn_decode_append(const mzattn_decode_append_args* a, void* stream) {
  mzattn_decode_args d;
  DecPlan pl;
  const int st = validate_append_full(a, &d, &pl);
  if (st != MZ_OK) return st;
  if (pl.empty) return ok();
  mz::DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.dtype = a->dtype;
  p.B = a->batch; p.Hq = a->heads_q; p.Hkv = a->heads_kv; p.G = a->heads_q / a->heads_kv;
  p.T = a->q_len; p.R = pl.R; p.C = a->cache_len; p.span = a->cache_len; p.D = a->head_dim;
  p.n_chunks = pl.n_chunks_max;
  p.scale_log2 = scale_log2(a->scale, a->head_dim);
  p.q = a->q;
  for (int i = 0; i < 3; ++i) p.qs[i] = a->q_stride[i];
  if (a->rope_base > 0.0) {
    p.rope = 1;
    p.rope_style = a->rope_style;
    p.rs = rope_spec(a->rope_base, a->rope_precision, a->rope_mscale, a->rope_factors);
  }
  p.k = a->k_cache; p.v = a->v_cache; p.o = a->o;
  p.k_w = a->k_cache; p.v_w = a->v_cache;
  for (int i = 0; i < 3; ++i) { p.ks[i] = a->k_stride[i]; p.vs[i] = a->v_stride[i]; p.os[i] = a->o_stride[i]; }
  p.mask = a->mask;
  if (a->mask)
    for (int i = 0; i < 4; ++i) p.ms[i] = a->mask_stride[i];
  p.app = 1;
  p.len = a->len; p.len_sb = a->len_stride_b;
  p.k_new = a->k_new; p.v_new = a->v_new;
  for (int i = 0; i < 3; ++i) { p.kn_s[i] = a->k_new_stride[i]; p.vn_s[i] = a->v_new_stride[i]; }
  p.overflow = a->overflow;
  char* ws = static_cast<char*>(a->workspace);
  p.part_ml = reinterpret_cast<float2*>(ws + pl.off_ml);
  p.part_acc = reinterpret_cast<float*>(ws + pl.off_acc);
  const hipError_t e = mz::launch_decode(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MZ_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
