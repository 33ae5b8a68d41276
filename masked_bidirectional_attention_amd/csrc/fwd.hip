// mzattn_fwd kernels for gfx950: prepasses, the bf16/fp16 MFMA main kernel
// and the fp32 kernel.
//
// What is computed (OmniVoice page, "What matches upstream", attention mask;
// "Memory and speed", packed_guidance; F5-TTS page, "How it works"):
// o_i = sum_j p_ij v_j / sum_j p_ij over the live keys j of query i, with
// p_ij = exp(scale * <q_i, k_j> - max), after interleaved RoPE on q and k.
// Non-live keys are removed by a select (their score becomes -inf before the
// max and their weight exactly 0), never by a finite bias.
#include "mz_common.h"
#include "mz_internal.h"

namespace mz {

// ---------------------------------------------------------------------------
// Prepass 1: cos/sin table of the rotary angles, positions [0, len).
// ---------------------------------------------------------------------------
__global__ void rope_table_kernel(float2* tab, int len, int D, double log2_base) {
  const int half = D / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)len * half) return;
  const int pos = (int)(idx / half), i = (int)(idx % half);
  tab[idx] = rope_cs_direct(pos, i, D, log2_base);
}

// ---------------------------------------------------------------------------
// Prepass 2 (segment mode): live key range of every query and, per query
// tile, the key tiles to visit and the ones that need no per-element check.
// Segment ids are non-decreasing along a row, so the keys sharing a query's
// id form one contiguous run, found by binary search.
// ---------------------------------------------------------------------------
__device__ inline int lower_bound_i32(const int32_t* row, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (row[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}
__device__ inline int upper_bound_i32(const int32_t* row, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (row[mid] <= v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ void seg_prep_kernel(const FwdParams p, int bm) {
  __shared__ int s_min_lo, s_max_hi, s_max_lo, s_min_hi;
  const int qt = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  if (t == 0) {
    s_min_lo = INT_MAX; s_max_hi = INT_MIN; s_max_lo = INT_MIN; s_min_hi = INT_MAX;
  }
  __syncthreads();
  const int32_t* sq = p.seg_q + b * p.seg_q_sb;
  const int32_t* sk = p.seg_k + b * p.seg_k_sb;
  for (int i = qt * bm + t; i < min((qt + 1) * bm, p.Sq); i += blockDim.x) {
    const int id = sq[i];
    int lo = 0, hi = 0;
    if (id >= 0) {
      lo = lower_bound_i32(sk, p.Sk, id);
      hi = upper_bound_i32(sk, p.Sk, id);
    }
    p.q_range[(int64_t)b * p.Sq + i] = make_int2(lo, hi);
    if (p.qpos_ws) p.qpos_ws[(int64_t)b * p.Sq + i] = i - lower_bound_i32(sq, p.Sq, id);
    if (hi > lo) {
      atomicMin(&s_min_lo, lo);
      atomicMax(&s_max_hi, hi);
    }
    atomicMax(&s_max_lo, hi > lo ? lo : 0);
    atomicMin(&s_min_hi, hi > lo ? hi : 0);
  }
  __syncthreads();
  if (t == 0) {
    int4 r;
    if (s_max_hi == INT_MIN) {  // no query of the tile has a live key
      r = make_int4(0, 0, 0, 0);
    } else {
      r.x = s_min_lo / FWD_BN;
      r.y = (s_max_hi + FWD_BN - 1) / FWD_BN;
      r.z = (s_max_lo + FWD_BN - 1) / FWD_BN;
      r.w = s_min_hi / FWD_BN;
      if (r.w < r.z) r.w = r.z;
    }
    p.qt_range[(int64_t)b * p.n_qt + qt] = r;
  }
}

// ---------------------------------------------------------------------------
// Prepass 3: rotate the K heads that get RoPE into the workspace (once per
// key, instead of once per query tile that visits it).
// ---------------------------------------------------------------------------
__device__ inline int key_position(const FwdParams& p, int b, int j) {
  if (p.pos_k_mode == POS_ARRAY) return p.pos_k[b * p.pos_k_sb + j];
  if (p.pos_k_mode == POS_SEGMENT) {
    const int32_t* sk = p.seg_k + b * p.seg_k_sb;
    return j - lower_bound_i32(sk, p.Sk, sk[j]);
  }
  return j;
}

__device__ inline int query_position(const FwdParams& p, int b, int i) {
  if (p.pos_q_mode == POS_ARANGE) return i;
  return p.pos_q[b * p.pos_q_sb + i];
}

template <typename T>
__global__ void k_rotate16_kernel(const FwdParams p) {
  const int half = p.D / 2;
  const int rows_per_blk = blockDim.x / half;
  const int64_t row = (int64_t)blockIdx.x * rows_per_blk + threadIdx.x / half;
  const int i = threadIdx.x % half;
  const int64_t nrows = (int64_t)p.B * p.n_rot_kv * p.Sk;
  if (row >= nrows) return;
  const int j = (int)(row % p.Sk);
  const int hk = (int)((row / p.Sk) % p.n_rot_kv);
  const int b = (int)(row / ((int64_t)p.Sk * p.n_rot_kv));
  const uint16_t* src = (const uint16_t*)p.k + b * p.ks[0] + hk * p.ks[1] + (int64_t)j * p.ks[2] + 2 * i;
  const uint32_t w = *(const uint32_t*)src;
  const float a = Elem<T>::to_f32((uint16_t)(w & 0xFFFF));
  const float c = Elem<T>::to_f32((uint16_t)(w >> 16));
  const float2 cs = rope_cs(p.rope_tab, p.rope_tab_len, key_position(p, b, j), i, p.D, p.log2_base);
  const float ra = fmaf(a, cs.x, -c * cs.y);
  const float rc = fmaf(c, cs.x, a * cs.y);
  ((uint32_t*)p.k_rot)[row * half + i] = Elem<T>::pack2(ra, rc);
}

__global__ void k_rotate32_kernel(const FwdParams p) {
  const int half = p.D / 2;
  const int rows_per_blk = blockDim.x / half;
  const int64_t row = (int64_t)blockIdx.x * rows_per_blk + threadIdx.x / half;
  const int i = threadIdx.x % half;
  const int64_t nrows = (int64_t)p.B * p.n_rot_kv * p.Sk;
  if (row >= nrows) return;
  const int j = (int)(row % p.Sk);
  const int hk = (int)((row / p.Sk) % p.n_rot_kv);
  const int b = (int)(row / ((int64_t)p.Sk * p.n_rot_kv));
  const float* src = (const float*)p.k + b * p.ks[0] + hk * p.ks[1] + (int64_t)j * p.ks[2] + 2 * i;
  const float2 x = *(const float2*)src;
  const float2 cs = rope_cs(p.rope_tab, p.rope_tab_len, key_position(p, b, j), i, p.D, p.log2_base);
  float2 r;
  r.x = fmaf(x.x, cs.x, -x.y * cs.y);
  r.y = fmaf(x.y, cs.x, x.x * cs.y);
  ((float2*)p.k_rot)[row * half + i] = r;
}

// ---------------------------------------------------------------------------
// Prepass 4 (boolean mask): one class byte per (query tile, key tile):
// 0 = no live pair (skipped without touching K/V), 1 = every in-range pair
// live (no mask reads), 2 = mixed (mask read per element).
// ---------------------------------------------------------------------------
__global__ void mask_tiles_kernel(const FwdParams p, int bm) {
  const int64_t tile = blockIdx.x;
  const int kt = (int)(tile % p.n_kt);
  const int qt = (int)((tile / p.n_kt) % p.n_qt);
  const int bh = (int)(tile / ((int64_t)p.n_kt * p.n_qt));
  const int bb = bh / p.Hm, hh = bh % p.Hm;
  const uint8_t* base = p.mask + bb * p.ms[0] + hh * p.ms[1];
  const int q_lo = qt * bm, k_lo = kt * FWD_BN;
  const int nq = p.ms[2] == 0 ? 1 : min(bm, p.Sq - q_lo);
  const int nk = min(FWD_BN, p.Sk - k_lo);
  int any = 0, all = 1;
  if (p.mask_vec16 && nk == FWD_BN) {
    // rows are 16-byte aligned: 4 x 16 bytes per row
    for (int idx = threadIdx.x; idx < nq * 4; idx += blockDim.x) {
      const int r = idx >> 2, c = idx & 3;
      const uint4 v = *(const uint4*)(base + (int64_t)(q_lo + r) * p.ms[2] + k_lo + c * 16);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // a byte is live iff nonzero
        const uint32_t x = w[e];
        const uint32_t nz = ((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x;  // high bit of each byte = byte != 0
        const uint32_t hi = nz & 0x80808080u;
        any |= hi != 0;
        all &= hi == 0x80808080u;
      }
    }
  } else {
    for (int idx = threadIdx.x; idx < nq * nk; idx += blockDim.x) {
      const int r = idx / nk, c = idx % nk;
      const int v = base[(int64_t)(q_lo + r) * p.ms[2] + k_lo + c] != 0;
      any |= v;
      all &= v;
    }
  }
  any = __syncthreads_or(any);
  all = __syncthreads_and(all);
  if (threadIdx.x == 0) p.tile_cls[tile] = !any ? 0 : (all ? 1 : 2);
}

// ---------------------------------------------------------------------------
// Main kernel, bf16 / fp16, MFMA 32x32x16.
//
// One work-group = (b, h, 128 queries); 4 waves of 32 queries each.  Scores
// are computed transposed, S^T = K Q^T, so that every lane owns one query:
// the row max and row sum need one cross-lane exchange (lanes l, l^32) and
// the output O^T = V^T P^T is rescaled lane-locally.  P^T leaves the
// accumulator registers directly as the B operand of the P.V MFMA; V^T comes
// from LDS through the transposing read.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256, 2) void fwd_mfma_kernel(const FwdParams p) {
  constexpr int BM = FWD_BM, BN = FWD_BN;
  constexpr int KS = D + 8;   // LDS row stride (elements) of K
  constexpr int VS = D + 16;  // LDS row stride (elements) of V
  constexpr int NS = D / 16;  // k-steps of K Q^T
  constexpr int ND = D / 32;  // 32-row d blocks of O^T
  constexpr int CH = D / 8;   // 16-byte chunks per row
  constexpr int RPP = 256 / CH;
  constexpr int NP = BN / RPP;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BN * VS];

  const int nwork = p.B * p.Hq * p.n_qt;
  const int w = xcd_remap(blockIdx.x, nwork);
  const int qt = w % p.n_qt;
  const int bh = w / p.n_qt;
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int hk = h / p.G;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int qi = qt * BM + wave * 32 + l32;
  const bool qvalid = qi < p.Sq;

  // ---- Q fragment: B operand of S^T = K Q^T (query l32, d = s*16 + hh*8 + e)
  uint4 qf[NS];
  {
    const uint16_t* qrow = (const uint16_t*)p.q + b * p.qs[0] + h * p.qs[1] + (int64_t)qi * p.qs[2];
    const bool rot = h < p.n_rot;
    const int qpos = (rot && qvalid) ? query_position(p, b, qi) : 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (qvalid) {
        x = *(const uint4*)(qrow + s * 16 + hh * 8);
        if (rot) x = rope_quad<T>(x, p.rope_tab, p.rope_tab_len, qpos, s * 16 + hh * 8, D, p.log2_base);
      }
      qf[s] = x;
    }
  }

  // ---- K / V sources
  const uint16_t* kbase;
  int64_t kstride;
  if (hk < p.n_rot_kv) {
    kbase = (const uint16_t*)p.k_rot + ((int64_t)(b * p.n_rot_kv + hk) * p.Sk) * D;
    kstride = D;
  } else {
    kbase = (const uint16_t*)p.k + b * p.ks[0] + hk * p.ks[1];
    kstride = p.ks[2];
  }
  const uint16_t* vbase = (const uint16_t*)p.v + b * p.vs[0] + hk * p.vs[1];
  const int64_t vstride = p.vs[2];

  // ---- which key tiles to visit
  int kt_beg = 0, kt_end = p.n_kt, full_beg = 0, full_end = 0;
  int lo = 0, hi = p.Sk;
  const uint8_t* cls_row = nullptr;
  const uint8_t* mrow = nullptr;
  if (p.mask_kind == 2) {
    const int4 r = p.qt_range[(int64_t)b * p.n_qt + qt];
    kt_beg = r.x; kt_end = r.y; full_beg = r.z; full_end = r.w;
    if (qvalid) {
      const int2 qr = p.q_range[(int64_t)b * p.Sq + qi];
      lo = qr.x; hi = qr.y;
    } else {
      lo = 0; hi = 0;
    }
  } else if (p.mask_kind == 1) {
    const int bm_ = p.Bm == 1 ? 0 : b, hm_ = p.Hm == 1 ? 0 : h;
    cls_row = p.tile_cls + ((int64_t)(bm_ * p.Hm + hm_) * p.n_qt + qt) * p.n_kt;
    if (qvalid) mrow = p.mask + b * p.ms[0] + h * p.ms[1] + (int64_t)qi * p.ms[2];
  }
  const int first_tail_tile = p.Sk / BN;  // tiles from here on reach past Sk

  uint4 kreg[NP], vreg[NP];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int r = pp * RPP + tid / CH, c = tid % CH;
      const int key = kt * BN + r;
      if (key < p.Sk) {
        kreg[pp] = *(const uint4*)(kbase + (int64_t)key * kstride + c * 8);
        vreg[pp] = *(const uint4*)(vbase + (int64_t)key * vstride + c * 8);
      } else {
        kreg[pp] = make_uint4(0, 0, 0, 0);
        vreg[pp] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto next_live = [&](int kt) {
    if (cls_row) {
      while (kt < kt_end && cls_row[kt] == 0) ++kt;
    }
    return kt;
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;

  const int grp = lane >> 4, gi = lane & 15, rr = gi >> 2, cc = gi & 3;

  int kt = next_live(kt_beg);
  if (kt < kt_end) load_tile(kt);
  while (kt < kt_end) {
    __syncthreads();
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int r = pp * RPP + tid / CH, c = tid % CH;
      *(uint4*)&Ks[r * KS + c * 8] = kreg[pp];
      *(uint4*)&Vs[r * VS + c * 8] = vreg[pp];
    }
    __syncthreads();
    const int kt_next = next_live(kt + 1);
    if (kt_next < kt_end) load_tile(kt_next);

    bool check;
    if (p.mask_kind == 2) check = !(kt >= full_beg && kt < full_end);
    else if (p.mask_kind == 1) check = cls_row[kt] == 2 || kt >= first_tail_tile;
    else check = kt >= first_tail_tile;

    // ---- S^T = K Q^T for two 32-key blocks
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint4 a = *(const uint4*)&Ks[(kb * 32 + l32) * KS + s * 16 + hh * 8];
        sacc[kb] = mfma32<T>(a, qf[s], sacc[kb]);
      }
    }

    // ---- scale into the log2 domain; remove non-live keys
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = sacc[kb][v] * p.scale_log2;
        if (check) {
          const int key = kt * BN + kb * 32 + (v >> 2) * 8 + hh * 4 + (v & 3);
          bool live;
          if (p.mask_kind == 2) live = key >= lo && key < hi;
          else if (p.mask_kind == 1) live = key < p.Sk && mrow != nullptr && mrow[key] != 0;
          else live = key < p.Sk;
          x = live ? x : -INFINITY;
        }
        sacc[kb][v] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = wave_xor_max(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float ls = 0.f;
    uint4 pk[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        uint32_t wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(sacc[kb][jj * 8 + 2 * e] - m_use);
          const float p1 = fast_exp2(sacc[kb][jj * 8 + 2 * e + 1] - m_use);
          ls += p0 + p1;
          wv[e] = Elem<T>::pack2(p0, p1);
        }
        pk[kb][jj] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
    }
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int col = db * 32 + (grp & 1) * 16 + 4 * cc;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int row0 = kb * 32 + jj * 16 + 4 * hh + rr;
          const uint2 a0 = lds_read_tr<T>(&Vs[row0 * VS + col]);
          const uint2 a1 = lds_read_tr<T>(&Vs[(row0 + 8) * VS + col]);
          oacc[db] = mfma32<T>(make_uint4(a0.x, a0.y, a1.x, a1.y), pk[kb][jj], oacc[db]);
        }
      }
    }
    kt = kt_next;
  }

  // ---- epilogue: O = O^T / l, lse
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qvalid) {
    uint16_t* orow = (uint16_t*)p.o + b * p.os[0] + h * p.os[1] + (int64_t)qi * p.os[2];
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hh * 4;
        uint2 st;
        st.x = Elem<T>::pack2(oacc[db][g4 * 4 + 0] * inv, oacc[db][g4 * 4 + 1] * inv);
        st.y = Elem<T>::pack2(oacc[db][g4 * 4 + 2] * inv, oacc[db][g4 * 4 + 3] * inv);
        *(uint2*)(orow + d) = st;
      }
    }
    if (p.lse != nullptr && hh == 0)
      p.lse[((int64_t)b * p.Hq + h) * p.Sq + qi] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: one wave per 64 queries, one lane per query, fp32 FMA.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const FwdParams p) {
  constexpr int BM = F32_BM, SUB = 16;
  __shared__ float Qs[BM][D + 1];  // each lane's own (rotated, scaled) query row
  __shared__ float Ks[SUB][D];
  __shared__ float Vs[SUB][D];
  const int nwork = p.B * p.Hq * p.n_qt;
  const int w = blockIdx.x;
  if (w >= nwork) return;
  const int qt = w % p.n_qt;
  const int bh = w / p.n_qt;
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int hk = h / p.G;
  const int lane = threadIdx.x;
  const int qi = qt * BM + lane;
  const bool qvalid = qi < p.Sq;

  {
    const float* qrow = (const float*)p.q + b * p.qs[0] + h * p.qs[1] + (int64_t)qi * p.qs[2];
    const bool rot = h < p.n_rot;
    const int qpos = (rot && qvalid) ? query_position(p, b, qi) : 0;
    for (int i = 0; i < D / 2; ++i) {
      float2 x = qvalid ? *(const float2*)(qrow + 2 * i) : make_float2(0.f, 0.f);
      if (rot && qvalid) {
        const float2 cs = rope_cs(p.rope_tab, p.rope_tab_len, qpos, i, D, p.log2_base);
        const float a = fmaf(x.x, cs.x, -x.y * cs.y);
        const float c = fmaf(x.y, cs.x, x.x * cs.y);
        x = make_float2(a, c);
      }
      Qs[lane][2 * i] = x.x * p.scale_log2;
      Qs[lane][2 * i + 1] = x.y * p.scale_log2;
    }
  }
  const float* kbase;
  int64_t kstride;
  if (hk < p.n_rot_kv) {
    kbase = (const float*)p.k_rot + ((int64_t)(b * p.n_rot_kv + hk) * p.Sk) * D;
    kstride = D;
  } else {
    kbase = (const float*)p.k + b * p.ks[0] + hk * p.ks[1];
    kstride = p.ks[2];
  }
  const float* vbase = (const float*)p.v + b * p.vs[0] + hk * p.vs[1];

  int kt_beg = 0, kt_end = p.n_kt;
  int lo = 0, hi = p.Sk;
  const uint8_t* cls_row = nullptr;
  const uint8_t* mrow = nullptr;
  if (p.mask_kind == 2) {
    const int4 r = p.qt_range[(int64_t)b * p.n_qt + qt];
    kt_beg = r.x; kt_end = r.y;
    if (qvalid) {
      const int2 qr = p.q_range[(int64_t)b * p.Sq + qi];
      lo = qr.x; hi = qr.y;
    } else {
      lo = 0; hi = 0;
    }
  } else if (p.mask_kind == 1) {
    const int bm_ = p.Bm == 1 ? 0 : b, hm_ = p.Hm == 1 ? 0 : h;
    cls_row = p.tile_cls + ((int64_t)(bm_ * p.Hm + hm_) * p.n_qt + qt) * p.n_kt;
    if (qvalid) mrow = p.mask + b * p.ms[0] + h * p.ms[1] + (int64_t)qi * p.ms[2];
  }

  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int kt = kt_beg; kt < kt_end; ++kt) {
    if (cls_row && cls_row[kt] == 0) continue;
    for (int sub = 0; sub < FWD_BN / SUB; ++sub) {
      const int key0 = kt * FWD_BN + sub * SUB;
      if (key0 >= p.Sk) break;
      __syncthreads();
      for (int idx = lane; idx < SUB * D; idx += 64) {
        const int r = idx / D, d = idx % D;
        const int key = key0 + r;
        Ks[r][d] = key < p.Sk ? kbase[(int64_t)key * kstride + d] : 0.f;
        Vs[r][d] = key < p.Sk ? vbase[(int64_t)key * p.vs[2] + d] : 0.f;
      }
      __syncthreads();
      float s[SUB];
      float mx = -INFINITY;
      for (int r = 0; r < SUB; ++r) {
        const int key = key0 + r;
        bool live;
        if (p.mask_kind == 2) live = key >= lo && key < hi;
        else if (p.mask_kind == 1) live = key < p.Sk && mrow != nullptr && mrow[key] != 0;
        else live = key < p.Sk;
        float acc = 0.f;
#pragma unroll 16
        for (int d = 0; d < D; ++d) acc = fmaf(Qs[lane][d], Ks[r][d], acc);
        s[r] = live ? acc : -INFINITY;
        mx = fmaxf(mx, s[r]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= alpha;
      for (int r = 0; r < SUB; ++r) {
        const float pr = exp2f(s[r] - m_use);
        l_run += pr;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(pr, Vs[r][d], o[d]);
      }
      m_run = m_new;
    }
  }
  if (qvalid) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* orow = (float*)p.o + b * p.os[0] + h * p.os[1] + (int64_t)qi * p.os[2];
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
    if (p.lse != nullptr)
      p.lse[((int64_t)b * p.Hq + h) * p.Sq + qi] =
          l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994530942f : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_fwd_plan(const FwdParams& p, hipStream_t s) {
  const bool f32 = p.dtype == 0;
  const int bm = f32 ? F32_BM : FWD_BM;
  if (p.n_rot > 0 && p.rope_tab_len > 0) {
    const int64_t n = (int64_t)p.rope_tab_len * (p.D / 2);
    rope_table_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(p.rope_tab, p.rope_tab_len, p.D,
                                                                              p.log2_base);
  }
  if (p.mask_kind == 2) seg_prep_kernel<<<dim3(p.n_qt, p.B), dim3(bm), 0, s>>>(p, bm);
  if (p.n_rot_kv > 0) {
    const int rows_per_blk = 256 / (p.D / 2);
    const int64_t nrows = (int64_t)p.B * p.n_rot_kv * p.Sk;
    const unsigned nblk = (unsigned)((nrows + rows_per_blk - 1) / rows_per_blk);
    if (f32) k_rotate32_kernel<<<dim3(nblk), dim3(256), 0, s>>>(p);
    else if (p.dtype == 2) k_rotate16_kernel<BF16><<<dim3(nblk), dim3(256), 0, s>>>(p);
    else k_rotate16_kernel<F16><<<dim3(nblk), dim3(256), 0, s>>>(p);
  }
  if (p.mask_kind == 1) {
    const int64_t ntiles = (int64_t)p.Bm * p.Hm * p.n_qt * p.n_kt;
    mask_tiles_kernel<<<dim3((unsigned)ntiles), dim3(256), 0, s>>>(p, bm);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_main(const FwdParams& p, hipStream_t s) {
  const bool f32 = p.dtype == 0;
  const unsigned nwork = (unsigned)((int64_t)p.B * p.Hq * p.n_qt);
  if (f32) {
    if (p.D == 64) fwd_f32_kernel<64><<<dim3(nwork), dim3(64), 0, s>>>(p);
    else fwd_f32_kernel<128><<<dim3(nwork), dim3(64), 0, s>>>(p);
  } else if (p.dtype == 2) {
    if (p.D == 64) fwd_mfma_kernel<BF16, 64><<<dim3(nwork), dim3(256), 0, s>>>(p);
    else fwd_mfma_kernel<BF16, 128><<<dim3(nwork), dim3(256), 0, s>>>(p);
  } else {
    if (p.D == 64) fwd_mfma_kernel<F16, 64><<<dim3(nwork), dim3(256), 0, s>>>(p);
    else fwd_mfma_kernel<F16, 128><<<dim3(nwork), dim3(256), 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace mz
