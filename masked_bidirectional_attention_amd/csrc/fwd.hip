// mzattn_fwd kernels for gfx950: prepasses, the bf16/fp16 MFMA main kernel
// and the fp32 kernel.
//
// What is computed (OmniVoice page, "What matches upstream", attention mask;
// "Memory and speed", packed_guidance; F5-TTS page, "How it works"):
// o_i = sum_j p_ij v_j / sum_j p_ij over the live keys j of query i, with
// p_ij = exp(scale * <q_i, k_j> - max), after interleaved RoPE on q and k.
// Non-live keys are removed by a select (their score becomes -inf before the
// max and their weight exactly 0), never by a finite bias.
#include <atomic>

#include "fwd_mfma.h"
#include "mz_common.h"
#include "mz_internal.h"

namespace mz {

// ---------------------------------------------------------------------------
// Prepass 1: cos/sin of the rotary angles, one launch for three ranges of
// rows (all by the same formula, so a position gives the same bits
// wherever it is held):
//   the table, row j = position j, j < tab_len (index positions read it);
//   the query rows, row b * Sq + i = position pos_q[b * pos_q_sb + i], for
//   q_rows_b batch rows, when the positions are given or derived from
//   segments;
//   the key rows likewise;
//   for the 16-bit kernels, the query rows again in chunk-major order (the
//   16-byte chunk c of every query of a batch row, then chunk c + 1), so
//   that the 32 queries of a wave read contiguous bytes in the Q prologue.
// The kernels after the plan read these rows and need neither the
// positions nor the direct formula.  In segment mode it runs after the
// segment prepass, which derives the positions.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rope_prep_kernel(const FwdParams p) {
  __shared__ double theta[64];
  const int half = p.D / 2;
  if (threadIdx.x < half) theta[threadIdx.x] = rope_theta(threadIdx.x, p.D, p.rs);
  __syncthreads();
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_tab = (int64_t)p.rope_tab_len * half;
  const int64_t n_q = p.q_rows != nullptr ? (int64_t)p.q_rows_b * p.Sq * half : 0;
  const int64_t n_k = p.k_rows != nullptr ? (int64_t)p.k_rows_b * p.Sk * half : 0;
  const int64_t n_c = p.q_cst != nullptr ? (int64_t)p.q_cst_b * p.Sq * half : 0;
  const int i = (int)(idx % half);
  if (idx < n_tab) {
    p.rope_tab[idx] = rope_cs_theta((int)(idx / half), theta[i], p.rs);
    return;
  }
  idx -= n_tab;
  if (idx < n_q) {
    const int64_t r = idx / half;
    const int j = (int)(r % p.Sq), b = (int)(r / p.Sq);
    p.q_rows[idx] = rope_cs_theta(p.pos_q[b * p.pos_q_sb + j], theta[i], p.rs);
    return;
  }
  idx -= n_q;
  if (idx < n_k) {
    const int64_t r = idx / half;
    const int j = (int)(r % p.Sk), b = (int)(r / p.Sk);
    p.k_rows[idx] = rope_cs_theta(p.pos_k[b * p.pos_k_sb + j], theta[i], p.rs);
    return;
  }
  idx -= n_k;
  if (idx < n_c) {
    // chunk-major query rows: element idx is pair 2c + e of query j, batch
    // row b, at ((b * D/4 + c) * Sq + j) * 2 + e
    const int e = (int)(idx & 1);
    const int64_t r = idx >> 1;
    const int j = (int)(r % p.Sq);
    const int64_t r2 = r / p.Sq;
    const int c = (int)(r2 % (half / 2)), b = (int)(r2 / (half / 2));
    const int pos = p.pos_q_mode == POS_ARANGE ? j : p.pos_q[b * p.pos_q_sb + j];
    reinterpret_cast<float2*>(p.q_cst)[idx] = rope_cs_theta(pos, theta[2 * c + e], p.rs);
  }
}

// ---------------------------------------------------------------------------
// Prepass 2 (segment mode): live key range of every query and, per query
// tile, the key tiles to visit and the ones that need no per-element check.
// Segment ids are non-decreasing along a row, so the keys sharing a query's
// id form one contiguous run, found by binary search.
// ---------------------------------------------------------------------------
// Rows of up to SEG_LDS ids are searched in LDS (one coalesced load per
// block instead of a chain of dependent global loads); longer rows are
// searched in global memory.
constexpr int SEG_LDS = 4096;

// Binary searches over a non-decreasing id row.  Row is either an LDS array
// (indexed directly, so the compiler emits LDS reads) or a global pointer.
template <typename Row>
__device__ inline int seg_lower(Row row, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (row[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}
template <typename Row>
__device__ inline int seg_upper(Row row, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (row[mid] <= v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <typename KRow, typename QRow>
__device__ void seg_prep_body(const FwdParams& p, int bm, int bx, int b, KRow K, QRow Q, int* red) {
  const int t = threadIdx.x;
  // key positions: index within the key's run of equal ids
  if (p.kpos_ws) {
    const int j = bx * 256 + t;
    if (j < p.Sk) p.kpos_ws[(int64_t)b * p.Sk + j] = j - seg_lower(K, p.Sk, K[j]);
  }
  if (bx >= p.n_qt) return;  // uniform per block
  const int i = bx * bm + t;
  // per-lane contributions; lanes without a query give the identities
  int a0 = INT_MAX, a1 = INT_MIN, a2 = INT_MIN, a3 = INT_MAX;
  if (t < bm && i < p.Sq) {
    const int id = Q[i];
    int lo = 0, hi = 0;
    if (id >= 0) {
      lo = seg_lower(K, p.Sk, id);
      hi = seg_upper(K, p.Sk, id);
    }
    p.q_range[(int64_t)b * p.Sq + i] = make_int2(lo, hi);
    if (p.qpos_ws) p.qpos_ws[(int64_t)b * p.Sq + i] = i - seg_lower(Q, p.Sq, id);
    const bool live = hi > lo;
    a0 = live ? lo : INT_MAX;  // min over queries with live keys
    a1 = live ? hi : INT_MIN;  // max over queries with live keys
    a2 = live ? lo : 0;        // max over all queries (empty ranges count as 0)
    a3 = live ? hi : 0;        // min over all queries
  }
  // wave-level reductions (every lane takes part), one LDS atomic per wave
  for (int off = 32; off > 0; off >>= 1) {
    a0 = min(a0, __shfl_xor(a0, off, 64));
    a1 = max(a1, __shfl_xor(a1, off, 64));
    a2 = max(a2, __shfl_xor(a2, off, 64));
    a3 = min(a3, __shfl_xor(a3, off, 64));
  }
  if ((t & 63) == 0) {
    atomicMin(&red[0], a0);
    atomicMax(&red[1], a1);
    atomicMax(&red[2], a2);
    atomicMin(&red[3], a3);
  }
}

// grid (max(n_qt, ceil(Sk / 256)), B), 256 threads.  Block x handles query
// tile x (if any) and keys [256 x, 256 x + 256) (derived key positions).
__global__ __launch_bounds__(256) void seg_prep_kernel(const FwdParams p, int bm) {
  __shared__ int32_t sk_l[SEG_LDS];
  __shared__ int32_t sq_l[SEG_LDS];
  __shared__ int red[4];
  const int bx = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int32_t* sq = p.seg_q + b * p.seg_q_sb;
  const int32_t* sk = p.seg_k + b * p.seg_k_sb;
  const bool same = sq == sk && p.Sq == p.Sk;
  const bool k_lds = p.Sk <= SEG_LDS, q_lds = !same && p.Sq <= SEG_LDS;
  // copy the rows with every load in flight at once (SEG_LDS / 256 each)
  constexpr int PER = SEG_LDS / 256;
  if (k_lds) {
    int32_t v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) v[u] = t + u * 256 < p.Sk ? sk[t + u * 256] : 0;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (t + u * 256 < p.Sk) sk_l[t + u * 256] = v[u];
  }
  if (q_lds) {
    int32_t v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) v[u] = t + u * 256 < p.Sq ? sq[t + u * 256] : 0;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (t + u * 256 < p.Sq) sq_l[t + u * 256] = v[u];
  }
  if (t == 0) {
    red[0] = INT_MAX; red[1] = INT_MIN; red[2] = INT_MIN; red[3] = INT_MAX;
  }
  __syncthreads();
  if (k_lds && same) seg_prep_body(p, bm, bx, b, sk_l, sk_l, red);
  else if (k_lds && q_lds) seg_prep_body(p, bm, bx, b, sk_l, sq_l, red);
  else if (k_lds) seg_prep_body(p, bm, bx, b, sk_l, sq, red);
  else if (same) seg_prep_body(p, bm, bx, b, sk, sk, red);
  else if (q_lds) seg_prep_body(p, bm, bx, b, sk, sq_l, red);
  else seg_prep_body(p, bm, bx, b, sk, sq, red);
  __syncthreads();
  if (t == 0 && bx < p.n_qt) {
    int4 r;
    if (red[1] == INT_MIN) {  // no query of the tile has a live key
      r = make_int4(0, 0, 0, 0);
    } else {
      r.x = red[0] / FWD_BN;
      r.y = (red[1] + FWD_BN - 1) / FWD_BN;
      r.z = (red[2] + FWD_BN - 1) / FWD_BN;
      r.w = red[3] / FWD_BN;
      if (r.w < r.z) r.w = r.z;
    }
    p.qt_range[(int64_t)b * p.n_qt + bx] = r;
  }
}

// ---------------------------------------------------------------------------
// Prepass 3: rotate the K heads that get RoPE into the workspace (once per
// key, instead of once per query tile that visits it).
// ---------------------------------------------------------------------------

// One thread per 8 consecutive elements of a K row: 4 adjacent pairs
// (interleaved), or with HALF 8 elements of the first half and their 8
// partners D/2 further (half split).  The q8 threads of a row are adjacent
// lanes, so the row's sum of squares (RMSNorm of k) is a reduction over
// them.  Heads below n_rotk are rotated; all are normalised when k_norm_w
// is set.  Grid: x over the Sk * q8 threads of one (batch, head) (32-bit
// index math), y the K head, z the batch row.  gridDim.x is a multiple of 8,
// so block x runs on XCD x % 8 in every (head, batch) slab; the remap gives
// each XCD one contiguous eighth of the key rows, and with it one eighth of
// the cos/sin table rows in its L2 instead of most of the table.
template <typename T, bool HALF>
__global__ __launch_bounds__(256) void k_rotate16_kernel(const FwdParams p) {
  const int q8 = HALF ? p.D / 16 : p.D / 8;
  const int idx = xcd_remap((int)blockIdx.x, (int)gridDim.x) * 256 + (int)threadIdx.x;
  if (idx >= p.Sk * q8) return;  // whole rows only (q8 divides the block)
  const int hk = (int)blockIdx.y, b = (int)blockIdx.z;
  const int j = idx / q8;
  const int d0 = (idx - j * q8) * 8;
  const bool rot = hk < p.n_rotk;  // uniform over the block
  const int64_t row = ((int64_t)b * p.n_rot_kv + hk) * p.Sk + j;
  const uint16_t* src = (const uint16_t*)p.k + b * p.ks[0] + hk * p.ks[1] + (int64_t)j * p.ks[2] + d0;
  uint16_t* dst = (uint16_t*)p.k_rot + row * p.D + d0;
  const int hd = p.D / 2;
  constexpr int NE = HALF ? 16 : 8;
  float x[NE];  // HALF: x[0..7] at d0 + e, x[8..15] at d0 + hd + e
  const u32x4_t a0 = *(const u32x4_t*)src;
  u32x4_t a1 = {0u, 0u, 0u, 0u};
  if constexpr (HALF) a1 = *(const u32x4_t*)(src + hd);
  // RMSNorm weights of the same elements (16-byte vectors, issued early)
  const bool norm = p.k_norm_w != nullptr;
  u32x4_t wv0 = {0u, 0u, 0u, 0u}, wv1 = wv0;
  if (norm) {
    const uint16_t* wp = (const uint16_t*)p.k_norm_w + d0;
    wv0 = *(const u32x4_t*)wp;
    if constexpr (HALF) wv1 = *(const u32x4_t*)(wp + hd);
  }
  // the pairs' cos / sin from the key's cos / sin row, read as 16-byte
  // vectors issued with the K row (no dependent load)
  constexpr int NP = HALF ? 8 : 4;    // pairs of this thread
  const int i0 = HALF ? d0 : d0 / 2;  // first pair index (a multiple of 4)
  float4 tv[NP / 2];
  if (rot) {
    const float4* trow = (const float4*)(p.k_cs + ((size_t)b * p.k_cs_sb + j) * (p.D / 2) + i0);
#pragma unroll
    for (int u = 0; u < NP / 2; ++u) tv[u] = trow[u];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = Elem<T>::to_f32((uint16_t)(a0[e / 2] >> (16 * (e & 1))));
  if constexpr (HALF) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[8 + e] = Elem<T>::to_f32((uint16_t)(a1[e / 2] >> (16 * (e & 1))));
  }
  if (norm) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) ss = fmaf(x[e], x[e], ss);
    for (int off = q8 / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = rsqrtf(ss / (float)p.D + p.norm_eps);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const uint32_t w = (e < 8 ? wv0 : wv1)[(e & 7) / 2];
      x[e] = x[e] * inv * Elem<T>::to_f32((uint16_t)(w >> (16 * (e & 1))));
    }
  }
  if (rot) {
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      // pair: interleaved (x[2t], x[2t+1]) of pair index d0/2 + t; half
      // split (x[t], x[8+t]) of pair index d0 + t
      const int ia = HALF ? t : 2 * t, ic = HALF ? 8 + t : 2 * t + 1;
      const float2 cs = (t & 1) ? make_float2(tv[t / 2].z, tv[t / 2].w) : make_float2(tv[t / 2].x, tv[t / 2].y);
      const float a = x[ia], c = x[ic];
      x[ia] = fmaf(a, cs.x, -c * cs.y);
      x[ic] = fmaf(c, cs.x, a * cs.y);
    }
  }
  uint32_t o0[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) o0[t] = Elem<T>::pack2(x[2 * t], x[2 * t + 1]);
  *(uint4*)dst = make_uint4(o0[0], o0[1], o0[2], o0[3]);
  if constexpr (HALF) {
    uint32_t o1[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) o1[t] = Elem<T>::pack2(x[8 + 2 * t], x[8 + 2 * t + 1]);
    *(uint4*)(dst + hd) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
  }
}

// fp32: one thread per pair; the D/2 threads of a row are adjacent lanes.
// Grid as for the 16-bit pass: x over the key rows of one (batch, head), a
// multiple of 8 remapped per XCD, y the K head, z the batch row.
__global__ void k_rotate32_kernel(const FwdParams p) {
  const int half = p.D / 2;
  const int rows_per_blk = 256 / half;
  const int j = xcd_remap((int)blockIdx.x, (int)gridDim.x) * rows_per_blk + (int)threadIdx.x / half;
  const int i = (int)threadIdx.x % half;
  if (j >= p.Sk) return;  // whole rows only
  const int hk = (int)blockIdx.y, b = (int)blockIdx.z;
  const int64_t row = ((int64_t)b * p.n_rot_kv + hk) * p.Sk + j;
  // pair i: (2i, 2i+1) interleaved, (i, i + D/2) half split
  const int d0 = p.rope_style == 1 ? i : 2 * i, d1 = p.rope_style == 1 ? i + half : 2 * i + 1;
  const float* src = (const float*)p.k + b * p.ks[0] + hk * p.ks[1] + (int64_t)j * p.ks[2];
  float2 x = make_float2(src[d0], src[d1]);
  if (p.k_norm_w != nullptr) {
    float ss = fmaf(x.x, x.x, x.y * x.y);
    for (int off = half / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = rsqrtf(ss / (float)p.D + p.norm_eps);
    const float* wp = (const float*)p.k_norm_w;
    x = make_float2(x.x * inv * wp[d0], x.y * inv * wp[d1]);
  }
  if (hk < p.n_rotk) {
    const float2 cs = p.k_cs[((size_t)b * p.k_cs_sb + j) * half + i];
    x = make_float2(fmaf(x.x, cs.x, -x.y * cs.y), fmaf(x.y, cs.x, x.x * cs.y));
  }
  float* dst = (float*)p.k_rot + row * p.D;
  dst[d0] = x.x;
  dst[d1] = x.y;
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
  // key bits: written once per mask row (a broadcast row by query tile 0)
  uint16_t* bits = nullptr;
  if (p.mask_bits != nullptr && (p.ms[2] != 0 || qt == 0))
    bits = reinterpret_cast<uint16_t*>(p.mask_bits + ((int64_t)bh * p.mask_rows + (p.ms[2] == 0 ? 0 : q_lo)) * p.n_kt + kt);
  int any = 0, all = 1;
  // one item = 16 keys of one row: 16 key bits, and their share of the class
  for (int idx = threadIdx.x; idx < nq * 4; idx += blockDim.x) {
    const int r = idx >> 2, c = idx & 3;
    const uint8_t* row = base + (int64_t)(q_lo + r) * p.ms[2] + k_lo + c * 16;
    const int n = min(16, nk - c * 16);  // keys of this item below Sk
    uint32_t m16 = 0;
    if (p.mask_vec16 && n == 16) {
      const uint4 v = *(const uint4*)row;
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // high bit of each byte = byte != 0
        const uint32_t x = w[e];
        const uint32_t hi = (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
        m16 |= (((hi >> 7) & 1u) | ((hi >> 14) & 2u) | ((hi >> 21) & 4u) | ((hi >> 28) & 8u)) << (4 * e);
      }
    } else {
      for (int e = 0; e < n; ++e) m16 |= (uint32_t)(row[e] != 0) << e;
    }
    if (n > 0) {
      const uint32_t full = n == 16 ? 0xFFFFu : ((1u << n) - 1u);
      any |= m16 != 0;
      all &= m16 == full;
    }
    if (bits != nullptr) bits[(int64_t)r * p.n_kt * 4 + c] = (uint16_t)m16;
  }
  any = __syncthreads_or(any);
  all = __syncthreads_and(all);
  if (threadIdx.x == 0) p.tile_cls[tile] = !any ? 0 : (all ? 1 : 2);
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
    const float2* qcs = p.q_cs + ((size_t)b * p.q_cs_sb + (qvalid ? qi : 0)) * (D / 2);
    // pair i: (2i, 2i+1) interleaved, (i, i + D/2) half split
    const bool half = p.rope_style == 1;
    // RMSNorm of q (one lane holds the whole row)
    float qinv = 1.f;
    const float* wq = (const float*)p.q_norm_w;
    if (wq != nullptr && qvalid) {
      float ss = 0.f;
      for (int d = 0; d < D; ++d) ss = fmaf(qrow[d], qrow[d], ss);
      qinv = rsqrtf(ss / (float)D + p.norm_eps);
    }
    for (int i = 0; i < D / 2; ++i) {
      const int d0 = half ? i : 2 * i, d1 = half ? i + D / 2 : 2 * i + 1;
      float2 x = qvalid ? make_float2(qrow[d0], qrow[d1]) : make_float2(0.f, 0.f);
      if (wq != nullptr) x = make_float2(x.x * qinv * wq[d0], x.y * qinv * wq[d1]);
      if (rot && qvalid) {
        const float2 cs = qcs[i];
        const float a = fmaf(x.x, cs.x, -x.y * cs.y);
        const float c = fmaf(x.y, cs.x, x.x * cs.y);
        x = make_float2(a, c);
      }
      Qs[lane][d0] = x.x * p.scale_log2;
      Qs[lane][d1] = x.y * p.scale_log2;
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
  } else if (p.mask_kind == 3) {
    // causal: keys [0, i]; tiles past the tile's last query are skipped
    const int q_last = min(p.Sq, qt * BM + BM) - 1;
    kt_end = (min(p.Sk, q_last + 1) + FWD_BN - 1) / FWD_BN;
    lo = 0;
    hi = qvalid ? min(p.Sk, qi + 1) : 0;
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
        if (p.mask_kind == 2 || p.mask_kind == 3) live = key >= lo && key < hi;
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
  if (p.mask_kind == 2) {
    const int nkb = (p.Sk + 255) / 256;
    seg_prep_kernel<<<dim3(p.n_qt > nkb ? p.n_qt : nkb, p.B), dim3(256), 0, s>>>(p, bm);
  }
  if (p.n_rot > 0) {
    // pairs of the table rows, then of the query rows, then of the key rows
    const int64_t half = p.D / 2;
    const int64_t n = (int64_t)p.rope_tab_len * half + (p.q_rows ? (int64_t)p.q_rows_b * p.Sq * half : 0) +
                      (p.k_rows ? (int64_t)p.k_rows_b * p.Sk * half : 0) +
                      (p.q_cst ? (int64_t)p.q_cst_b * p.Sq * half : 0);
    if (n > 0) rope_prep_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(p);
  }
  if (p.mask_kind == 1) {
    // (no key tiles: nothing to classify; the attention kernel visits none)
    const int64_t ntiles = (int64_t)p.Bm * p.Hm * p.n_qt * p.n_kt;
    if (ntiles > 0) mask_tiles_kernel<<<dim3((unsigned)ntiles), dim3(256), 0, s>>>(p, bm);
  }
  return hipGetLastError();
}

// Rows of at most KR_MAX_TILES key tiles (16-bit types) rotate their K in
// the attention kernel: no K pass, one launch per execute.  Only with the
// default key positions 0 .. Sk-1; explicit or segment-derived ones take
// the K pass (so an explicit position array selects either path for the
// same keys, which the tests compare bit for bit).
constexpr int KR_MAX_TILES = 1;
static bool k_in_attention(const FwdParams& p) {
  if (p.dtype == 0 || p.n_rot_kv == 0 || p.n_kt > KR_MAX_TILES) return false;
  return p.n_rotk == 0 || p.pos_k_mode == POS_ARANGE;
}

// K heads that get RoPE, rotated into the workspace (reads the keys' cos /
// sin rows written by the plan).
hipError_t launch_fwd_rotate(const FwdParams& p, hipStream_t s) {
  if (p.n_rot_kv > 0 && p.Sk > 0 && p.B > 0 && !k_in_attention(p)) {
    if (p.dtype == 0) {
      const int rows_per_blk = 256 / (p.D / 2);
      const unsigned nx = (unsigned)((p.Sk + rows_per_blk - 1) / rows_per_blk);
      k_rotate32_kernel<<<dim3((nx + 7) & ~7u, (unsigned)p.n_rot_kv, (unsigned)p.B), dim3(256), 0, s>>>(p);
    } else {
      const bool half = p.rope_style == 1;
      const unsigned nx = (unsigned)((p.Sk * (p.D / (half ? 16 : 8)) + 255) / 256);
      const dim3 nblk((nx + 7) & ~7u, (unsigned)p.n_rot_kv, (unsigned)p.B);
      if (p.dtype == 2) {
        if (half) k_rotate16_kernel<BF16, true><<<nblk, dim3(256), 0, s>>>(p);
        else k_rotate16_kernel<BF16, false><<<nblk, dim3(256), 0, s>>>(p);
      } else {
        if (half) k_rotate16_kernel<F16, true><<<nblk, dim3(256), 0, s>>>(p);
        else k_rotate16_kernel<F16, false><<<nblk, dim3(256), 0, s>>>(p);
      }
    }
  }
  return hipGetLastError();
}

// Key streams per work-group.  Two when there are no more work-groups than
// CUs and the rows are long: each CU then holds one query tile, the
// one-stream kernel would run a single wave per SIMD, and splitting the keys
// of the tile over two waves per SIMD shortens the chain of steps (measured
// 7-13 % faster for 128 and 256 work-groups at 2048 keys, 32 key tiles).
// With 16 key tiles or fewer per row the second stream's own prologue and
// the final merge cost more than the shorter chain saves (measured slower
// at 16 to 1024 keys), and with more work-groups than CUs the one-stream
// kernel already places two per CU.  A caller's key_streams of 1 or 2
// overrides the choice.
constexpr int KEY_STREAMS_MIN_TILES = 24;
// Compute units of the current device, queried once per device.
static int cu_count() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

static int key_streams(int forced, unsigned nwork, int n_kt) {
  if (forced == 1 || forced == 2) return forced;
  if (n_kt < KEY_STREAMS_MIN_TILES) return 1;
  return (int64_t)nwork <= (int64_t)cu_count() ? 2 : 1;
}

hipError_t launch_fwd_main(const FwdParams& p, hipStream_t s) {
  const bool f32 = p.dtype == 0;
  const unsigned nwork = (unsigned)((int64_t)p.B * p.Hq * p.n_qt);
  if (f32) {
    if (p.D == 64) fwd_f32_kernel<64><<<dim3(nwork), dim3(64), 0, s>>>(p);
    else fwd_f32_kernel<128><<<dim3(nwork), dim3(64), 0, s>>>(p);
  } else {
    const bool kr = k_in_attention(p);
    const int nstr = kr ? 1 : key_streams(p.key_streams, nwork, p.n_kt);
    if (p.dtype == 2) {
      if (p.D == 64) launch_mfma_bf16_d64(p, nwork, nstr, kr, s);
      else launch_mfma_bf16_d128(p, nwork, nstr, kr, s);
    } else {
      if (p.D == 64) launch_mfma_f16_d64(p, nwork, nstr, kr, s);
      else launch_mfma_f16_d128(p, nwork, nstr, kr, s);
    }
  }
  return hipGetLastError();
}

}  // namespace mz
