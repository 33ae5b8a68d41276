// mzattn_decode kernels for gfx950: a few queries against a static KV cache.
//
// VoxCPM page, "What matches upstream" (attention bullet) and "Memory and
// speed" (attention_span): each generation step attends to the cache under
// an explicit boolean mask; masked positions add exact zeros, so a key span
// cut anywhere past the last live key must not change the result.
//
// Split-K over fixed 128-key chunks aligned to key index 0.  Each
// work-group of the chunk kernel reduces one chunk of one (batch, kv-head)
// for all G*q_len query rows of that head group (the rows share every K/V
// byte it loads) and writes a partial (m, l, acc).  The merge kernel then
// folds the partials of every row in an order fixed by chunk index alone.
// A chunk with no live key is skipped by the fold, which is an exact
// identity, and chunk boundaries do not depend on the span, so any span
// past the last live key gives the same bits.
#include "mz_common.h"
#include "mz_internal.h"

namespace mz {

// ---------------------------------------------------------------------------
// Optional: rotate q at q_pos into the workspace (every head).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void decode_q_rotate16_kernel(const DecodeParams p) {
  const int half = p.D / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)p.B * p.Hq * p.T * half;
  if (idx >= n) return;
  const int i = (int)(idx % half);
  const int64_t row = idx / half;
  const int t = (int)(row % p.T);
  const int h = (int)((row / p.T) % p.Hq);
  const int b = (int)(row / ((int64_t)p.T * p.Hq));
  const uint16_t* src = (const uint16_t*)p.q_in + b * p.q_in_s[0] + h * p.q_in_s[1] + (int64_t)t * p.q_in_s[2];
  const float2 cs = rope_cs_direct(p.q_pos[b * p.q_pos_sb + t], i, p.D, p.rs);
  if (p.rope_style == 1) {
    // half split: pair (i, i + D/2)
    const float a = Elem<T>::to_f32(src[i]), c = Elem<T>::to_f32(src[i + half]);
    const uint32_t r = Elem<T>::pack2(fmaf(a, cs.x, -c * cs.y), fmaf(c, cs.x, a * cs.y));
    uint16_t* dst = (uint16_t*)p.q + row * p.D;
    dst[i] = (uint16_t)(r & 0xFFFF);
    dst[i + half] = (uint16_t)(r >> 16);
  } else {
    const uint32_t w = *(const uint32_t*)(src + 2 * i);
    const float a = Elem<T>::to_f32((uint16_t)(w & 0xFFFF));
    const float c = Elem<T>::to_f32((uint16_t)(w >> 16));
    ((uint32_t*)p.q)[row * half + i] = Elem<T>::pack2(fmaf(a, cs.x, -c * cs.y), fmaf(c, cs.x, a * cs.y));
  }
}

__global__ void decode_q_rotate32_kernel(const DecodeParams p) {
  const int half = p.D / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)p.B * p.Hq * p.T * half;
  if (idx >= n) return;
  const int i = (int)(idx % half);
  const int64_t row = idx / half;
  const int t = (int)(row % p.T);
  const int h = (int)((row / p.T) % p.Hq);
  const int b = (int)(row / ((int64_t)p.T * p.Hq));
  const float* src = (const float*)p.q_in + b * p.q_in_s[0] + h * p.q_in_s[1] + (int64_t)t * p.q_in_s[2];
  // pair i: (2i, 2i+1) interleaved, (i, i + D/2) half split
  const int d0 = p.rope_style == 1 ? i : 2 * i, d1 = p.rope_style == 1 ? i + half : 2 * i + 1;
  const float2 x = make_float2(src[d0], src[d1]);
  const float2 cs = rope_cs_direct(p.q_pos[b * p.q_pos_sb + t], i, p.D, p.rs);
  float* dst = (float*)p.q + row * p.D;
  dst[d0] = fmaf(x.x, cs.x, -x.y * cs.y);
  dst[d1] = fmaf(x.y, cs.x, x.x * cs.y);
}

__device__ inline bool dec_live(const DecodeParams& p, int b, int kvh, int n, int key, int span) {
  if (n >= p.R || key >= span) return false;
  if (p.mask == nullptr) return true;
  const int g = n / p.T, t = n % p.T;
  const int h = kvh * p.G + g;
  return p.mask[b * p.ms[0] + h * p.ms[1] + t * p.ms[2] + key] != 0;
}

// ---------------------------------------------------------------------------
// Fold of two partials (m in log2 units, l, acc).  A partial with l == 0 is
// the identity and is skipped, so folding it changes no bit.
// ---------------------------------------------------------------------------
struct Part2 {
  float m, l, a0, a1;
};

__device__ inline void fold_into(Part2& x, float m, float l, float a0, float a1) {
  if (!(l > 0.f)) return;
  if (!(x.l > 0.f)) {
    x.m = m; x.l = l; x.a0 = a0; x.a1 = a1;
    return;
  }
  const float mn = fmaxf(x.m, m);
  const float sa = fast_exp2(x.m - mn), sb = fast_exp2(m - mn);
  x.l = x.l * sa + l * sb;
  x.a0 = x.a0 * sa + a0 * sb;
  x.a1 = x.a1 * sa + a1 * sb;
  x.m = mn;
}

// ---------------------------------------------------------------------------
// Merge kernel: one work-group per (batch, kv-head, row, slice of DS d
// pairs).  Chunks are taken in super-groups of 64; within one, thread group
// g holds chunks [g*CG, (g+1)*CG) of it.  The super-group's maximum m over its live chunks
// (l > 0) is exact; every live chunk then contributes its l and acc scaled
// by 2^(m_c - m), summed in chunk order within a group and in group order
// across groups; super-groups are folded in order.  Chunks at or past
// n_chunks contribute exact zeros and a super-group without live chunks is
// the identity of the fold, so the result does not depend on how many
// chunks the span covered beyond its live keys.
// ---------------------------------------------------------------------------
constexpr int MERGE_DS = 16;  // d pairs per merge work-group

template <int D, typename Store>
__device__ void decode_merge_row(const DecodeParams& p, Store store) {
  constexpr int HD = MERGE_DS;  // d pairs of this work-group
  constexpr int NS = D / 2 / HD;  // slices per row
  constexpr int NG = 256 / HD;  // chunk groups (16)
  constexpr int CG = 64 / NG;   // chunks per group per super-group (4)
  __shared__ float gmax[NG];
  __shared__ Part2 red[256];
  const int row = blockIdx.x / NS, slice = blockIdx.x % NS;  // (unit, n), d slice
  const int n = row % p.R, unit = row / p.R;
  const int kvh = unit % p.Hkv, b = unit / p.Hkv;
  const int t = threadIdx.x, dp = slice * HD + t % HD, g = t / HD;
  const float2* ml = p.part_ml + (int64_t)unit * p.n_chunks * p.R + n;
  const float* pa = p.part_acc + ((int64_t)unit * p.n_chunks * p.R + n) * D + 2 * dp;
  Part2 tot = {0.f, 0.f, 0.f, 0.f};
  for (int sg = 0; sg * 64 < p.n_chunks; ++sg) {
    const int c0 = sg * 64 + g * CG;
    // every load of the group first
    float2 mc[CG], ac[CG];
#pragma unroll
    for (int i = 0; i < CG; ++i) {
      const int c = c0 + i;
      mc[i] = make_float2(0.f, 0.f);
      ac[i] = make_float2(0.f, 0.f);
      if (c < p.n_chunks) {
        mc[i] = ml[(int64_t)c * p.R];
        ac[i] = *(const float2*)(pa + (int64_t)c * p.R * D);
      }
    }
    // exact maximum over the super-group's live chunks
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < CG; ++i) mx = mc[i].y > 0.f ? fmaxf(mx, mc[i].x) : mx;
    if (t % HD == 0) gmax[g] = mx;
    __syncthreads();
    float m = gmax[0];
#pragma unroll
    for (int gg = 1; gg < NG; ++gg) m = fmaxf(m, gmax[gg]);
    Part2 x = {m, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < CG; ++i) {
      const float f = mc[i].y > 0.f ? fast_exp2(mc[i].x - m) : 0.f;
      x.l = fmaf(mc[i].y, f, x.l);
      x.a0 = fmaf(ac[i].x, f, x.a0);
      x.a1 = fmaf(ac[i].y, f, x.a1);
    }
    red[t] = x;
    __syncthreads();
    if (g == 0) {
      Part2 y = red[t];
#pragma unroll
      for (int gg = 1; gg < NG; ++gg) {
        const Part2 z = red[gg * HD + t];
        y.l += z.l;
        y.a0 += z.a0;
        y.a1 += z.a1;
      }
      fold_into(tot, y.m, y.l, y.a0, y.a1);
    }
    __syncthreads();
  }
  if (g == 0) {
    const float inv = tot.l > 0.f ? 1.f / tot.l : 0.f;
    const int gq = n / p.T, tq = n % p.T;
    store(b, kvh * p.G + gq, tq, 2 * dp, tot.a0 * inv, tot.a1 * inv);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge16_kernel(const DecodeParams p) {
  decode_merge_row<D>(p, [&](int b, int h, int t, int d, float x0, float x1) {
    uint16_t* orow = (uint16_t*)p.o + b * p.os[0] + h * p.os[1] + (int64_t)t * p.os[2] + d;
    *(uint32_t*)orow = Elem<T>::pack2(x0, x1);
  });
}

template <int D>
__global__ __launch_bounds__(256) void decode_merge32_kernel(const DecodeParams p) {
  decode_merge_row<D>(p, [&](int b, int h, int t, int d, float x0, float x1) {
    float* orow = (float*)p.o + b * p.os[0] + h * p.os[1] + (int64_t)t * p.os[2] + d;
    *(float2*)orow = make_float2(x0, x1);
  });
}

// ---------------------------------------------------------------------------
// bf16 / fp16 chunk kernel, MFMA 16x16x32.  Wave w owns keys
// [chunk*128 + 32w, +32); rows n = g*q_len + t in NB blocks of 16.
// S^T = K Q^T, then O^T = V^T P^T with V^T read transposed from LDS.
// ---------------------------------------------------------------------------
// Rotate the 8 * NS elements a lane holds of one row (d = s*32 + g4*8 + e)
// with the row's cosines and sines cs[i] (pair i): pairs (2i, 2i+1) inside
// each 8-element piece, or with half-split pairing element d of piece s
// with element d + D/2, which is the same element of piece s + NS/2 in the
// same lane.
template <typename T, int NS>
__device__ inline void rope_lane_row(uint4 (&x)[NS], const float2* cs, int g4, int style) {
  if (style == 1) {
#pragma unroll
    for (int s = 0; s < NS / 2; ++s) {
      uint32_t lo[4] = {x[s].x, x[s].y, x[s].z, x[s].w};
      uint32_t hi[4] = {x[s + NS / 2].x, x[s + NS / 2].y, x[s + NS / 2].z, x[s + NS / 2].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float r[2][2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float a = Elem<T>::to_f32((uint16_t)(lo[t] >> (16 * e)));
          const float c = Elem<T>::to_f32((uint16_t)(hi[t] >> (16 * e)));
          const float2 w = cs[s * 32 + g4 * 8 + 2 * t + e];
          r[0][e] = fmaf(a, w.x, -c * w.y);
          r[1][e] = fmaf(c, w.x, a * w.y);
        }
        lo[t] = Elem<T>::pack2(r[0][0], r[0][1]);
        hi[t] = Elem<T>::pack2(r[1][0], r[1][1]);
      }
      x[s] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      x[s + NS / 2] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    }
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      uint32_t w[4] = {x[s].x, x[s].y, x[s].z, x[s].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float a = Elem<T>::to_f32((uint16_t)(w[t] & 0xFFFF));
        const float c = Elem<T>::to_f32((uint16_t)(w[t] >> 16));
        const float2 r = cs[(s * 32 + g4 * 8) / 2 + t];
        w[t] = Elem<T>::pack2(fmaf(a, r.x, -c * r.y), fmaf(c, r.x, a * r.y));
      }
      x[s] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// APP: the append step (mzattn_decode_append).  The row's filled length
// len[b] is read here; keys from len[b] + q_len on are past the span, the
// new rows [len[b], len[b] + q_len) are loaded from k_new / v_new, rotated
// at their position and written into the caches by the one wave that owns
// them, q is rotated at len[b] + t in registers, and query t sees keys
// j <= len[b] + t only.
template <typename T, int D, int NB, bool APP>
__global__ __launch_bounds__(256) void decode_mfma_kernel(const DecodeParams p) {
  constexpr int AS = D + 4;        // LDS row stride of the parked acc blocks (floats)
  constexpr int NS = D / 32;       // k-steps of K Q^T
  constexpr int NDB = D / 16;      // 16-row d blocks of O^T
  constexpr int VSD = D + 16;      // LDS row stride of V (elements)
  constexpr int CH = D / 8;        // 16-byte chunks per row
  constexpr int RPI = 64 / CH;     // V rows per wave load instruction
  constexpr int NVL = 32 / RPI;    // V loads per lane
  constexpr int RP = NB * 16;      // padded rows
  __shared__ __attribute__((aligned(16))) uint16_t Vs[4][32 * VSD];
  __shared__ float red_m[4][RP];
  __shared__ float red_l[4][RP];
  __shared__ uint8_t live_s[RP][DEC_CHUNK];
  // (append) cosines and sines of the new tokens' positions len + t
  __shared__ float2 cs_s[APP ? 16 : 1][APP ? D / 2 : 1];
  static_assert(sizeof(float) * RP * AS <= sizeof(uint16_t) * 4 * 32 * VSD, "acc fold reuses the V region");
  float* acc_lds = reinterpret_cast<float*>(&Vs[0][0]);

  const int w = blockIdx.x;
  const int c = w % p.n_chunks;
  const int unit = w / p.n_chunks;
  const int kvh = unit % p.Hkv, b = unit / p.Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int key0 = c * DEC_CHUNK + wave * 32;

  const uint16_t* kbase = (const uint16_t*)p.k + b * p.ks[0] + kvh * p.ks[1];
  const uint16_t* vbase = (const uint16_t*)p.v + b * p.vs[0] + kvh * p.vs[1];

  // keys [0, span_b) of this row are considered
  int lenb = 0, span_b = p.span;
  if constexpr (APP) {
    lenb = p.len[(int64_t)b * p.len_sb];
    const bool fits = lenb >= 0 && (int64_t)lenb + p.T <= (int64_t)p.C;
    span_b = fits ? lenb + p.T : 0;
    if (!fits && c == 0 && kvh == 0 && tid == 0 && p.overflow != nullptr) *p.overflow = 1;
  }
  // (append) this chunk holds some of the new rows: never skipped, so they
  // are written into the caches whatever the mask says
  const bool holds_new = APP && c * DEC_CHUNK < span_b && (c + 1) * DEC_CHUNK > lenb;

  // ---- a chunk in which no (row, key) pair is live is the identity of the
  // merge: found from the mask alone, its K/V are never read.  The scan
  // keeps the chunk's liveness bytes in LDS (one row when the mask is
  // broadcast over heads and queries) for the score test below, so no mask
  // load sits among the K/V loads.
  const bool bcast = p.mask != nullptr && p.ms[1] == 0 && p.ms[2] == 0;
  // (a chunk at or past the span, e.g. the one chunk of an empty span, has
  // no key index valid to load)
  bool dead = span_b <= c * DEC_CHUNK;
  if (p.mask != nullptr && !dead) {
    const int ckey0 = c * DEC_CHUNK;
    const int rows = bcast ? 1 : p.R;
    bool any = false;
    for (int idx = tid; idx < rows * DEC_CHUNK; idx += 256) {
      const bool lv = dec_live(p, b, kvh, idx / DEC_CHUNK, ckey0 + idx % DEC_CHUNK, span_b);
      live_s[idx / DEC_CHUNK][idx % DEC_CHUNK] = lv;
      any |= lv;
    }
    dead = !__syncthreads_or(any) && !holds_new;
  }
  if (dead) {
    const int64_t pb = ((int64_t)unit * p.n_chunks + c) * p.R;
    for (int idx = tid; idx < p.R * (D / 4); idx += 256)
      *(float4*)(p.part_acc + (pb + idx / (D / 4)) * D + (idx % (D / 4)) * 4) = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int n = tid; n < p.R; n += 256) p.part_ml[pb + n] = make_float2(0.f, 0.f);
    return;
  }

  // ---- issue every global load of this wave up front, unconditionally:
  // keys past the span read row span - 1 and rows past R read row R - 1
  // (in bounds; their scores are masked to -inf below, so their weights
  // are exact zeros).  Conditional loads would each end in a wait, making
  // the loads one dependent round trip after another.
  const int klast = span_b - 1;
  const uint16_t* knew = nullptr;
  const uint16_t* vnew = nullptr;
  if constexpr (APP) {
    knew = (const uint16_t*)p.k_new + b * p.kn_s[0] + kvh * p.kn_s[1];
    vnew = (const uint16_t*)p.v_new + b * p.vn_s[0] + kvh * p.vn_s[1];
  }
  uint4 qf[NB][NS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = min(nb * 16 + l16, p.R - 1);
    const int g = n / p.T, t = n % p.T;
    const int h = kvh * p.G + g;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qf[nb][s] = *(const uint4*)((const uint16_t*)p.q + b * p.qs[0] + h * p.qs[1] + (int64_t)t * p.qs[2] + s * 32 +
                                  g4 * 8);
  }
  u32x4_t vr[NVL];  // a native vector type: one load each, kept in registers
#pragma unroll
  for (int it = 0; it < NVL; ++it) {
    const int r = it * RPI + lane / CH, cc = lane % CH;
    const int key = min(key0 + r, klast);
    const uint16_t* row = (APP && key >= lenb) ? vnew + (int64_t)(key - lenb) * p.vn_s[2] : vbase + (int64_t)key * p.vs[2];
    vr[it] = *(const u32x4_t*)(row + cc * 8);
  }
  uint4 kf[2][NS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = min(key0 + kb * 16 + l16, klast);
    const uint16_t* row = (APP && key >= lenb) ? knew + (int64_t)(key - lenb) * p.kn_s[2] : kbase + (int64_t)key * p.ks[2];
#pragma unroll
    for (int s = 0; s < NS; ++s) kf[kb][s] = *(const uint4*)(row + s * 32 + g4 * 8);
  }
  // every load above is issued before the first use of any of them (the
  // scheduler would otherwise start the V loads after the K.Q MFMAs)
  asm volatile("" ::: "memory");
  if constexpr (APP) {
    // q at len + t (its loads came first: this overlaps the K/V loads)
    if (p.rope) {
      for (int idx = tid; idx < p.T * (D / 2); idx += 256)
        cs_s[idx / (D / 2)][idx % (D / 2)] = rope_cs_direct(lenb + idx / (D / 2), idx % (D / 2), D, p.rs);
      __syncthreads();
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int n = min(nb * 16 + l16, p.R - 1);
        rope_lane_row<T, NS>(qf[nb], cs_s[n % p.T], g4, p.rope_style);
      }
    }
    // the new rows this wave holds: K rotated at its position, then both
    // written into the caches (every lane of the row writes its pieces)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = key0 + kb * 16 + l16;
      if (key >= lenb && key < span_b) {
        if (p.rope) rope_lane_row<T, NS>(kf[kb], cs_s[key - lenb], g4, p.rope_style);
        uint16_t* dst = (uint16_t*)p.k_w + b * p.ks[0] + kvh * p.ks[1] + (int64_t)key * p.ks[2];
#pragma unroll
        for (int s = 0; s < NS; ++s) *(uint4*)(dst + s * 32 + g4 * 8) = kf[kb][s];
      }
    }
#pragma unroll
    for (int it = 0; it < NVL; ++it) {
      const int r = it * RPI + lane / CH, cc = lane % CH;
      const int key = key0 + r;
      if (key >= lenb && key < span_b) {
        uint16_t* dst = (uint16_t*)p.v_w + b * p.vs[0] + kvh * p.vs[1] + (int64_t)key * p.vs[2];
        *(u32x4_t*)(dst + cc * 8) = vr[it];
      }
    }
  }
  // liveness of this lane's score elements (mask bytes from the scan)
  bool live[2][NB][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int n = nb * 16 + l16, j = wave * 32 + kb * 16 + g4 * 4 + v;
        const int key = c * DEC_CHUNK + j;
        const bool in = n < p.R && key < span_b && (!APP || key <= lenb + n % p.T);
        live[kb][nb][v] = in && (p.mask == nullptr || live_s[bcast ? 0 : n][j] != 0);
      }
  // V rows into this wave's LDS region
#pragma unroll
  for (int it = 0; it < NVL; ++it) {
    const int r = it * RPI + lane / CH, cc = lane % CH;
    *(u32x4_t*)&Vs[wave][r * VSD + cc * 8] = vr[it];
  }

  // ---- scores S^T (keys x rows), masked, in the log2 domain
  f32x4_t sacc[2][NB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) a = mfma16<T>(kf[kb][s], qf[nb][s], a);
      sacc[kb][nb] = a;
    }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + l16;
    float m = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float x = live[kb][nb][v] ? sacc[kb][nb][v] * p.scale_log2 : -INFINITY;
        sacc[kb][nb][v] = x;
        m = fmaxf(m, x);
      }
    m = wave_xor_max(m, 16);
    m = wave_xor_max(m, 32);
    if (g4 == 0) red_m[wave][n] = m;
  }
  __syncthreads();
  // chunk max over the 4 waves (fixed order), exponentials, partial sums
  uint4 pb[NB];
  float m_use[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + l16;
    const float m = fmaxf(fmaxf(red_m[0][n], red_m[1][n]), fmaxf(red_m[2][n], red_m[3][n]));
    m_use[nb] = m == -INFINITY ? 0.f : m;
    float ls = 0.f;
    uint32_t wv[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float p0 = fast_exp2(sacc[kb][nb][0] - m_use[nb]);
      const float p1 = fast_exp2(sacc[kb][nb][1] - m_use[nb]);
      const float p2 = fast_exp2(sacc[kb][nb][2] - m_use[nb]);
      const float p3 = fast_exp2(sacc[kb][nb][3] - m_use[nb]);
      ls += (p0 + p1) + (p2 + p3);
      wv[kb * 2 + 0] = Elem<T>::pack2(p0, p1);
      wv[kb * 2 + 1] = Elem<T>::pack2(p2, p3);
    }
    pb[nb] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    if (g4 == 0) red_l[wave][n] = ls;
  }

  // ---- O^T = V^T P^T over this wave's 32 keys
  f32x4_t oacc[NB][NDB];
  const int rr = l16 >> 2, cq = l16 & 3;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int col = db * 16 + 4 * cq;
    const uint2 a0 = lds_read_tr<T>(&Vs[wave][(g4 * 4 + rr) * VSD + col]);
    const uint2 a1 = lds_read_tr<T>(&Vs[wave][(16 + g4 * 4 + rr) * VSD + col]);
    const uint4 a = make_uint4(a0.x, a0.y, a1.x, a1.y);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      oacc[nb][db] = mfma16<T>(a, pb[nb], z);
    }
  }
  // fold the 4 waves in fixed order through LDS (reusing the V region once
  // every wave has finished reading it) and write the chunk partial
  __syncthreads();
  const int64_t pbase = ((int64_t)unit * p.n_chunks + c) * p.R;
  // (rows AS = D + 4 floats apart: the 16 rows one 16-byte store
  // instruction touches then fall on distinct banks)
  if constexpr (sizeof(float) * 4 * RP * AS <= sizeof(uint16_t) * 4 * 32 * VSD) {
    // every wave parks its block in its own region; then all threads add
    // the four in wave order
    float* const own = acc_lds + wave * (RP * AS);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *(f32x4_t*)&own[(nb * 16 + l16) * AS + db * 16 + g4 * 4] = oacc[nb][db];
    __syncthreads();
    for (int idx = tid; idx < p.R * (D / 4); idx += 256) {
      const int n = idx / (D / 4), d = (idx % (D / 4)) * 4;
      float4 x = *(const float4*)&acc_lds[n * AS + d];
#pragma unroll
      for (int wv = 1; wv < 4; ++wv) {
        const float4 y = *(const float4*)&acc_lds[wv * (RP * AS) + n * AS + d];
        x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
      }
      *(float4*)(p.part_acc + (pbase + n) * D + d) = x;
    }
  } else {
    // larger row counts: one shared block, waves adding in turn
    for (int step = 0; step < 4; ++step) {
      if (wave == step) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              float* slot = &acc_lds[(nb * 16 + l16) * AS + db * 16 + g4 * 4 + v];
              *slot = step == 0 ? oacc[nb][db][v] : *slot + oacc[nb][db][v];
            }
      }
      __syncthreads();
    }
    for (int idx = tid; idx < p.R * (D / 4); idx += 256) {
      const int n = idx / (D / 4), d = (idx % (D / 4)) * 4;
      *(float4*)(p.part_acc + (pbase + n) * D + d) = *(const float4*)&acc_lds[n * AS + d];
    }
  }
  for (int n = tid; n < p.R; n += 256) {
    const float m = fmaxf(fmaxf(red_m[0][n], red_m[1][n]), fmaxf(red_m[2][n], red_m[3][n]));
    const float l = (red_l[0][n] + red_l[1][n]) + (red_l[2][n] + red_l[3][n]);
    p.part_ml[pbase + n] = make_float2(m == -INFINITY ? 0.f : m, l);
  }
}

// ---------------------------------------------------------------------------
// fp32 chunk kernel: plain FMA, same partial format and fold.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void decode_f32_kernel(const DecodeParams p) {
  __shared__ float S[64][DEC_CHUNK];
  __shared__ float s_m[64], s_l[64];
  const int w = blockIdx.x;
  const int c = w % p.n_chunks;
  const int unit = w / p.n_chunks;
  const int kvh = unit % p.Hkv, b = unit / p.Hkv;
  const int tid = threadIdx.x;
  const int D = p.D;
  const float* kbase = (const float*)p.k + b * p.ks[0] + kvh * p.ks[1];
  const float* vbase = (const float*)p.v + b * p.vs[0] + kvh * p.vs[1];
  const int key0 = c * DEC_CHUNK;

  for (int idx = tid; idx < p.R * DEC_CHUNK; idx += 256) {
    const int n = idx / DEC_CHUNK, j = idx % DEC_CHUNK;
    const int key = key0 + j;
    float x = -INFINITY;
    if (dec_live(p, b, kvh, n, key, p.span)) {
      const int g = n / p.T, t = n % p.T;
      const int h = kvh * p.G + g;
      const float* qrow = (const float*)p.q + b * p.qs[0] + h * p.qs[1] + (int64_t)t * p.qs[2];
      const float* krow = kbase + (int64_t)key * p.ks[2];
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(qrow[d], krow[d], acc);
      x = acc * p.scale_log2;
    }
    S[n][j] = x;
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  for (int n = wave; n < p.R; n += 4) {
    float m = fmaxf(S[n][lane], S[n][lane + 64]);
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    const float mu = m == -INFINITY ? 0.f : m;
    const float p0 = exp2f(S[n][lane] - mu), p1 = exp2f(S[n][lane + 64] - mu);
    S[n][lane] = p0;
    S[n][lane + 64] = p1;
    float l = p0 + p1;
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off, 64);
    if (lane == 0) {
      s_m[n] = mu;
      s_l[n] = l;
    }
  }
  __syncthreads();
  const int64_t pbase = ((int64_t)unit * p.n_chunks + c) * p.R;
  for (int idx = tid; idx < p.R * D; idx += 256) {
    const int n = idx / D, d = idx % D;
    float acc = 0.f;
    for (int j = 0; j < DEC_CHUNK; ++j) {
      const int key = key0 + j;
      if (key >= p.span) break;
      acc = fmaf(S[n][j], vbase[(int64_t)key * p.vs[2] + d], acc);
    }
    p.part_acc[(pbase + n) * D + d] = acc;
  }
  for (int n = tid; n < p.R; n += 256) p.part_ml[pbase + n] = make_float2(s_m[n], s_l[n]);
}

// ---------------------------------------------------------------------------
template <typename T, int D, bool APP>
static void launch_dec16_k(const DecodeParams& p, unsigned nblk, hipStream_t s) {
  if (p.R <= 16) decode_mfma_kernel<T, D, 1, APP><<<dim3(nblk), dim3(256), 0, s>>>(p);
  else if (p.R <= 32) decode_mfma_kernel<T, D, 2, APP><<<dim3(nblk), dim3(256), 0, s>>>(p);
  else decode_mfma_kernel<T, D, 4, APP><<<dim3(nblk), dim3(256), 0, s>>>(p);
}
template <typename T, int D>
static void launch_dec16(const DecodeParams& p, unsigned nblk, hipStream_t s) {
  if (p.app) launch_dec16_k<T, D, true>(p, nblk, s);
  else launch_dec16_k<T, D, false>(p, nblk, s);
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  if (p.rope && !p.app) {  // (the append step rotates q in the chunk kernel)
    const int64_t n = (int64_t)p.B * p.Hq * p.T * (p.D / 2);
    const unsigned nb = (unsigned)((n + 255) / 256);
    if (p.dtype == 0) decode_q_rotate32_kernel<<<dim3(nb), dim3(256), 0, s>>>(p);
    else if (p.dtype == 2) decode_q_rotate16_kernel<BF16><<<dim3(nb), dim3(256), 0, s>>>(p);
    else decode_q_rotate16_kernel<F16><<<dim3(nb), dim3(256), 0, s>>>(p);
  }
  const unsigned nblk = (unsigned)((int64_t)p.B * p.Hkv * p.n_chunks);
  const unsigned nrows = (unsigned)((int64_t)p.B * p.Hkv * p.R * (p.D / 2 / MERGE_DS));
  if (p.dtype == 0) {
    decode_f32_kernel<<<dim3(nblk), dim3(256), 0, s>>>(p);
    if (p.D == 64) decode_merge32_kernel<64><<<dim3(nrows), dim3(256), 0, s>>>(p);
    else decode_merge32_kernel<128><<<dim3(nrows), dim3(256), 0, s>>>(p);
  } else if (p.dtype == 2) {
    if (p.D == 64) {
      launch_dec16<BF16, 64>(p, nblk, s);
      decode_merge16_kernel<BF16, 64><<<dim3(nrows), dim3(256), 0, s>>>(p);
    } else {
      launch_dec16<BF16, 128>(p, nblk, s);
      decode_merge16_kernel<BF16, 128><<<dim3(nrows), dim3(256), 0, s>>>(p);
    }
  } else {
    if (p.D == 64) {
      launch_dec16<F16, 64>(p, nblk, s);
      decode_merge16_kernel<F16, 64><<<dim3(nrows), dim3(256), 0, s>>>(p);
    } else {
      launch_dec16<F16, 128>(p, nblk, s);
      decode_merge16_kernel<F16, 128><<<dim3(nrows), dim3(256), 0, s>>>(p);
    }
  }
  return hipGetLastError();
}

}  // namespace mz
