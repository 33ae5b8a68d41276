// The bf16 / fp16 attention kernel of mzattn_fwd (gfx950), as a template:
// each fwd_mfma_*.hip file instantiates one element type and head_dim, so
// they compile in parallel.  What it computes: see fwd.hip.
#pragma once

#include <type_traits>

#include "mz_common.h"
#include "mz_internal.h"

namespace mz {

// ---------------------------------------------------------------------------
// Main kernel, bf16 / fp16, MFMA 32x32x16.
//
// One work-group = (b, h, 128 queries); 4 waves of 32 queries each.  Scores
// are computed transposed, S^T = K Q^T, so that every lane owns one query:
// the row max and row sum need one cross-lane exchange (lanes l, l^32) and
// the output O^T = V^T P^T is rescaled lane-locally.  P^T leaves the
// accumulator registers directly as the B operand of the P.V MFMA; V^T comes
// from LDS through the transposing read.
//
// Q is pre-multiplied by scale * log2(e) before rounding to the MFMA type,
// so scores arrive in the log2 domain.  The running max is raised only when
// a new score exceeds it by more than 2^8 (otherwise exponentials stay below
// 256 and nothing is rescaled); numerator and denominator always share the
// same reference, so the result is the same softmax.
//
// ---------------------------------------------------------------------------
constexpr float LAZY_RESCALE_LOG2 = 8.0f;

// LDS layout of the 64-row K and V tiles (64 four-byte banks, 256 bytes a
// cycle).  Each copy instruction (1 KB) reads whole rows from global
// memory, so it touches as few cache lines as the rows allow.
//  K: rows KS = D + 8 elements apart (one 16-byte pad chunk, filled with a
//     copy of chunk 0).  An operand fetch reads one chunk of 16
//     consecutive rows per 16 lanes, and those start 4 banks apart.
//  V: no padding.  Groups of 4 rows (one copy instruction at D 128, half of
//     one at D 64); inside a group, quads of 4 chunks, then the row, then
//     the chunk.  A transposing read takes 4 rows x 4 chunks per 32 lanes
//     (two lanes per chunk): 256 contiguous bytes.  v_at is the element
//     offset of chunk c (elements 8c .. 8c + 7) of row r; copy slot s (the
//     s-th 16 bytes of the tile) holds chunk v_chunk(s) of row v_row(s).
template <int D> struct Lay {
  static constexpr int CH = D / 8;  // chunks per row
  static constexpr int KS = D + 8;
  static_assert(CH % 4 == 0, "whole chunk quads per row");
  __device__ static constexpr int v_at(int r, int c) {
    return (r >> 2) * (4 * D) + (c >> 2) * 128 + (r & 3) * 32 + (c & 3) * 8;
  }
  __device__ static constexpr int v_row(int s) { return (s / (4 * CH)) * 4 + ((s >> 2) & 3); }
  __device__ static constexpr int v_chunk(int s) { return ((s % (4 * CH)) >> 4) * 4 + (s & 3); }
};

// Tile class bytes kept in LDS (boolean-mask mode) when the key axis has at
// most this many tiles; longer rows read them from global memory.
constexpr int CLS_LDS = 4096;

// Causal kind: which query tile the slot-th work item of a (batch,
// kv-head) unit takes.  Query tile t has ~2t + 2 key tiles, so a plain
// order hands each XCD (a contiguous range of slots) only long or only
// short tiles.  When each XCD holds C (even) whole slots of one unit, the
// XCD's C slots take C/2 tiles from the long end, longest first, then C/2
// from the short end, shortest first: every XCD gets the same work, and the
// two work-groups the dispatcher places on one CU (its i-th and (C/2 + i)-
// th slots' heads) pair a long tile with a short one.  Otherwise the tiles
// go longest first.
__device__ inline int causal_query_tile(int slot, int n_qt, int nwork, int G) {
  const int per_xcd = (nwork & 7) == 0 ? nwork >> 3 : 0;
  const int C = per_xcd % G == 0 ? per_xcd / G : 0;
  if (C >= 2 && (C & 1) == 0 && n_qt % C == 0) {
    const int c = slot / C, r = slot % C, h = C / 2;
    return r < h ? n_qt - 1 - (c * h + r) : c * h + (r - h);
  }
  return n_qt - 1 - slot;
}

// NSTR key streams per work-group.  With NSTR 2 the work-group has 8 waves:
// waves w and w + 4 own the same 32 queries and take alternate live key
// tiles (each stream with its own copies and LDS stages), and the two
// partial results are combined through LDS at the end.  A query tile's
// chain of dependent steps is then half as long, at the same number of
// waves per CU, which evens out work-groups whose key ranges differ.
// KR (rows of one key tile): 0 = K tiles come pre-rotated from the K pass
// (or from k); 1 / 2 = this kernel loads the K tile through registers and
// normalises and rotates it there (1 interleaved pairs, 2 half split), heads
// without RoPE or norm passing unchanged: a short row is then one launch.
template <typename T, int D, int MK, int NSTR, int KR = 0>
__global__ __launch_bounds__(256 * NSTR, 3 - NSTR) void fwd_mfma_kernel(const FwdParams p) {
  static_assert(NSTR == 1 || NSTR == 2, "one or two key streams");
  static_assert(KR == 0 || NSTR == 1, "in-kernel K rotation: one key stream");
  constexpr int NT = 256 * NSTR;
  constexpr int BM = FWD_BM, BN = FWD_BN;
  constexpr int NS = D / 16;  // k-steps of K Q^T
  constexpr int ND = D / 32;  // 32-row d blocks of O^T
  constexpr int CH = D / 8;   // 16-byte chunks of data per row
  using L = Lay<D>;
  constexpr int KS = L::KS, KCH = KS / 8;  // K: 16-byte slots per padded row
  // one direct-to-LDS wave instruction fills 64 consecutive copy slots
  // (1 KB); a K tile takes KCH of them, a V tile CH
  constexpr int KINS = KCH, VINS = CH;
  constexpr int KPW = (KINS + 3) / 4, VPW = VINS / 4;  // per wave, at most
  static_assert(VINS % 4 == 0, "every wave issues the same V copies");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NSTR][2][BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[NSTR][2][BN * D];
  __shared__ uint8_t cls_lds[MK == 1 ? CLS_LDS : 1];
  __shared__ int n_live_lds;

  // work order: (kv-head, b, query tile, head within the group).  The G
  // heads that share K/V run side by side and long tiles start first; the
  // contiguous range each XCD receives covers whole kv-heads, so their K/V
  // stay in that XCD's L2, and batches mix within every XCD.
  const int nwork = p.B * p.Hq * p.n_qt;
  const int w = xcd_remap(blockIdx.x, nwork);
  const int g = w % p.G;
  const int qt = MK == 3 ? causal_query_tile((w / p.G) % p.n_qt, p.n_qt, nwork, p.G) : (w / p.G) % p.n_qt;
  const int kvb = w / (p.G * p.n_qt);
  const int b = kvb % p.B, hk = kvb / p.B;
  const int h = hk * p.G + g;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (tid >> 6) & 3;  // query strip
  const int str = NSTR == 1 ? 0 : tid >> 8;  // key stream
  const int l32 = lane & 31, hh = lane >> 5;
  const int qi = qt * BM + wave * 32 + l32;
  const bool qvalid = qi < p.Sq;

  // ---- Q fragment, pre-scaled: B operand of S^T = K Q^T.  Its loads (q,
  // the norm weights, the query's cos / sin row) are issued here; the
  // arithmetic (finish_q) runs once the first K / V tile copies are
  // issued, so the two latencies overlap.
  // No load here sits inside a per-lane branch (a lane past Sq reads row
  // Sq - 1, and its result is never stored): such a load ends in a wait for
  // everything issued before it, which would make the prologue a chain of
  // round trips.  Loads nobody needs (absent norm weights, waves with no
  // query) are skipped by wave-uniform branches only.
  uint4 qf[NS];
  const int qi_c = qvalid ? qi : p.Sq - 1;
  const uint16_t* qrow = (const uint16_t*)p.q + b * p.qs[0] + h * p.qs[1] + (int64_t)qi_c * p.qs[2];
  const bool rot = h < p.n_rot;  // uniform over the work-group
  // A wave whose 32 queries all lie past Sq (short rows: 112 of the 128
  // queries of a 16-token tile) issues none of the loads below.  The test
  // is wave-uniform (a scalar branch, no per-lane masking), and the vector
  // memory instructions it saves are what a short row's prologue is bound
  // by: every wave-wide load costs the compute unit's load path the same
  // whatever its lanes' addresses.
  const bool wave_live = qt * BM + __builtin_amdgcn_readfirstlane(wave) * 32 < p.Sq;
  const float qsc = p.scale_log2;
  // (the one-tile kernels load the q row on every wave: a skipped load's
  // registers merge with the loaded ones, and that merge waits for the
  // loads before the cos / sin and K loads can issue, a round trip these
  // one-step launches cannot hide; measured 0.4 us per 16-token launch.
  // The multi-tile kernels keep the skip: there it measured ~1 % faster.)
  if (KR != 0 || wave_live) {
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *(const uint4*)(qrow + s * 16 + hh * 8);
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = make_uint4(0u, 0u, 0u, 0u);
  }
  // RMSNorm of q: this lane holds half of the row (elements s*16 + hh*8
  // + e), lane ^ 32 the other half
  const bool qnorm = p.q_norm_w != nullptr;
  uint4 wq[NS];
  if (qnorm && wave_live) {
#pragma unroll
    for (int s = 0; s < NS; ++s) wq[s] = *(const uint4*)((const uint16_t*)p.q_norm_w + s * 16 + hh * 8);
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) wq[s] = make_uint4(0u, 0u, 0u, 0u);
  }
  // cos / sin of this lane's pairs, from the query's cos / sin row (the
  // plan's: no position is read here, so these loads wait for nothing),
  // read as 16-byte vectors, all issued before any is used: interleaved,
  // piece s holds pairs s*8 + hh*4 + t (t < 4), slot 4s + t; half split,
  // piece s < NS/2 holds pairs s*16 + hh*8 + j (j < 8), slot 8s + j; slot
  // m is half of tb[m / 2].
  float4 tb[2 * NS];
  if (rot && wave_live) {
    // the style only picks each slot's offset (a uniform select between two
    // constants), so either pairing costs the same 2 * NS 16-byte loads
    // slot m is chunk (hs ? oh : oi) + hh * (hs ? 4 : 2) of the query's
    // row (float4 chunk c = pairs 2c, 2c + 1), read from the plan's
    // chunk-major copy: the 32 queries of a wave are contiguous per load
    const bool hs = p.rope_style == 1;
    const float4* tl = p.q_cst + b * p.q_cst_sb + (int64_t)(hh * (hs ? 4 : 2)) * p.Sq + qi_c;
    static_for<2 * NS>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int oi = (m >> 1) * 4 + (m & 1), oh = (m >> 2) * 8 + (m & 3);
      tb[m] = tl[(int64_t)(hs ? oh : oi) * p.Sq];
    });
  }
  auto finish_q = [&]() {
    float qinv = 1.f;
    if (qnorm) {
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint32_t wv[4] = {qf[s].x, qf[s].y, qf[s].z, qf[s].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float a = Elem<T>::to_f32((uint16_t)(wv[t] & 0xFFFF)), c = Elem<T>::to_f32((uint16_t)(wv[t] >> 16));
          ss = fmaf(a, a, fmaf(c, c, ss));
        }
      }
      qinv = rsqrtf(half_swap_sum(ss) / (float)D + p.norm_eps);
    }
    // element e (0..7) of piece s, normalised when q_norm_w is set
    auto qn = [&](float x, int s, int e) __attribute__((always_inline)) -> float {
      if (!qnorm) return x;
      const uint32_t w2 = e < 4 ? (e < 2 ? wq[s].x : wq[s].y) : (e < 6 ? wq[s].z : wq[s].w);
      return x * qinv * Elem<T>::to_f32((uint16_t)(w2 >> (16 * (e & 1))));
    };
    // cos / sin of slot m
    auto cs_at = [&](int m) -> float2 {
      const float4 v = tb[m >> 1];
      return (m & 1) ? make_float2(v.z, v.w) : make_float2(v.x, v.y);
    };
    // half split: element e of chunk s pairs with element e of chunk
    // s + NS/2 (d and d + D/2), both held by this lane
    auto half_split = [&]() {
#pragma unroll
      for (int s = 0; s < NS / 2; ++s) {
        uint32_t lo[4] = {qf[s].x, qf[s].y, qf[s].z, qf[s].w};
        uint32_t hi[4] = {qf[s + NS / 2].x, qf[s + NS / 2].y, qf[s + NS / 2].z, qf[s + NS / 2].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float r[2][2];  // [first half, second half][element 2t, 2t + 1]
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float a = qn(Elem<T>::to_f32((uint16_t)(lo[t] >> (16 * e))), s, 2 * t + e);
            const float c = qn(Elem<T>::to_f32((uint16_t)(hi[t] >> (16 * e))), s + NS / 2, 2 * t + e);
            const float2 cs = cs_at(8 * s + 2 * t + e);
            r[0][e] = fmaf(a, cs.x, -c * cs.y);
            r[1][e] = fmaf(c, cs.x, a * cs.y);
          }
          lo[t] = Elem<T>::pack2(r[0][0] * qsc, r[0][1] * qsc);
          hi[t] = Elem<T>::pack2(r[1][0] * qsc, r[1][1] * qsc);
        }
        qf[s] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        qf[s + NS / 2] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      }
    };
    // interleaved: the pairs are the two halves of each 32-bit word
    auto interleaved = [&](auto rotate) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        uint32_t wv[4] = {qf[s].x, qf[s].y, qf[s].z, qf[s].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float a = qn(Elem<T>::to_f32((uint16_t)(wv[t] & 0xFFFF)), s, 2 * t);
          float c = qn(Elem<T>::to_f32((uint16_t)(wv[t] >> 16)), s, 2 * t + 1);
          if constexpr (decltype(rotate)::value) {
            const float2 cs = cs_at(4 * s + t);
            const float ra = fmaf(a, cs.x, -c * cs.y);
            const float rc = fmaf(c, cs.x, a * cs.y);
            a = ra;
            c = rc;
          }
          wv[t] = Elem<T>::pack2(a * qsc, c * qsc);
        }
        qf[s] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
    };
    // Every lane of a live wave runs the same code (a lane past Sq holds a
    // copy of row Sq - 1 and its result is never stored), so each branch
    // here is uniform over the wave: no per-lane masking around the
    // arithmetic.
    if (!wave_live) return;
    if (rot && p.rope_style == 1) half_split();
    else if (rot) interleaved(std::true_type{});
    else interleaved(std::false_type{});
  };

  // ---- K / V sources (KR: every head is read from k, through registers)
  const uint16_t* kbase;
  int64_t kstride;
  if (KR == 0 && hk < p.n_rot_kv) {
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
  const uint64_t* brow = nullptr;  // this lane's key-bit words (valid queries)
  bool cls_in_lds = false;
  if constexpr (MK == 2) {
    const int4 r = p.qt_range[(int64_t)b * p.n_qt + qt];
    kt_beg = r.x; kt_end = r.y; full_beg = r.z; full_end = r.w;
    if (qvalid) {
      const int2 qr = p.q_range[(int64_t)b * p.Sq + qi];
      lo = qr.x; hi = qr.y;
    } else {
      lo = 0; hi = 0;
    }
  } else if constexpr (MK == 3) {
    // causal: keys [0, i] of query i; whole tiles below the tile's first
    // query need no per-element test
    const int q_first = qt * BM, q_last = min(p.Sq, q_first + BM) - 1;
    kt_end = (min(p.Sk, q_last + 1) + BN - 1) / BN;
    full_end = min(p.Sk, q_first + 1) / BN;
    lo = 0;
    hi = qvalid ? min(p.Sk, qi + 1) : 0;
  } else if constexpr (MK == 1) {
    const int bm_ = p.Bm == 1 ? 0 : b, hm_ = p.Hm == 1 ? 0 : h;
    cls_row = p.tile_cls + ((int64_t)(bm_ * p.Hm + hm_) * p.n_qt + qt) * p.n_kt;
    if (qvalid)
      brow = p.mask_bits + ((int64_t)(bm_ * p.Hm + hm_) * p.mask_rows + (p.ms[2] == 0 ? 0 : qi)) * p.n_kt;
    cls_in_lds = p.n_kt <= CLS_LDS;
    if (cls_in_lds) {
      for (int i = tid; i < p.n_kt; i += NT) cls_lds[i] = cls_row[i];
      if (NSTR == 2 && tid == 0) n_live_lds = 0;
      __syncthreads();
    } else if (NSTR == 2) {
      if (tid == 0) n_live_lds = 0;
      __syncthreads();
    }
  }
  auto cls_at = [&](int kt) -> int {
    if constexpr (MK == 1) return cls_in_lds ? cls_lds[kt] : cls_row[kt];
    return 1;
  };
  // rows of at most 64 key tiles: the live and the mixed tiles as two
  // wave-uniform bit sets (one class byte per lane, gathered by ballot), so
  // finding the next live tile and the boundary test are scalar bit
  // operations with no LDS read in the step
  const bool cls_bits = MK == 1 && p.n_kt <= 64;
  uint64_t live_bits = 0, mixed_bits = 0;
  if constexpr (MK == 1) {
    if (cls_bits) {
      const int c = lane < p.n_kt ? (int)cls_row[lane] : 0;
      live_bits = __ballot(c != 0);
      mixed_bits = __ballot(c == 2);
    }
  }
  auto next_live = [&](int kt) {
    if constexpr (MK == 1) {
      if (cls_bits) {
        const uint64_t r = kt < 64 ? live_bits >> kt : 0;
        return r != 0 ? kt + (int)__builtin_ctzll(r) : kt_end;
      }
      while (kt < kt_end && cls_at(kt) == 0) ++kt;
    }
    return kt;
  };
  const int first_tail_tile = p.Sk / BN;  // tiles from here on reach past Sk
  // live key tiles of the query tile; with two streams their count fixes how
  // many barriers each stream passes (the read is after the prologue barrier)
  int n_live = kt_end > kt_beg ? kt_end - kt_beg : 0;
  if constexpr (MK == 1 && NSTR == 2) {
    int c = 0;
    for (int i = tid; i < p.n_kt; i += NT) c += cls_at(i) != 0;
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
    if (lane == 0 && c != 0) atomicAdd(&n_live_lds, c);
  }

  // ---- direct-to-LDS tile loads.  Lane i of copy instruction u fills slot
  // u * 64 + i of the tile: K slot q is row q / KCH, chunk q % KCH (the pad
  // slot, chunk CH, loads chunk 0 again); V slots as Lay places them.  The
  // per-lane byte offsets from the tile's first row are the same for every
  // tile (row strides are below 2^24 elements, so a 64-row tile spans less
  // than 2^31 bytes); rows past Sk read as zeros through the tile's
  // descriptor.
  uint32_t koff[KPW], voff[VPW];
  // (the "& 3" tells the compiler wave_u < 4, so a slot test that holds for
  // every wave folds away instead of costing a branch per copy)
  const int wave_u = __builtin_amdgcn_readfirstlane(wave) & 3;
#pragma unroll
  for (int u = 0; u < KPW; ++u) {
    const int q = (u * 4 + wave_u) * 64 + lane;
    const int ch = q % KCH;
    koff[u] = (uint32_t)(((q / KCH) * kstride + (ch < CH ? ch : 0) * 8) * 2);
  }
#pragma unroll
  for (int u = 0; u < VPW; ++u) {
    const int q = (u * 4 + wave_u) * 64 + lane;
    voff[u] = (uint32_t)((L::v_row(q) * vstride + L::v_chunk(q) * 8) * 2);
  }
  const uint32_t ks_lds = lds_addr(&Ks[str][0][0]), vs_lds = lds_addr(&Vs[str][0][0]);
  // descriptor of one K or V tile: its rows below Sk only, so rows past Sk
  // read as zeros (their keys are masked)
  auto tile_desc = [&](const uint16_t* base, int64_t stride, int kt) -> u32x4_t {
    const int key0 = kt * BN;
    const int rows = min(BN, p.Sk - key0);
    return buf_desc(base + (int64_t)key0 * stride, (uint32_t)(((int64_t)(rows - 1) * stride + D) * 2));
  };
  auto load_k = [&](int kt, int stage) {
    const u32x4_t d = tile_desc(kbase, kstride, kt);
    const uint32_t kdst = ks_lds + stage * (BN * KS * 2);
#pragma unroll
    for (int u = 0; u < KPW; ++u)
      if (u * 4 + wave_u < KINS) lds_dma16_b(d, koff[u], kdst + (u * 4 + wave_u) * 1024);
  };
  auto load_v = [&](int kt, int stage) {
    const u32x4_t d = tile_desc(vbase, vstride, kt);
    const uint32_t vdst = vs_lds + stage * (BN * D * 2);
#pragma unroll
    for (int u = 0; u < VPW; ++u) lds_dma16_b(d, voff[u], vdst + (u * 4 + wave_u) * 1024);
  };
  // the copies of one step spread over its MFMA slots: slot u < KPW is K
  // copy instruction u of this wave, slot KPW + u V copy u.  Every step
  // issues all of them, with no branch (a branch per copy costs more than
  // the copy it would skip) but the one for the K instruction that only
  // some waves have.
  struct DmaPlan {
    u32x4_t dk, dv;
    uint32_t kdst, vdst;
  };
  auto dma_slot = [&](const DmaPlan& pl, int slot) {
    if (slot < KPW) {
      if (slot * 4 + wave_u < KINS) lds_dma16_b(pl.dk, koff[slot], pl.kdst + (slot * 4 + wave_u) * 1024);
    } else {
      const int u = slot - KPW;
      lds_dma16_b(pl.dv, voff[u], pl.vdst + (u * 4 + wave_u) * 1024);
    }
  };


  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
  const int grp = lane >> 4, gi = lane & 15, rr = gi >> 2, cc = gi & 3;
  // element offsets of the operand reads inside a tile (layout: Lay).  K
  // fragment (kb, s): chunk 2s + hh of row kb*32 + l32.  Transposing V read
  // (kb, jj, db): 4 elements at d column db*32 + (grp&1)*16 + 4cc of row
  // kb*32 + jj*16 + 4hh + rr, and of the row 8 further (+ 8 D).
  auto k_off = [&](int kb, int s) { return (kb * 32 + l32) * KS + (2 * s + hh) * 8; };
  const int v_lane = L::v_at(4 * hh + rr, (grp & 1) * 2 + (cc >> 1)) + (cc & 1) * 4;
  auto v_off = [&](int kb, int jj, int db) { return v_lane + kb * 32 * D + jj * 16 * D + db * 128; };

  const f32x16_t zero16 = {};
  // scores of two consecutive tiles; the steady-state loop is unrolled by
  // two so that the arrays swap roles instead of being copied
  f32x16_t sA[2], sB[2];
  float mu = 0.f;  // reference of the exponentials (m, or 0 before any live key)
  // CINIT: the K Q^T accumulators start from -mu in every element, so
  // scores arrive relative to the reference and the exponentials need no
  // subtraction (32 VALU operations fewer per wave and step).  It costs 16
  // registers, which fit everywhere but in the two-stream D 128 kernels;
  // those start from zero and subtract mu before each exponential.
  constexpr bool CINIT = D == 64 || NSTR == 1;
  f32x16_t cinit = {};

  // S^T = K Q^T + cinit of one tile, plain (prologue)
  auto qk = [&](int stage, f32x16_t (&sacc)[2]) {
    const uint16_t* kt_lds = &Ks[str][stage][0];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint4 a = *(const uint4*)&kt_lds[k_off(kb, s)];
        sacc[kb] = mfma32<T>(a, qf[s], s == 0 ? (CINIT ? cinit : zero16) : sacc[kb]);
      }
    }
  };
  // non-live keys of a boundary tile -> -inf.  Key kb*32 + c + hh*4 of the
  // tile (c a compile-time constant per register) is compared through
  // per-tile thresholds, so no per-register key offset stays in registers.
  auto mask_tile = [&](int kt, f32x16_t (&sc)[2]) {
    bool check;
    if constexpr (MK == 2 || MK == 3) check = !(kt >= full_beg && kt < full_end);
    else if constexpr (MK == 1)
      check = (cls_bits ? ((mixed_bits >> kt) & 1) != 0 : cls_at(kt) == 2) || kt >= first_tail_tile;
    else check = kt >= first_tail_tile;
    if (__builtin_expect(check, 0)) {
      // kept a branch (boundary tiles are few): without the barrier to
      // speculation the compiler turns this into selects on every tile
      __asm__ volatile("");
      const int base = kt * BN + hh * 4;
      const int lim = p.Sk - base;       // keys past Sk
      const int lo_t = lo - base, hi_t = hi - base;
      // the lane's key bits of this tile, shifted to its half (keys past Sk
      // carry 0 bits); lanes without a query see none live
      uint64_t kbits = 0;
      if constexpr (MK == 1) {
        if (brow != nullptr) kbits = brow[kt] >> (hh * 4);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int c = kb * 32 + (v >> 2) * 8 + (v & 3);
          bool live;
          if constexpr (MK == 2 || MK == 3) live = c >= lo_t && c < hi_t;
          else if constexpr (MK == 1) live = (kbits >> c) & 1;
          else live = c < lim;
          sc[kb][v] = live ? sc[kb][v] : -INFINITY;
        }
      }
    }
  };
  auto rowmax = [&](const f32x16_t (&sc)[2]) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; v += 2) mx = fmaxf(fmaxf(mx, sc[kb][v]), sc[kb][v + 1]);
    return half_swap_max(mx);
  };

  // Software pipeline over the live key tiles t(0), t(1), ...  During step
  // j, K of t(j+1) and V of t(j) are resident (K one tile ahead of V) while
  // K of t(j+2) and V of t(j+1) stream in; one barrier per step.  LDS
  // operands are read PF MFMAs ahead of their use; a scheduling fence after
  // each MFMA keeps the planned order.
  constexpr int PF = 2;
  uint4 pk[2][2];
  constexpr int NSLOT = KPW + VPW;  // copy instructions per wave and step, at most
  // P.V of one whole tile, P from pk
  auto pv_all = [&](int vstage) {
    const uint16_t* vt_lds = &Vs[str][vstage][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const uint2 a0 = lds_read_tr<T>(&vt_lds[v_off(kb, jj, db)]);
          const uint2 a1 = lds_read_tr<T>(&vt_lds[v_off(kb, jj, db) + 8 * D]);
          oacc[db] = mfma32<T>(make_uint4(a0.x, a0.y, a1.x, a1.y), pk[kb][jj], oacc[db]);
        }
      }
    }
  };
  // the last tile: its exponentials, then its P.V
  auto last_tile = [&](int vstage, f32x16_t (&scur)[2]) {
    float lsa = 0.f, lsb = 0.f;
    uint32_t wv[2][2][4];
    static_for<16>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      constexpr int kb = h >> 3, jj = (h >> 2) & 1, e = h & 3;
      const float p0 = fast_exp2(scur[kb][jj * 8 + 2 * e] - (CINIT ? 0.f : mu));
      const float p1 = fast_exp2(scur[kb][jj * 8 + 2 * e + 1] - (CINIT ? 0.f : mu));
      wv[kb][jj][e] = Elem<T>::pack2(p0, p1);
      if constexpr (e & 1) lsb = Elem<T>::add_pair(wv[kb][jj][e], lsb);
      else lsa = Elem<T>::add_pair(wv[kb][jj][e], lsa);
      if constexpr (e == 3) pk[kb][jj] = make_uint4(wv[kb][jj][0], wv[kb][jj][1], wv[kb][jj][2], wv[kb][jj][3]);
    });
    l_run += lsa + lsb;
    pv_all(vstage);
  };

  // One exponential piece: 2 of the 32 scores of a lane (tile t(j)), packed
  // into P block (kb, jj) and added to the row sum.  The exponentials of a
  // piece are issued in one K Q^T MFMA slot and packed in the next
  // (pack_piece), so the wave, which issues in order, does not wait for
  // their results before its next MFMA (dense rows ~2 % faster).
  constexpr int NQK = 2 * NS, NPV = 4 * ND;
  static_assert(16 % NQK == 0, "exponential pieces spread evenly over the K Q^T MFMAs");
  static_assert(NSLOT <= NPV, "every copy has a P.V slot");
  auto exp_pair = [&](auto hc, f32x16_t (&scur)[2]) -> float2 {
    constexpr int h = decltype(hc)::value;
    constexpr int kb = h >> 3, jj = (h >> 2) & 1, e = h & 3;
    const float p0 = fast_exp2(scur[kb][jj * 8 + 2 * e] - (CINIT ? 0.f : mu));
    const float p1 = fast_exp2(scur[kb][jj * 8 + 2 * e + 1] - (CINIT ? 0.f : mu));
    return make_float2(p0, p1);
  };
  auto pack_piece = [&](auto hc, float2 pp, float& lsa, float& lsb, uint32_t (&wv)[2][2][4]) {
    constexpr int h = decltype(hc)::value;
    constexpr int kb = h >> 3, jj = (h >> 2) & 1, e = h & 3;
    wv[kb][jj][e] = Elem<T>::pack2(pp.x, pp.y);
    __asm__ volatile("" ::"v"(wv[kb][jj][e]));
    if constexpr (e & 1) lsb = Elem<T>::add_pair(wv[kb][jj][e], lsb);
    else lsa = Elem<T>::add_pair(wv[kb][jj][e], lsa);
    if constexpr (e == 3) pk[kb][jj] = make_uint4(wv[kb][jj][0], wv[kb][jj][1], wv[kb][jj][2], wv[kb][jj][3]);
  };

  float mx = -INFINITY;  // row max of the newest scores
  // Steady-state step, split: the 2*NS K Q^T MFMAs of t(j+1) come first,
  // one exponential piece of t(j) after each (P block (kb, jj) is complete
  // before the P.V half starts); then the 4*ND P.V MFMAs of t(j) with the
  // copies of the step and, once the K Q^T results have landed, the mask and
  // row max of t(j+1) (after the half for boolean masks), so that the next
  // step does not wait on them.
  auto step_split = [&](int kstage, int vstage, const DmaPlan& pl, f32x16_t (&scur)[2], f32x16_t (&snext)[2],
                        int kt_next) {
    const uint16_t* kt_lds = &Ks[str][kstage][0];
    const uint16_t* vt_lds = &Vs[str][vstage][0];
    float lsa = 0.f, lsb = 0.f;
    uint32_t wv[2][2][4];
    auto kfrag = [&](auto gc) -> uint4 {
      constexpr int g = decltype(gc)::value, ss = g >> 1, kb = g & 1;
      return *(const uint4*)&kt_lds[k_off(kb, ss)];
    };
    auto vfrag = [&](auto gc) -> uint4 {
      constexpr int g = decltype(gc)::value, kb = g / (2 * ND), jj = (g / ND) & 1, db = g % ND;
      const uint2 a0 = lds_read_tr<T>(&vt_lds[v_off(kb, jj, db)]);
      const uint2 a1 = lds_read_tr<T>(&vt_lds[v_off(kb, jj, db) + 8 * D]);
      return make_uint4(a0.x, a0.y, a1.x, a1.y);
    };
    uint4 frk[PF], frv[PF];
    constexpr int PPS = 16 / NQK;  // exponential pieces per K Q^T MFMA slot
    float2 held[PPS];
    static_for<PF>([&](auto gc) { frk[decltype(gc)::value] = kfrag(gc); });
    static_for<NQK>([&](auto ic) {
      constexpr int i = decltype(ic)::value, ss = i >> 1, kb = i & 1;
      const uint4 f = frk[i % PF];
      if constexpr (i + PF < NQK) frk[i % PF] = kfrag(std::integral_constant<int, i + PF>{});
      else frv[i + PF - NQK] = vfrag(std::integral_constant<int, i + PF - NQK>{});
      snext[kb] = mfma32<T>(f, qf[ss], ss == 0 ? (CINIT ? cinit : zero16) : snext[kb]);
      if constexpr (i > 0)
        static_for<PPS>([&](auto pc) { pack_piece(std::integral_constant<int, (i - 1) * PPS + decltype(pc)::value>{}, held[decltype(pc)::value], lsa, lsb, wv); });
      static_for<PPS>([&](auto pc) { held[decltype(pc)::value] = exp_pair(std::integral_constant<int, i * PPS + decltype(pc)::value>{}, scur); });
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<PPS>([&](auto pc) { pack_piece(std::integral_constant<int, (NQK - 1) * PPS + decltype(pc)::value>{}, held[decltype(pc)::value], lsa, lsb, wv); });
    static_for<NPV>([&](auto ic) {
      constexpr int i = decltype(ic)::value, kb = i / (2 * ND), jj = (i / ND) & 1, db = i % ND;
      const uint4 f = frv[i % PF];
      if constexpr (i + PF < NPV) frv[i % PF] = vfrag(std::integral_constant<int, i + PF>{});
      oacc[db] = mfma32<T>(f, pk[kb][jj], oacc[db]);
      if constexpr (i < NSLOT) dma_slot(pl, i);
      if constexpr (i == 3 && MK != 1) {
        mask_tile(kt_next, snext);
        mx = rowmax(snext);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // boolean masks: a mixed tile loads its key bits, a wait that would
    // also cover the copies just issued, so it comes after the P.V half
    if constexpr (MK == 1) {
      mask_tile(kt_next, snext);
      mx = rowmax(snext);
    }
    l_run += lsa + lsb;
  };

  // this stream's live tiles: every NSTR-th one, starting at its index
  auto advance = [&](int k) {
    k = next_live(k + 1);
    if constexpr (NSTR == 2) {
      if (k < kt_end) k = next_live(k + 1);
    }
    return k;
  };
  // ---- KR: the rows of the one K tile, normalised and rotated in registers
  // and written into K stage 0.  Thread piece u is 8 elements of one row
  // (interleaved pairs inside it) or 8 + 8 elements d0 and d0 + D/2 (half
  // split); the pieces of a row are adjacent lanes, so the row's RMSNorm sum
  // is a shuffle reduction over them.  Every load of the tile (rows, norm
  // weights, the keys' cos / sin rows) is issued right after the Q loads,
  // then the V tile copy, so
  // the three are in flight together.  Rows past Sk are
  // written as zeros (their keys are masked).  The arithmetic is the K
  // pass's (k_rotate16_kernel).
  auto kr_tile = [&](int t) {
    constexpr bool HALF = KR == 2;
    constexpr int Q8 = HALF ? D / 16 : D / 8;  // threads per row
    constexpr int NPC = BN * Q8 / 256;         // pieces per thread
    constexpr int NE = HALF ? 16 : 8;          // elements per piece
    constexpr int NP = HALF ? 8 : 4;           // pairs per piece
    const uint16_t* src = (const uint16_t*)p.k + b * p.ks[0] + hk * p.ks[1];
    const bool rot = hk < p.n_rotk;
    const bool norm = p.k_norm_w != nullptr;
    u32x4_t a0[NPC], a1[NPC], w0[NPC], w1[NPC];
    float4 tv[NPC * (NP / 2)];
    int jr[NPC];
    // The V tile's copies go first.  The compiler waits for the K rows
    // below by counting only the loads it can see (the copies are opaque to
    // it), so copies issued after the K loads would be waited for too;
    // issued before them they land first (vector memory completes in
    // order), and the wait for the K rows costs nothing more.
    load_v(t, 0);
    // (loads unconditional or under wave-uniform branches only, as in the
    // Q prologue)
#pragma unroll
    for (int u = 0; u < NPC; ++u) jr[u] = min(t * BN + (tid + u * 256) / Q8, p.Sk - 1);
    // piece block u covers rows [u * 256 / Q8, (u + 1) * 256 / Q8) of the
    // tile; a block wholly past Sk loads nothing (a work-group-uniform
    // branch) and writes zeros
    bool u_live[NPC];
#pragma unroll
    for (int u = 0; u < NPC; ++u) u_live[u] = t * BN + u * (256 / Q8) < p.Sk;
    const u32x4_t zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < NPC; ++u) {
      const int d0 = ((tid + u * 256) % Q8) * 8;
      const uint16_t* row = src + (int64_t)jr[u] * p.ks[2] + d0;
      const uint16_t* wr = (const uint16_t*)p.k_norm_w + d0;
      a0[u] = a1[u] = w0[u] = w1[u] = zero4;
      if (u_live[u]) {
        a0[u] = *(const u32x4_t*)row;
        a1[u] = a0[u];
        if constexpr (HALF) a1[u] = *(const u32x4_t*)(row + D / 2);
      }
      if (norm && u_live[u]) {
        w0[u] = *(const u32x4_t*)wr;
        w1[u] = w0[u];
        if constexpr (HALF) w1[u] = *(const u32x4_t*)(wr + D / 2);
      }
    }
    if (rot) {
#pragma unroll
      for (int u = 0; u < NPC; ++u) {
        if (!u_live[u]) {
#pragma unroll
          for (int k = 0; k < NP / 2; ++k) tv[u * (NP / 2) + k] = make_float4(0.f, 0.f, 0.f, 0.f);
          continue;
        }
        const int d0 = ((tid + u * 256) % Q8) * 8;
        const float4* trow = (const float4*)(p.k_cs + ((size_t)b * p.k_cs_sb + jr[u]) * (D / 2) + (HALF ? d0 : d0 / 2));
#pragma unroll
        for (int k = 0; k < NP / 2; ++k) tv[u * (NP / 2) + k] = trow[k];
      }
    }
    uint16_t* kst = &Ks[0][0][0];
#pragma unroll
    for (int u = 0; u < NPC; ++u) {
      const int piece = tid + u * 256;
      const int r = piece / Q8, d0 = (piece % Q8) * 8;
      const bool valid = t * BN + r < p.Sk;
      if (!u_live[u]) {
        *(uint4*)&kst[r * KS + d0] = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (HALF) *(uint4*)&kst[r * KS + d0 + D / 2] = make_uint4(0u, 0u, 0u, 0u);
        continue;
      }
      float x[NE];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = Elem<T>::to_f32((uint16_t)(a0[u][e / 2] >> (16 * (e & 1))));
      if constexpr (HALF) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 + e] = Elem<T>::to_f32((uint16_t)(a1[u][e / 2] >> (16 * (e & 1))));
      }
      if (norm) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < NE; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
        for (int off = Q8 / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
        const float inv = rsqrtf(ss / (float)D + p.norm_eps);
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const uint32_t w = e < 8 ? w0[u][(e & 7) / 2] : w1[u][(e & 7) / 2];
          x[e] = x[e] * inv * Elem<T>::to_f32((uint16_t)(w >> (16 * (e & 1))));
        }
      }
      if (rot) {
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          const float4 tq = tv[u * (NP / 2) + q / 2];
          const float2 cs = (q & 1) ? make_float2(tq.z, tq.w) : make_float2(tq.x, tq.y);
          const int ia = HALF ? q : 2 * q, ic = HALF ? 8 + q : 2 * q + 1;
          const float a = x[ia], c = x[ic];
          x[ia] = fmaf(a, cs.x, -c * cs.y);
          x[ic] = fmaf(c, cs.x, a * cs.y);
        }
      }
      uint32_t o0[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) o0[q] = valid ? Elem<T>::pack2(x[2 * q], x[2 * q + 1]) : 0u;
      *(uint4*)&kst[r * KS + d0] = make_uint4(o0[0], o0[1], o0[2], o0[3]);
      if constexpr (HALF) {
        uint32_t o1[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o1[q] = valid ? Elem<T>::pack2(x[8 + 2 * q], x[8 + 2 * q + 1]) : 0u;
        *(uint4*)&kst[r * KS + d0 + D / 2] = make_uint4(o1[0], o1[1], o1[2], o1[3]);
      }
    }
  };

  int kt = next_live(kt_beg);
  if (NSTR == 2 && str == 1 && kt < kt_end) kt = next_live(kt + 1);
  int kn = kt < kt_end ? advance(kt) : kt_end;
  if constexpr (KR != 0) {
    if (kt < kt_end) kr_tile(kt);  // (rows of one key tile: kn is past the end)
  } else {
    if (kt < kt_end) {
      load_k(kt, 0);
      load_v(kt, 0);
    }
    if (kn < kt_end) load_k(kn, 1);
  }
  finish_q();
  // every prologue load completes here (the first tile copies are in flight
  // meanwhile), so that no wait for one is left inside the tile loop, where
  // it would also wait for the tile copies
#pragma unroll
  for (int s = 0; s < NS; ++s) __asm__ volatile("" ::"v"(qf[s].x), "v"(qf[s].y), "v"(qf[s].z), "v"(qf[s].w));
  __asm__ volatile("" ::"v"(lo), "v"(hi));
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  auto rescale_step = [&](f32x16_t (&sc)[2]) {
    // ---- online softmax with lazy rescaling.  The reference m of a query
    // moves only when a score exceeds it by more than 2^8 (otherwise the
    // exponentials stay below 256); numerator and denominator always share
    // it, so the result is the same softmax.  With CINIT, scores and mx are
    // relative to the current reference mu, and a move shifts the scores of
    // the tile at hand and the start value of the next ones.
    const float mx_abs = CINIT ? mu + mx : mx;
    const bool need = m_run == -INFINITY ? mx > -INFINITY : mx_abs > m_run + LAZY_RESCALE_LOG2;
    if (__any(need)) {
      const float m_new = need ? mx_abs : m_run;
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
      const float mu_new = m_new == -INFINITY ? 0.f : m_new;
      const float shift = mu - mu_new;
      m_run = m_new;
      mu = mu_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
      if constexpr (CINIT) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) sc[kb][v] += shift;
#pragma unroll
        for (int v = 0; v < 16; ++v) cinit[v] = -mu;
      }
    }
  };
  auto step_top = [&](int j) {
    // K of t(j+1) and V of t(j) have landed once this barrier passes, and
    // every wave is done with the stages the next copies overwrite
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  int j = 0;
  // copies of one step: K of t(j+2) and V of t(j+1).  On the last steady
  // step there is no t(j+2); K of t(j+1) is copied again instead, into the
  // stage that held K of t(j), which no later step reads.
  auto plan_step = [&](int kn2) {
    DmaPlan pl;
    pl.dk = tile_desc(kbase, kstride, kn2 < kt_end ? kn2 : kn);
    pl.kdst = ks_lds + (j & 1) * (BN * KS * 2);
    pl.dv = tile_desc(vbase, vstride, kn);
    pl.vdst = vs_lds + ((j + 1) & 1) * (BN * D * 2);
    return pl;
  };
  // one steady-state step: tile t(j) scores in sc, t(j+1) scores into sn
  auto steady = [&](f32x16_t (&sc)[2], f32x16_t (&sn)[2]) {
    step_top(j);
    const int kn2 = advance(kn);
    // K of t(j+2) and V of t(j+1), issued between the MFMAs of this step
    const DmaPlan pl = plan_step(kn2);
    rescale_step(sc);
    step_split((j + 1) & 1, j & 1, pl, sc, sn, kn);
    kt = kn;
    kn = kn2;
    ++j;
  };
  if (kt < kt_end) {
    qk(0, sA);
    mask_tile(kt, sA);
    mx = rowmax(sA);
    bool in_b = false;  // the current tile's scores are in sB
    while (kn < kt_end) {
      steady(sA, sB);
      if (kn >= kt_end) {
        in_b = true;
        break;
      }
      steady(sB, sA);
    }
    // the last tile
    step_top(j);
    if (in_b) {
      rescale_step(sB);
      last_tile(j & 1, sB);
    } else {
      rescale_step(sA);
      last_tile(j & 1, sA);
    }
  }

  if constexpr (NSTR == 2) {
    // a stream passes one barrier per live tile it takes (plus the prologue
    // one), so stream 1 passes one fewer when the count is odd
    if constexpr (MK == 1) n_live = n_live_lds;  // counted before the prologue barrier
    if (str == 1 && (n_live & 1)) __syncthreads();
    // no K stage is read any more (a last P.V, from V stages, may still be
    // running): stream 1 parks (m, l, O^T) in the K stages, lane-major so
    // that each access is a conflict-free 16-byte one, and stream 0 folds
    // it in
    static_assert(sizeof(float) * (4 * ND * 16 * 64 + 2 * 4 * 64) <= sizeof(Ks), "partials fit the K stages");
    float* part = reinterpret_cast<float*>(&Ks[0][0][0]);
    float2* part_ml = reinterpret_cast<float2*>(part + 4 * ND * 16 * 64);
    if (str == 1) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
          *(float4*)&part[((wave * ND + db) * 4 + v4) * 256 + lane * 4] =
              make_float4(oacc[db][v4 * 4], oacc[db][v4 * 4 + 1], oacc[db][v4 * 4 + 2], oacc[db][v4 * 4 + 3]);
      part_ml[wave * 64 + lane] = make_float2(m_run, l_run);
    }
    __syncthreads();
    if (str == 1) return;
    // both partials are relative to their own reference (m, or nothing
    // accumulated when m = -inf); rebase both to the larger one
    const float2 mlb = part_ml[wave * 64 + lane];
    const float m_new = fmaxf(m_run, mlb.x);
    const float fa = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
    const float fb = mlb.x == -INFINITY ? 0.f : fast_exp2(mlb.x - m_new);
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const float4 y = *(const float4*)&part[((wave * ND + db) * 4 + v4) * 256 + lane * 4];
        oacc[db][v4 * 4 + 0] = oacc[db][v4 * 4 + 0] * fa + y.x * fb;
        oacc[db][v4 * 4 + 1] = oacc[db][v4 * 4 + 1] * fa + y.y * fb;
        oacc[db][v4 * 4 + 2] = oacc[db][v4 * 4 + 2] * fa + y.z * fb;
        oacc[db][v4 * 4 + 3] = oacc[db][v4 * 4 + 3] * fa + y.w * fb;
      }
    l_run = l_run * fa + mlb.y * fb;
    m_run = m_new;
  }

  // ---- epilogue: O = O^T / l, lse
  const float l_tot = half_swap_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // One key stream, all 32 rows of the wave inside Sq (a wave-uniform
  // test): the wave stages its output rows in its own quarter of the K
  // stages (no K stage is read after the last step's barrier) and stores
  // whole rows, 1 KB per instruction, where the MFMA layout would store 16
  // bytes of each of 32 rows per instruction.  (A partly filled wave, as in
  // rows of a few tokens, keeps the direct stores: there the staging's LDS
  // round trip measured slower than the scattered stores it saves.)
  if (NSTR == 1 && qt * BM + __builtin_amdgcn_readfirstlane(wave) * 32 + 32 <= p.Sq) {
    constexpr int OS = KS;                     // padded row, elements
    constexpr int NCH = D / 8;                 // 16-byte chunks per row
    static_assert(4 * 32 * OS <= 2 * BN * KS, "four waves' rows fit the K stages");
    uint16_t* ost = &Ks[0][0][0] + wave * 32 * OS;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        uint2 st;
        st.x = Elem<T>::pack2(oacc[db][g4 * 4 + 0] * inv, oacc[db][g4 * 4 + 1] * inv);
        st.y = Elem<T>::pack2(oacc[db][g4 * 4 + 2] * inv, oacc[db][g4 * 4 + 3] * inv);
        *(uint2*)&ost[l32 * OS + db * 32 + g4 * 8 + hh * 4] = st;
      }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    const int q0 = qt * BM + wave * 32;
    uint16_t* obase = (uint16_t*)p.o + b * p.os[0] + h * p.os[1];
#pragma unroll
    for (int it = 0; it < 32 * NCH / 64; ++it) {
      const int q = it * 64 + lane, r = q / NCH, c = q % NCH;
      const uint4 v = *(const uint4*)&ost[r * OS + c * 8];
      if (q0 + r < p.Sq) *(uint4*)(obase + (int64_t)(q0 + r) * p.os[2] + c * 8) = v;
    }
    if (qvalid && p.lse != nullptr && hh == 0)
      p.lse[((int64_t)b * p.Hq + h) * p.Sq + qi] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    return;
  }
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


// Launchers of fwd_mfma_kernel for one element type and head_dim (defined
// in fwd_mfma_<type>_d<D>.hip): nstr key streams, kr: K rotated in the
// kernel (short rows).
void launch_mfma_bf16_d64(const FwdParams& p, unsigned nwork, int nstr, bool kr, hipStream_t s);
void launch_mfma_bf16_d128(const FwdParams& p, unsigned nwork, int nstr, bool kr, hipStream_t s);
void launch_mfma_f16_d64(const FwdParams& p, unsigned nwork, int nstr, bool kr, hipStream_t s);
void launch_mfma_f16_d128(const FwdParams& p, unsigned nwork, int nstr, bool kr, hipStream_t s);

template <typename T, int D, int NSTR, int KR>
inline void launch_mfma_n(const FwdParams& p, unsigned nwork, hipStream_t s) {
  const dim3 blk(256 * NSTR);
  if (p.mask_kind == 3) fwd_mfma_kernel<T, D, 3, NSTR, KR><<<dim3(nwork), blk, 0, s>>>(p);
  else if (p.mask_kind == 2) fwd_mfma_kernel<T, D, 2, NSTR, KR><<<dim3(nwork), blk, 0, s>>>(p);
  else if (p.mask_kind == 1) fwd_mfma_kernel<T, D, 1, NSTR, KR><<<dim3(nwork), blk, 0, s>>>(p);
  else fwd_mfma_kernel<T, D, 0, NSTR, KR><<<dim3(nwork), blk, 0, s>>>(p);
}

template <typename T, int D>
inline void launch_mfma_td(const FwdParams& p, unsigned nwork, int nstr, bool kr, hipStream_t s) {
  if (kr && p.rope_style == 1) launch_mfma_n<T, D, 1, 2>(p, nwork, s);
  else if (kr) launch_mfma_n<T, D, 1, 1>(p, nwork, s);
  else if (nstr == 2) launch_mfma_n<T, D, 2, 0>(p, nwork, s);
  else launch_mfma_n<T, D, 1, 0>(p, nwork, s);
}

}  // namespace mz
