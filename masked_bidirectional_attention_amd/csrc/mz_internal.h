// Host <-> kernel plumbing for mzattn: parameter blocks and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mz {

// Tile sizes of the forward: queries per work-group, keys per iteration.
constexpr int FWD_BM = 128;
constexpr int FWD_BN = 64;
// fp32 forward: queries per work-group, keys per LDS tile.
constexpr int F32_BM = 64;
constexpr int F32_BN = 32;
// Decode: keys per chunk (fixed, aligned to key index 0).
constexpr int DEC_CHUNK = 128;

// Rotary embedding: base, optional per-pair factors (LongRoPE), scale of
// cos / sin, and how cos / sin are formed (0 exact, 1 fp16 angles, 2 bf16
// table).
struct RopeSpec {
  double log2_base;
  const float* factors;  // [D/2] (device) or nullptr
  float mscale;          // 1 when not given
  int precision;
};

enum PosMode { POS_ARANGE = 0, POS_ARRAY = 1, POS_SEGMENT = 2 };

struct FwdParams {
  int dtype, B, Hq, Hkv, G, Sq, Sk, D;
  int n_qt, n_kt;  // query tiles (FWD_BM or F32_BM), key tiles (FWD_BN)
  int mask_kind;
  int key_streams;   // 0 automatic, 1 or 2 forced (16-bit kernel)
  float scale_log2;  // scale * log2(e)
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t qs[3], ks[3], vs[3], os[3];
  // rotary embedding; the K pass covers heads [0, n_rot_kv) (rotated when
  // below n_rotk, normalised when k_norm_w is set)
  int n_rot, n_rot_kv, n_rotk;
  // q / k RMSNorm weights [D] (storage dtype) or nullptr
  const void* q_norm_w;
  const void* k_norm_w;
  float norm_eps;
  int rope_style;  // 0 interleaved (2i, 2i+1), 1 half split (i, i + D/2)
  RopeSpec rs;
  int pos_q_mode, pos_k_mode;
  const int32_t* pos_q;  // user array (POS_ARRAY) or derived (POS_SEGMENT)
  int64_t pos_q_sb;
  const int32_t* pos_k;  // user array (POS_ARRAY) or derived (POS_SEGMENT)
  int64_t pos_k_sb;
  float2* rope_tab;  // cos / sin of positions [0, rope_tab_len) (plan)
  int rope_tab_len;
  // cos / sin rows: query i of batch row b rotates with the D/2 pairs at
  // q_cs + (b * q_cs_sb + i) * D/2, key j with k_cs + (b * k_cs_sb + j) * D/2.
  // Index positions read the table itself (sb 0); explicit or
  // segment-derived positions read per-row arrays (q_rows / k_rows, 1 or B
  // batch rows) that the plan fills from the same formula.
  const float2* q_cs;
  int64_t q_cs_sb;
  const float2* k_cs;
  int64_t k_cs_sb;
  float2* q_rows;
  float2* k_rows;
  int q_rows_b, k_rows_b;
  // the queries' cos / sin again, chunk-major for the 16-bit kernels' Q
  // prologue: float4 (pairs 2c, 2c + 1) of query i at q_cst + b * q_cst_sb
  // + c * Sq + i, c < D / 4 (q_cst_b batch rows, sb 0 when shared), so the
  // 32 queries of a wave read 512 contiguous bytes per load
  float4* q_cst;
  int64_t q_cst_sb;
  int q_cst_b;
  void* k_rot;  // [B][n_rot_kv][Sk][D], storage dtype
  // boolean mask
  const uint8_t* mask;
  int64_t ms[4];
  int Bm, Hm;
  int mask_vec16;
  uint8_t* tile_cls;  // [Bm][Hm][n_qt][n_kt]
  // [Bm][Hm][mask_rows][n_kt] key bits of every (query, key tile): bit c of
  // word (i, t) is key t * FWD_BN + c (0 past Sk).  16-bit kernels only.
  uint64_t* mask_bits;
  int mask_rows;  // Sq, or 1 for a mask broadcast over queries
  // segments
  const int32_t* seg_q;
  const int32_t* seg_k;
  int64_t seg_q_sb, seg_k_sb;
  int2* q_range;   // [B][Sq] live key range of each query
  int4* qt_range;  // [B][n_qt] (first tile, end tile, first full tile, end full tile)
  int32_t* qpos_ws;  // [B][Sq] derived query positions
  int32_t* kpos_ws;  // [B][Sk] derived key positions
  float* lse;
};

struct DecodeParams {
  int dtype, B, Hq, Hkv, G, T, R, C, span, D;
  int n_chunks;
  float scale_log2;
  const void* q;  // possibly the rotated copy in the workspace
  int64_t qs[3];
  const void* k;
  int64_t ks[3];
  const void* v;
  int64_t vs[3];
  void* o;
  int64_t os[3];
  const uint8_t* mask;  // may be NULL
  int64_t ms[4];
  // rotary embedding of q (pre-kernel)
  const void* q_in;
  int64_t q_in_s[3];
  const int32_t* q_pos;
  int64_t q_pos_sb;
  RopeSpec rs;
  int rope;
  int rope_style;  // 0 interleaved, 1 half split
  // append step (mzattn_decode_append): the new tokens' rows come from
  // k_new / v_new, go into the caches at len[b] + t, and rotate in the
  // chunk kernel
  int app;
  const int32_t* len;
  int64_t len_sb;
  const void* k_new;
  int64_t kn_s[3];
  const void* v_new;
  int64_t vn_s[3];
  void* k_w;  // the caches, writable (same as k / v)
  void* v_w;
  int32_t* overflow;
  // workspace
  float2* part_ml;     // [B][Hkv][n_chunks][R]   (m in log2 units, l)
  float* part_acc;     // [B][Hkv][n_chunks][R][D]
};

hipError_t launch_fwd_plan(const FwdParams& p, hipStream_t s);
hipError_t launch_fwd_rotate(const FwdParams& p, hipStream_t s);
hipError_t launch_fwd_main(const FwdParams& p, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);

}  // namespace mz
