/*
 * mzattn.h - masked bidirectional multi-head attention for AMD Instinct
 * MI355X (gfx950), C ABI.
 *
 * Two operations, both defined by the source pages of three speech engines:
 *
 *   mzattn_fwd     softmax(scale * Q K^T restricted to live keys) V with no
 *                  causal mask.  The live set comes from a 4-D boolean mask
 *                  (OmniVoice page, "What matches upstream", attention-mask
 *                  bullet: a full 4-D boolean mask, K/V heads repeated to
 *                  the query heads) or from segment ids that pack the
 *                  conditional and unconditional guidance rows side by side
 *                  under a block-diagonal mask, positions restarting at 0 in
 *                  each segment (OmniVoice page, "Memory and speed",
 *                  packed_guidance).  Optional interleaved rotary embedding
 *                  on all heads or on the first pe_attn_head heads (F5-TTS
 *                  page, "Variants" table and "How it works").
 *
 *   mzattn_decode  one generation step: a few queries against a static KV
 *                  cache under an explicit boolean mask, over the key span
 *                  [0, span) (VoxCPM page, "What matches upstream",
 *                  attention bullet, and "Memory and speed",
 *                  attention_span).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller.  The
 *   library never allocates, frees or keeps device memory between calls;
 *   scratch space is the caller's `workspace`.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *   stream).  Buffers must stay valid until the stream has passed the call.
 * - Every argument is checked on the host before anything is launched; on
 *   error nothing is written and a negative status is returned.
 *   mzattn_last_error() then gives a thread-local detail message.
 * - Q, K, V and O share one element type (mz_dtype).  Element strides are
 *   given for the (batch, head, sequence) dims; the head_dim dim is
 *   contiguous (stride 1).  Base pointers must be 16-byte aligned and every
 *   stride a multiple of 8 elements (fp16/bf16) or 4 elements (fp32).
 *   mzattn_fwd also needs the K and V sequence strides below 2^24 elements
 *   (MZ_ERR_UNSUPPORTED otherwise).
 * - Boolean masks are bytes, nonzero = the key takes part; each of the 4
 *   mask strides (in bytes) may be 0 to broadcast that dim, the last
 *   (key) stride must be 1.
 * - A query with no live key produces an all-zero output row (and
 *   lse = -inf).  Masked keys contribute exactly nothing: any finite
 *   values in masked K/V positions leave the output unchanged.  NaN or Inf
 *   in masked positions is outside the contract.
 * - Fully masked query rows, empty batches and empty sequences are legal.
 */
#ifndef MZATTN_H_
#define MZATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MZATTN_VERSION 400 /* major * 10000 + minor * 100 + patch */

/* ---- status codes ------------------------------------------------------ */
#define MZ_OK 0
#define MZ_ERR_NULL (-1)        /* a required pointer is NULL                 */
#define MZ_ERR_SHAPE (-2)       /* inconsistent or out-of-range sizes         */
#define MZ_ERR_DTYPE (-3)       /* unknown element type                       */
#define MZ_ERR_STRIDE (-4)      /* negative stride, or a stride the kernels
                                   cannot take (mask key stride != 1)         */
#define MZ_ERR_ALIGN (-5)       /* base pointer / stride misaligned           */
#define MZ_ERR_UNSUPPORTED (-6) /* valid request the library does not cover   */
#define MZ_ERR_WORKSPACE (-7)   /* workspace missing, too small or misaligned */
#define MZ_ERR_ABI (-8)         /* struct_size does not match this library    */
#define MZ_ERR_HIP (-9)         /* a HIP launch failed                        */
#define MZ_ERR_VALUE (-10)      /* bad scalar: scale, rope_base, span ...     */

/* ---- enums ------------------------------------------------------------- */
typedef enum mz_dtype { MZ_F32 = 0, MZ_F16 = 1, MZ_BF16 = 2 } mz_dtype;

typedef enum mz_mask_kind {
  MZ_MASK_NONE = 0,    /* every key is live                                  */
  MZ_MASK_BOOL = 1,    /* live(b,h,i,j) = mask[b,h,i,j] != 0                 */
  MZ_MASK_SEGMENT = 2, /* live(b,i,j) = seg_q[b,i] >= 0 && seg_q[b,i] == seg_k[b,j] */
  MZ_MASK_CAUSAL = 3   /* live(i,j) = j <= i (top-left aligned, as SDPA's is_causal;
                          the prefill of the VoxCPM page, "What matches upstream",
                          attention bullet); mask and seg pointers are ignored */
} mz_mask_kind;

/* ---- mzattn_fwd -------------------------------------------------------- */
/*
 * Layouts (element strides, d contiguous):
 *   q [batch, heads_q,  seq_q, head_dim]   o  same shape as q
 *   k [batch, heads_kv, seq_k, head_dim]   v  same shape as k
 * GQA: heads_q must be a multiple of heads_kv; query head h reads K/V head
 * h / (heads_q / heads_kv) (each K/V head repeated G times in a row).
 * head_dim: 64 or 128.  seq_q, seq_k: 0 .. 2^20.
 *
 * scale: <= 0 selects 1/sqrt(head_dim); otherwise used as given.
 * rope_base: 0 = no rotary embedding; > 0 rotates the pairs of q and k
 *   chosen by rope_style by pos * rope_base^(-2i/head_dim), pair i.
 * rope_style: 0 = interleaved, pair i is (x[2i], x[2i+1]) (F5-TTS page,
 *   x-transformers style); 1 = half split, pair i is (x[i], x[i+D/2]) (the
 *   "rotate half" layout of Llama-family models).  Other values:
 *   MZ_ERR_VALUE.
 * rope_factors: optional device fp32 [head_dim/2]; pair i then rotates by
 *   pos * theta_i / rope_factors[i] (LongRoPE's per-dimension rescaling,
 *   the MiniCPM-4 LM of the VoxCPM page, "How it works").  NULL = 1.
 * rope_mscale: cosines and sines are multiplied by it (LongRoPE's
 *   attention factor); 0 = 1.
 * rope_precision: how the cosines and sines are formed.
 *   0 = exact: the angle in fp64, cos and sin to fp32 (the default);
 *   1 = fp16 angles: theta_i and the position rounded to fp16, their
 *       product rounded to fp16, its cos and sin rounded to fp16 (the F5-TTS
 *       page, "What matches upstream": on GPU the model runs in fp16 and so
 *       do inv_freq and the angles);
 *   2 = bf16 table: angle pos * fp32(theta_i) in fp32, cos and sin in fp32
 *       times rope_mscale, rounded to bf16 (the VoxCPM page: the LongRoPE
 *       table is built in fp32 and rounded with the model to bf16).
 *   Other values: MZ_ERR_VALUE.  The same fields, with the same meaning,
 *   are in mzattn_decode_args and mzattn_decode_append_args.
 * q_norm_w / k_norm_w: optional [head_dim] weights in the storage dtype,
 *   16-byte aligned.  Every q (k) row is first scaled to unit root mean
 *   square and multiplied by the weight, x / sqrt(mean(x^2) + norm_eps) *
 *   w, in fp32, before RoPE (the Qwen3 LM of the OmniVoice page normalises
 *   q and k separately, as transformers does).  NULL: no normalisation.
 * norm_eps: finite, >= 0 (used when a weight is given).
 * pe_attn_head: < 0 rotates every head; n >= 0 rotates query heads 0..n-1
 *   and the K heads they read.  With GQA only "none" (0) or "all" (< 0 or
 *   >= heads_q) is accepted (MZ_ERR_UNSUPPORTED otherwise).
 * pos_q / pos_k: optional int32 positions [batch, seq] with batch stride
 *   pos_*_stride_b (0 = shared by all rows).  When NULL: 0..seq-1, or in
 *   MZ_MASK_SEGMENT mode the index within the token's segment.
 * mask: bytes, [batch|1, heads_q|1, seq_q|1, seq_k] via mask_stride.
 * seg_q / seg_k: int32 [batch, seq] segment ids, non-decreasing along each
 *   row (each id occupies one contiguous run); ids < 0 mark padding, which
 *   neither attends nor is attended to.  Results for rows that violate the
 *   ordering are unspecified (memory accesses stay in bounds).
 * lse: optional fp32 [batch, heads_q, seq_q] (contiguous), natural-log
 *   log-sum-exp of the scaled live scores; -inf for rows with no live key.
 * workspace: device scratch of at least mzattn_fwd_workspace_size() bytes,
 *   256-byte aligned; contents need no initialisation.
 * key_streams: 0 lets the library choose how the 16-bit kernel walks the
 *   key tiles of one query tile; 1 forces one chain of steps per query tile,
 *   2 two chains over alternate tiles merged at the end (a tuning and test
 *   override: the results agree within rounding).  Other values:
 *   MZ_ERR_VALUE.  The fp32 kernel ignores it.
 */
typedef struct mzattn_fwd_args {
  uint32_t struct_size; /* = sizeof(mzattn_fwd_args), else MZ_ERR_ABI */
  int32_t dtype;        /* mz_dtype */
  int32_t batch, heads_q, heads_kv, seq_q, seq_k, head_dim;
  int32_t pe_attn_head;
  int32_t mask_kind;    /* mz_mask_kind */
  float scale;
  int32_t rope_style;   /* 0 interleaved, 1 half split */
  double rope_base;
  int32_t rope_precision;     /* 0 exact, 1 fp16 angles, 2 bf16 table */
  float rope_mscale;          /* cos / sin scale; 0 = 1 */
  const float* rope_factors;  /* optional device [head_dim/2], NULL = 1 */
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3]; /* (b, h, s) */
  const int32_t* pos_q;
  const int32_t* pos_k;
  int64_t pos_q_stride_b, pos_k_stride_b;
  const uint8_t* mask;
  int64_t mask_stride[4]; /* bytes, (b, h, i, j); j stride must be 1 */
  const int32_t* seg_q;
  const int32_t* seg_k;
  int64_t seg_q_stride_b, seg_k_stride_b;
  const void* q_norm_w;   /* optional [head_dim], storage dtype */
  const void* k_norm_w;   /* optional [head_dim], storage dtype */
  float norm_eps;
  float* lse;
  void* workspace;
  size_t workspace_bytes;
  int32_t key_streams;  /* 0 automatic, 1 or 2 forced */
} mzattn_fwd_args;

/* Launch the forward on `stream`.  Returns MZ_OK or a negative status.
 * Equivalent to mzattn_fwd_plan followed by mzattn_fwd_execute. */
int mzattn_fwd(const mzattn_fwd_args* args, void* stream);

/* The two halves of mzattn_fwd, for callers that run one layout (mask or
 * segment ids, positions, RoPE settings, shapes) over many inputs, as a
 * sampling loop does.
 *
 * mzattn_fwd_plan launches the prepasses that depend on the layout only and
 * writes their results into the workspace: the RoPE cosines and sines (a
 * table of the index positions 0 .. seq-1, and one row per query or key
 * whose position is given or derived from segment ids), per-query key
 * ranges and positions derived from the segment ids, and the class of every
 * (query tile, key tile) pair of a boolean mask.  It reads no Q, K or V.
 *
 * mzattn_fwd_execute launches the per-input work: the rotation of the K
 * heads that get RoPE into the workspace, then the attention kernel.  It
 * must follow a plan with the same arguments on the same stream (or after
 * the plan completed), with the workspace, mask, segment ids and positions
 * unchanged since; Q, K, V and O may change between executes.
 * mzattn_fwd_rotate_k and mzattn_fwd_attend are its two steps, in that
 * order, for callers that time them separately.
 *
 * Same argument checks and status codes as mzattn_fwd. */
int mzattn_fwd_plan(const mzattn_fwd_args* args, void* stream);
int mzattn_fwd_execute(const mzattn_fwd_args* args, void* stream);
int mzattn_fwd_rotate_k(const mzattn_fwd_args* args, void* stream);
int mzattn_fwd_attend(const mzattn_fwd_args* args, void* stream);

/* Bytes of workspace the call needs (depends on shapes, dtype, mask kind,
 * RoPE); pointer fields are not read.  Returns MZ_OK or a status. */
int mzattn_fwd_workspace_size(const mzattn_fwd_args* args, size_t* bytes);

/* Host-only check of every argument; makes no HIP call. */
int mzattn_validate_fwd(const mzattn_fwd_args* args);

/* ---- mzattn_decode ----------------------------------------------------- */
/*
 * Layouts (element strides, d contiguous):
 *   q        [batch, heads_q,  q_len,     head_dim]   o same shape as q
 *   k_cache  [batch, heads_kv, cache_len, head_dim]   v_cache same shape
 * Keys j in [0, span) are considered, span <= cache_len; key j is live for
 * query t of head h iff j < span and mask[b, h, t, j] != 0 (mask NULL =
 * every key in the span).  The cache holds keys already rotated; with
 * rope_base > 0 the queries are rotated at q_pos [batch, q_len] (int32,
 * batch stride q_pos_stride_b, required then), pairs chosen by rope_style
 * as in mzattn_fwd_args.  q_len: 1 .. 16.
 * heads_q / heads_kv * q_len must not exceed 64.  head_dim: 64 or 128.
 *
 * The result does not depend on span beyond the last live key, bit for
 * bit: keys are reduced in fixed 128-key chunks aligned to key index 0,
 * the chunk partials are folded in an order fixed by chunk index, and a
 * chunk with no live key is an exact identity.
 *
 * workspace: at least mzattn_decode_workspace_size() bytes, 256-byte
 * aligned; contents need no initialisation.  It holds the per-chunk
 * partials; calls sharing a workspace must not overlap in time (use one
 * workspace per stream).  Its size depends on cache_len, not on span, so
 * one workspace serves every step of a generation.
 */
#define MZATTN_DECODE_CHUNK 128

typedef struct mzattn_decode_args {
  uint32_t struct_size; /* = sizeof(mzattn_decode_args), else MZ_ERR_ABI */
  int32_t dtype;
  int32_t batch, heads_q, heads_kv, q_len, head_dim, cache_len, span;
  float scale;
  int32_t rope_style;   /* 0 interleaved, 1 half split */
  double rope_base;
  int32_t rope_precision;     /* 0 exact, 1 fp16 angles, 2 bf16 table */
  float rope_mscale;          /* cos / sin scale; 0 = 1 */
  const float* rope_factors;  /* optional device [head_dim/2], NULL = 1 */
  const void* q;
  int64_t q_stride[3];
  const void* k_cache;
  int64_t k_stride[3];
  const void* v_cache;
  int64_t v_stride[3];
  void* o;
  int64_t o_stride[3];
  const int32_t* q_pos;
  int64_t q_pos_stride_b;
  const uint8_t* mask;
  int64_t mask_stride[4]; /* bytes, (b, h, t, j); j stride must be 1 */
  void* workspace;
  size_t workspace_bytes;
} mzattn_decode_args;

int mzattn_decode(const mzattn_decode_args* args, void* stream);
int mzattn_decode_workspace_size(const mzattn_decode_args* args, size_t* bytes);
int mzattn_validate_decode(const mzattn_decode_args* args);

/* mzattn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks, kernels and result as mzattn_decode, except that
 * args->workspace and args->workspace_bytes are ignored: the partials go
 * to a device array of MZATTN_NOALLOC_SCRATCH_BYTES bytes inside this
 * library, one per GPU, which each GPU holds from its first call until the
 * process ends.  A step whose mzattn_decode_workspace_size() exceeds that
 * size is rejected with MZ_ERR_WORKSPACE before anything is launched.  The
 * call allocates and frees nothing.  Every call on one GPU uses that GPU's
 * array (its contents need no initialisation; each call writes what it
 * reads), so calls on one GPU that overlap in time (other streams, other
 * threads) race and must be serialised by the caller. */
#define MZATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
int mzattn_decode_noalloc(const mzattn_decode_args* args, void* stream);

/* ---- mzattn_decode_append ---------------------------------------------- */
/*
 * One generation step that appends its own keys and values to the static
 * cache and takes the filled length from device memory, so the step needs
 * no host value that changes from step to step and can be recorded once in
 * a HIP graph and replayed (VoxCPM page, "Memory and speed": each patch
 * waits on the device for the language models' positions, copied from
 * Python integers, and under CUDA graphs the attention spans the whole
 * cache; "What matches upstream", attention bullet: the step attends to a
 * static cache under an explicit boolean mask, zero and masked past the
 * current length).
 *
 * Row b holds len[b] filled cache rows (device int32, batch stride
 * len_stride_b, 0 = one length for every row).  Its q_len new tokens take
 * cache rows and positions len[b] + t, t = 0 .. q_len-1:
 *   - with rope_base > 0, q and k_new are rotated at that position (pairs
 *     chosen by rope_style, as in mzattn_fwd_args; every head);
 *   - the (rotated) k_new and v_new rows are written into k_cache and
 *     v_cache at that row;
 *   - query t attends to keys j <= len[b] + t (the filled rows and the new
 *     tokens up to itself), further restricted to mask[b, h, t, j] != 0
 *     when mask is not NULL (same layout as mzattn_decode's mask).
 * Keys past len[b] + q_len are never read.  A row with len[b] < 0 or
 * len[b] + q_len > cache_len writes nothing into the caches, gets an
 * all-zero output, and sets *overflow = 1 when overflow is not NULL (the
 * library never clears it).  The result is the one mzattn_decode gives on
 * the updated cache with that mask, and it has the same independence of
 * the key count beyond the last live key.
 *
 * Layouts: q and o [batch, heads_q, q_len, head_dim]; k_new, v_new
 * [batch, heads_kv, q_len, head_dim]; caches [batch, heads_kv, cache_len,
 * head_dim]; element strides, d contiguous.  dtype: MZ_BF16 or MZ_F16
 * (MZ_F32: MZ_ERR_UNSUPPORTED).  Other limits as for mzattn_decode.  The
 * launch depends on cache_len only (one work-group per 128-key chunk of
 * the whole cache; chunks past len[b] + q_len exit at once).
 *
 * workspace: mzattn_decode_append_workspace_size() bytes, 256-byte
 * aligned, no initialisation; calls sharing one must not overlap in time.
 */
typedef struct mzattn_decode_append_args {
  uint32_t struct_size; /* = sizeof(mzattn_decode_append_args), else MZ_ERR_ABI */
  int32_t dtype;
  int32_t batch, heads_q, heads_kv, q_len, head_dim, cache_len;
  float scale;
  int32_t rope_style;   /* 0 interleaved, 1 half split */
  double rope_base;     /* 0: no rotation */
  int32_t rope_precision;     /* 0 exact, 1 fp16 angles, 2 bf16 table */
  float rope_mscale;          /* cos / sin scale; 0 = 1 */
  const float* rope_factors;  /* optional device [head_dim/2], NULL = 1 */
  const void* q;
  int64_t q_stride[3];
  const void* k_new;
  int64_t k_new_stride[3];
  const void* v_new;
  int64_t v_new_stride[3];
  void* k_cache;        /* rows len[b] .. len[b] + q_len - 1 are written */
  int64_t k_stride[3];
  void* v_cache;
  int64_t v_stride[3];
  const int32_t* len;   /* device [batch] (or one value, len_stride_b = 0) */
  int64_t len_stride_b;
  void* o;
  int64_t o_stride[3];
  const uint8_t* mask;  /* optional, [B|1, Hq|1, q_len|1, cache_len] bool */
  int64_t mask_stride[4];
  int32_t* overflow;    /* optional device int, set to 1 on overflow */
  void* workspace;
  size_t workspace_bytes;
} mzattn_decode_append_args;

int mzattn_decode_append(const mzattn_decode_append_args* args, void* stream);
int mzattn_decode_append_workspace_size(const mzattn_decode_append_args* args, size_t* bytes);
int mzattn_validate_decode_append(const mzattn_decode_append_args* args);

/* ---- misc -------------------------------------------------------------- */
/* Static description of a status code. */
const char* mzattn_strerror(int status);
/* Detail of the last error raised on the calling thread ("" if none). */
const char* mzattn_last_error(void);
/* MZATTN_VERSION of the built library. */
int mzattn_version(void);
/* What the HIP runtime reports for `device`, for labelling measurements:
 * compute units, peak engine and memory clocks in kHz, and the gfx target
 * name (with its feature flags) copied into `arch` (at most arch_len bytes,
 * NUL-terminated).  Any output pointer may be NULL.  Returns MZ_OK, or
 * MZ_ERR_HIP when the runtime query fails (no such device). */
int mzattn_device_info(int device, int* compute_units, int* clock_khz, int* mem_clock_khz, char* arch, int arch_len);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* MZATTN_H_ */
