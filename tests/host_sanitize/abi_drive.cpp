// Drives the C ABI's host code (argument checks, workspace sizes, parameter
// fills) with valid calls and with seeded random mutations of every field,
// built with AddressSanitizer and UndefinedBehaviorSanitizer: any
// out-of-bounds access, signed overflow or bad shift in the host code
// aborts the run.  Device pointers are fake (never dereferenced: the
// launchers are stubs).  Exit 0 = every call returned a status in range.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mzattn.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint64_t next() {  // xorshift64
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return rng;
}
static const int64_t kEdge[] = {0, 1, -1, 2, 7, 8, 63, 64, 65, 127, 128, 129, 4096, 8192, 65535, 65536,
                                (1 << 20), (1 << 20) + 1, (1 << 24), INT_MAX, INT_MIN, (int64_t)1 << 40,
                                INT64_MAX, INT64_MIN};
static int64_t edge() { return kEdge[next() % (sizeof(kEdge) / sizeof(kEdge[0]))]; }
static void* fake(uint64_t off) { return (void*)(uintptr_t)(0x100000000000ull + off); }

static int checked = 0;
static int check_status(int st) {
  ++checked;
  if (st > 0 || st < -10) {
    fprintf(stderr, "status %d out of range\n", st);
    return 1;
  }
  (void)mzattn_strerror(st);
  (void)strlen(mzattn_last_error());
  return 0;
}

static mzattn_fwd_args good_fwd() {
  mzattn_fwd_args a;
  memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(a);
  a.dtype = MZ_BF16;
  a.batch = 2; a.heads_q = 16; a.heads_kv = 8; a.seq_q = 300; a.seq_k = 300; a.head_dim = 128;
  a.pe_attn_head = -1; a.mask_kind = MZ_MASK_BOOL; a.rope_base = 1e6;
  a.q = fake(0); a.k = fake(1 << 26); a.v = fake(2 << 26); a.o = fake(3 << 26);
  const int64_t qs[3] = {16 * 300 * 128, 300 * 128, 128}, ks[3] = {8 * 300 * 128, 300 * 128, 128};
  for (int i = 0; i < 3; ++i) { a.q_stride[i] = a.o_stride[i] = qs[i]; a.k_stride[i] = a.v_stride[i] = ks[i]; }
  a.mask = (const uint8_t*)fake(4 << 26);
  a.mask_stride[0] = 300 * 300; a.mask_stride[1] = 0; a.mask_stride[2] = 300; a.mask_stride[3] = 1;
  a.norm_eps = 1e-6f;
  return a;
}

static mzattn_decode_args good_dec() {
  mzattn_decode_args a;
  memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(a);
  a.dtype = MZ_BF16;
  a.batch = 2; a.heads_q = 16; a.heads_kv = 2; a.q_len = 1; a.head_dim = 128; a.cache_len = 8192; a.span = 8192;
  a.q = fake(0); a.k_cache = fake(1 << 26); a.v_cache = fake(2 << 26); a.o = fake(3 << 26);
  const int64_t qs[3] = {16 * 128, 128, 128}, ks[3] = {2 * 8192 * 128, 8192 * 128, 128};
  for (int i = 0; i < 3; ++i) { a.q_stride[i] = a.o_stride[i] = qs[i]; a.k_stride[i] = a.v_stride[i] = ks[i]; }
  a.mask = (const uint8_t*)fake(4 << 26);
  a.mask_stride[0] = 8192; a.mask_stride[3] = 1;
  return a;
}

static mzattn_decode_append_args good_app() {
  mzattn_decode_append_args a;
  memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(a);
  a.dtype = MZ_BF16;
  a.batch = 2; a.heads_q = 16; a.heads_kv = 2; a.q_len = 1; a.head_dim = 128; a.cache_len = 8192;
  a.rope_base = 1e4;
  a.q = fake(0); a.k_new = fake(5 << 26); a.v_new = fake(6 << 26);
  a.k_cache = fake(1 << 26); a.v_cache = fake(2 << 26); a.o = fake(3 << 26);
  a.len = (const int32_t*)fake(7 << 26);
  const int64_t qs[3] = {16 * 128, 128, 128}, ns[3] = {2 * 128, 128, 128}, ks[3] = {2 * 8192 * 128, 8192 * 128, 128};
  for (int i = 0; i < 3; ++i) {
    a.q_stride[i] = a.o_stride[i] = qs[i]; a.k_new_stride[i] = a.v_new_stride[i] = ns[i];
    a.k_stride[i] = a.v_stride[i] = ks[i];
  }
  return a;
}

// Overwrite one random 4- or 8-byte aligned field of the struct (past
// struct_size) with an edge value, or a random pointer-sized value.
template <typename A>
static void mutate(A& a) {
  unsigned char* bytes = reinterpret_cast<unsigned char*>(&a);
  const size_t n8 = sizeof(A) / 8;
  const size_t at = 1 + next() % (n8 - 1);  // 8-byte slot (slot 0 holds struct_size)
  const int64_t v = (next() & 3) == 0 ? (int64_t)next() : edge();
  if (next() & 1) {
    memcpy(bytes + at * 8, &v, 8);
  } else {
    const int32_t v32 = (int32_t)v;
    memcpy(bytes + at * 8 + ((next() & 1) ? 4 : 0), &v32, 4);
  }
}

int main() {
  int bad = 0;
  size_t bytes = 0;
  void* ws = fake(8ull << 26);
  for (int it = 0; it < 20000; ++it) {
    {
      mzattn_fwd_args a = good_fwd();
      const int kinds = (int)(next() % 4);
      a.mask_kind = kinds;
      if (kinds == MZ_MASK_SEGMENT) { a.seg_q = a.seg_k = (const int32_t*)fake(9ull << 26); a.seg_q_stride_b = 300; a.seg_k_stride_b = 300; }
      for (int m = 0; m < (int)(next() % 4); ++m) mutate(a);
      a.struct_size = sizeof(a);
      bad |= check_status(mzattn_fwd_workspace_size(&a, &bytes));
      a.workspace = ws; a.workspace_bytes = bytes;
      bad |= check_status(mzattn_validate_fwd(&a));
      bad |= check_status(mzattn_fwd(&a, nullptr));
      bad |= check_status(mzattn_fwd_plan(&a, nullptr));
      bad |= check_status(mzattn_fwd_execute(&a, nullptr));
    }
    {
      mzattn_decode_args a = good_dec();
      for (int m = 0; m < (int)(next() % 4); ++m) mutate(a);
      a.struct_size = sizeof(a);
      bad |= check_status(mzattn_decode_workspace_size(&a, &bytes));
      a.workspace = ws; a.workspace_bytes = bytes;
      bad |= check_status(mzattn_validate_decode(&a));
      bad |= check_status(mzattn_decode(&a, nullptr));
    }
    {
      mzattn_decode_append_args a = good_app();
      for (int m = 0; m < (int)(next() % 4); ++m) mutate(a);
      a.struct_size = sizeof(a);
      bad |= check_status(mzattn_decode_append_workspace_size(&a, &bytes));
      a.workspace = ws; a.workspace_bytes = bytes;
      bad |= check_status(mzattn_validate_decode_append(&a));
      bad |= check_status(mzattn_decode_append(&a, nullptr));
    }
  }
  // null and ABI-mismatch arguments
  bad |= check_status(mzattn_validate_fwd(nullptr));
  bad |= check_status(mzattn_fwd_workspace_size(nullptr, &bytes));
  bad |= check_status(mzattn_validate_decode(nullptr));
  bad |= check_status(mzattn_decode_noalloc(nullptr, nullptr));
  mzattn_fwd_args f = good_fwd();
  f.struct_size = 1;
  bad |= check_status(mzattn_validate_fwd(&f));
  for (int s = -20; s <= 5; ++s) (void)mzattn_strerror(s);
  {
    // with no device the query fails cleanly, whatever the outputs
    char arch[4];
    int cu = -1;
    bad |= check_status(mzattn_device_info(0, &cu, nullptr, nullptr, arch, (int)sizeof(arch)));
    bad |= check_status(mzattn_device_info(-1, nullptr, nullptr, nullptr, nullptr, 0));
    if (mzattn_device_info(0, &cu, nullptr, nullptr, arch, (int)sizeof(arch)) != MZ_ERR_HIP || cu != -1) bad = 1;
  }
  printf("%d calls checked, version %d\n", checked, mzattn_version());
  return bad;
}
