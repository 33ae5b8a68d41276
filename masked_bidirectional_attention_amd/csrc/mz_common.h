// Device-side helpers shared by the mzattn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "mz_internal.h"

namespace mz {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

#define MZ_LDS __attribute__((address_space(3)))

// Storage tags: the kernels move raw 16-bit patterns and convert explicitly.
struct BF16 {};
struct F16 {};

template <typename T> struct Elem;
template <> struct Elem<BF16> {
  __device__ static inline float to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  }
  // round to nearest even (hardware conversion on gfx950)
  __device__ static inline uint16_t from_f32(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
  }
  // two values, round to nearest even, one v_cvt_pk_bf16_f32
  __device__ static inline uint32_t pack2(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  }
  // acc + both halves of a packed pair (one v_dot2 with (1, 1))
  __device__ static inline float add_pair(uint32_t x, float acc) {
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x), one, acc, false);
  }
};
template <> struct Elem<F16> {
  __device__ static inline float to_f32(uint16_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
  }
  __device__ static inline uint16_t from_f32(float x) {
    _Float16 h = static_cast<_Float16>(x);
    return __builtin_bit_cast(uint16_t, h);
  }
  // two values, round to nearest even, one v_cvt_pk_f16_f32
  __device__ static inline uint32_t pack2(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  }
  // acc + both halves of a packed pair (one v_dot2 with (1, 1))
  __device__ static inline float add_pair(uint32_t x, float acc) {
    const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, x), one, acc, false);
  }
};

// ---- MFMA wrappers (operands as raw 16-byte register quads) --------------
// 32x32x16: A lane l holds A[l%32][(l/32)*8 + e]; B lane l holds
// B[(l/32)*8 + e][l%32]; C lane l register v holds
// C[(v/4)*8 + (l/32)*4 + v%4][l%32].
template <typename T> __device__ inline f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c);
template <> __device__ inline f32x16_t mfma32<BF16>(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
template <> __device__ inline f32x16_t mfma32<F16>(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
// 16x16x32: A lane l holds A[l%16][(l/16)*8 + e]; B lane l holds
// B[(l/16)*8 + e][l%16]; C lane l register v holds C[(l/16)*4 + v][l%16].
template <typename T> __device__ inline f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c);
template <> __device__ inline f32x4_t mfma16<BF16>(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
template <> __device__ inline f32x4_t mfma16<F16>(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// ---- LDS transpose read (ds_read_b64_tr_b16) -------------------------------
// Within each 16-lane group, lane (r = (i/4), c = i%4) supplies the address of
// 4 consecutive 16-bit elements of "row r"; lane i of the group receives
// element i%4 of the chunk supplied by lane (r, i/4) for r = 0..3, i.e.
// column i of the 4 x 16 block formed by the group's rows.
template <typename T> __device__ inline uint2 lds_read_tr(const uint16_t* p);
template <> __device__ inline uint2 lds_read_tr<BF16>(const uint16_t* p) {
  bf16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MZ_LDS bf16x4_t*)(p));
  return __builtin_bit_cast(uint2, r);
}
typedef __fp16 fp16x4_vs_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
template <> __device__ inline uint2 lds_read_tr<F16>(const uint16_t* p) {
  fp16x4_vs_t r = __builtin_amdgcn_ds_read_tr16_b64_v4f16((MZ_LDS fp16x4_vs_t*)(p));
  return __builtin_bit_cast(uint2, r);
}

// 16-byte global -> LDS copy without a register round trip: lane i of the
// wave writes its 16 bytes to lds_base + 16 * i (lds_base is wave-uniform).
__device__ inline void lds_dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}

// 16-byte global -> LDS copy: lane i reads bytes [voff_i, voff_i + 16) past
// the wave-uniform base and writes them to LDS byte address lds_addr + 16*i
// (lds_addr is wave-uniform; it goes to M0, and the s_nop gives the M0
// write the wait state the LDS-DMA path needs).  Issued as opaque assembly
// on purpose: the compiler then cannot see the LDS write and does not make
// the following LDS reads of the other pipeline stage wait for it; the
// caller waits with "s_waitcnt vmcnt(0)" and a barrier before reading the
// stage it fills.
__device__ inline void lds_dma16_s(const void* base, uint32_t voff, uint32_t lds_addr) {
  // the base is wave-uniform by contract; make it scalar explicitly
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t bs = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(bs),
                   "{m0}"((uint32_t)__builtin_amdgcn_readfirstlane(lds_addr))
                   : "memory");
}
// Raw buffer descriptor (stride 0, 32-bit data format) over nbytes bytes
// from a wave-uniform base, in scalar registers: a load whose bytes lie past
// nbytes returns zeros instead.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline u32x4_t buf_desc(const void* base, uint32_t nbytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  u32x4_t d;
  d.x = __builtin_amdgcn_readfirstlane((uint32_t)b);
  d.y = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xFFFFu;
  d.z = __builtin_amdgcn_readfirstlane(nbytes);
  d.w = 0x00020000u;
  return d;
}
// The same copy through a buffer descriptor (range-checked, see buf_desc).
__device__ inline void lds_dma16_b(u32x4_t desc, uint32_t voff, uint32_t lds_addr) {
  __asm__ volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(desc),
                   "{m0}"((uint32_t)__builtin_amdgcn_readfirstlane(lds_addr))
                   : "memory");
}

// LDS byte address of a pointer into shared memory
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const MZ_LDS void*)p;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float wave_xor_max(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask, 64));
}

// Combine a value with the one held by lane l ^ 32 without going through
// LDS: v_permlane32_swap exchanges the two 32-lane halves of a pair of
// registers, so each lane ends up holding its own value and its partner's.
__device__ inline float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- rotary embedding angles -----------------------------------------------
// theta_i = base^(-2i/D) / factor_i in fp64 (factor_i = 1 without LongRoPE
// factors).  Exact (precision 0): the angle pos * theta_i is formed in fp64
// and reduced to [-pi, pi] by subtracting the nearest multiple of 2 pi (2 pi
// split in two doubles, Cody-Waite), then its sine and cosine are taken in
// fp32 (accurate to about one fp32 ulp on the reduced range) and multiplied
// by mscale.  fp16 angles (1): theta_i and pos rounded to fp16, their
// product (exact in fp32) rounded to fp16, cos and sin of it (fp64)
// rounded to fp16, times mscale.  bf16 table (2): the angle pos *
// fp32(theta_i) rounded to fp32, cos and sin (fp64) rounded to fp32, times
// mscale, rounded to bf16.  The table
// holds positions [0, tab_len); other positions take the same formula
// directly, so both routes give identical bits.
__device__ inline double rope_theta(int i, int D, const RopeSpec& r) {
  const double th = exp2(-(double)(2 * i) / (double)D * r.log2_base);
  return r.factors != nullptr ? th / (double)r.factors[i] : th;
}
__device__ inline float2 rope_cs_theta(int pos, double theta, const RopeSpec& r) {
  float s, c;
  // (the rounding of cos / sin to fp16 or bf16 is taken from their fp64
  // values, so it does not depend on the fp32 routine's last bit)
  if (r.precision == 1) {
    const float th16 = (float)(_Float16)theta;
    const float p16 = (float)(_Float16)(float)pos;
    const float a16 = (float)(_Float16)(p16 * th16);  // exact product, one rounding to fp16
    double sd, cd;
    sincos((double)a16, &sd, &cd);
    c = (float)(_Float16)cd;
    s = (float)(_Float16)sd;
    return make_float2(c * r.mscale, s * r.mscale);
  }
  if (r.precision == 2) {
    const float a32 = (float)pos * (float)theta;
    double sd, cd;
    sincos((double)a32, &sd, &cd);
    const __bf16 cb = (__bf16)((float)cd * r.mscale), sb = (__bf16)((float)sd * r.mscale);
    return make_float2((float)cb, (float)sb);
  }
  const double ang = (double)pos * theta;
  const double k = rint(ang * 0.15915494309189533577);  // 1 / (2 pi)
  double rr = fma(-k, 6.28318530717958623200, ang);    // 2 pi, high part
  rr = fma(-k, 2.44929359829470635445e-16, rr);         // 2 pi, low part
  sincosf((float)rr, &s, &c);
  return make_float2(c * r.mscale, s * r.mscale);
}
__device__ inline float2 rope_cs_direct(int pos, int i, int D, const RopeSpec& r) {
  return rope_cs_theta(pos, rope_theta(i, D, r), r);
}

__device__ inline float2 rope_cs(const float2* tab, int tab_len, int pos, int i, int D, const RopeSpec& r) {
  if (pos >= 0 && pos < tab_len) return tab[(size_t)pos * (D / 2) + i];
  return rope_cs_direct(pos, i, D, r);
}

// Rotate the 8 consecutive elements held in a quad (d0 even) in fp32 and
// round back to the storage type.
template <typename T>
__device__ inline uint4 rope_quad(uint4 x, const float2* tab, int tab_len, int pos, int d0, int D,
                                  const RopeSpec& r) {
  uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float a = Elem<T>::to_f32((uint16_t)(w[t] & 0xFFFF));
    float b = Elem<T>::to_f32((uint16_t)(w[t] >> 16));
    float2 cs = rope_cs(tab, tab_len, pos, d0 / 2 + t, D, r);
    float ra = fmaf(a, cs.x, -b * cs.y);
    float rb = fmaf(b, cs.x, a * cs.y);
    w[t] = Elem<T>::pack2(ra, rb);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Map a hardware block id to a work item so that consecutive work items land
// on one XCD (blocks are dispatched round-robin over the 8 XCDs).
// Compile-time loop: f(std::integral_constant<int, 0>{}) ... up to N - 1,
// each body a separate straight-line copy (no reliance on the unroller).
template <typename F, int... Us>
__device__ __attribute__((always_inline)) inline void static_for_impl(F&& f, std::integer_sequence<int, Us...>) {
  (f(std::integral_constant<int, Us>{}), ...);
}
template <int N, typename F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ inline int xcd_remap(int bid, int n) {
  const int n8 = n - (n & 7);
  if (bid >= n8) return bid;
  return (bid & 7) * (n8 >> 3) + (bid >> 3);
}

}  // namespace mz
