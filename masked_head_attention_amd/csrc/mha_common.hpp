// mha_common.hpp -- definitions shared by the fused masked multi-head
// attention kernels for gfx950 (CDNA4): launch parameters, element
// conversions, 8-element MFMA operand fragments, lane maps and wave64
// exchange helpers.
//
// Sources (web pages, cited by title and section):
//   [MMHA]  "masked multi head attention" CUDA implementation notes (2kiu.com/news/6063113)
//   [MAX]   "Why attention must compute the max first" (gsyq.cn/news/340375)
//   [LNXA]  "How to fuse cross-attention and layer-norm into a single CUDA kernel?"
//           (cms365.cn question page)
#pragma once


#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mha {

enum : unsigned { K_CAUSAL = 1u, K_PADDING = 2u, K_ADDITIVE = 4u, K_KEEP = 8u, K_PER_HEAD = 16u };
enum : uint32_t { F_FULLY_MASKED_ROW = 1u, F_NONFINITE = 2u, F_BAD_LENGTH = 4u };

struct Params {
  const void* q;         // [B,H,Lq,D]
  const void* k;         // [B,H,Lk,D]
  const void* v;         // [B,H,Lk,D]
  const int32_t* lens;   // [B] (PADDING)
  const void* add;       // [B,1,Lq,Lk] (ADDITIVE)
  const void* x;         // [B,Lq,H*D] (pre-LN)
  const void* gamma;     // [H*D]
  const void* beta;      // [H*D]
  const void* residual;  // [B,Lq,H*D] or null
  void* out;             // [B,H,Lq,D] or [B,Lq,H*D] (pre-LN)
  int B, H, Lq, Lk;
  int nqblk;             // query blocks per (b, h)
  int hg;                // heads per workgroup (pre-LN kernel of 16-bit types)
  unsigned kind;         // K_* bits (a mask tensor -- ADDITIVE or KEEP -- is also a template switch)
  float c;               // scale * log2(e)
  float scale;           // scale
  float eps;
  int add_vec;           // additive-mask rows are 16-byte aligned
  uint32_t* flags;
  unsigned long long* counters;  // [3] or null
};

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte LDS read through a native vector type. The compiler keeps precise
// memory-operand information for it; a read of HIP's uint4 struct is treated
// as possibly overlapping every direct-to-LDS load still in flight, and gets
// an s_waitcnt vmcnt(0) in front of it.
__device__ inline uint4 lds_load16(const char* p) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Eight consecutive elements of type T, as raw 16-byte words.
template <typename T>
struct Frag8 {
  static constexpr int W = sizeof(T) / 2;  // uint4 words: 1 for half types, 2 for float
  uint4 u[W];
};

// ---- element conversions -------------------------------------------------
__device__ inline float lo_f(uint32_t w, _Float16*) {
  return (float)__builtin_bit_cast(f16x2, w)[0];
}
__device__ inline float hi_f(uint32_t w, _Float16*) {
  return (float)__builtin_bit_cast(f16x2, w)[1];
}
__device__ inline float lo_f(uint32_t w, __bf16*) { return __uint_as_float(w << 16); }
__device__ inline float hi_f(uint32_t w, __bf16*) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline uint32_t pack2(float a, float b, _Float16*) {
  f16x2 h = {(_Float16)a, (_Float16)b};  // v_cvt_pk_f16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}
__device__ inline uint32_t pack2(float a, float b, __bf16*) {
  bf16x2 h = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

template <typename T>
__device__ inline void unpack8(const Frag8<T>& f, float (&x)[8]) {
  if constexpr (sizeof(T) == 4) {
    x[0] = __uint_as_float(f.u[0].x); x[1] = __uint_as_float(f.u[0].y);
    x[2] = __uint_as_float(f.u[0].z); x[3] = __uint_as_float(f.u[0].w);
    x[4] = __uint_as_float(f.u[1].x); x[5] = __uint_as_float(f.u[1].y);
    x[6] = __uint_as_float(f.u[1].z); x[7] = __uint_as_float(f.u[1].w);
  } else {
    T* tag = nullptr;
    const uint32_t w[4] = {f.u[0].x, f.u[0].y, f.u[0].z, f.u[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = lo_f(w[i], tag);
      x[2 * i + 1] = hi_f(w[i], tag);
    }
  }
}

template <typename T>
__device__ inline Frag8<T> pack8(const float* x) {
  Frag8<T> f;
  if constexpr (sizeof(T) == 4) {
    f.u[0] = make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                        __float_as_uint(x[3]));
    f.u[1] = make_uint4(__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]),
                        __float_as_uint(x[7]));
  } else {
    T* tag = nullptr;
    f.u[0] = make_uint4(pack2(x[0], x[1], tag), pack2(x[2], x[3], tag), pack2(x[4], x[5], tag),
                        pack2(x[6], x[7], tag));
  }
  return f;
}

// ---- MFMA over an 8-element k-slice per lane -------------------------------
// A lane in half hh (lanes 32*hh .. 32*hh+31) supplies the 8 k-slots of its
// half; both operands use the same slot <-> index assignment, so any
// permutation of the contraction index inside a slice is harmless.
__device__ inline f32x16 mma8(const Frag8<_Float16>& a, const Frag8<_Float16>& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a.u[0]),
                                                __builtin_bit_cast(f16x8, b.u[0]), c, 0, 0, 0);
}
__device__ inline f32x16 mma8(const Frag8<__bf16>& a, const Frag8<__bf16>& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.u[0]),
                                                 __builtin_bit_cast(bf16x8, b.u[0]), c, 0, 0, 0);
}

// ---- lane maps -------------------------------------------------------------
// Accumulator register i of a 32x32 MFMA holds row 8*(i/4) + 4*hh + i%4.
// keymap sends that row to 8*hh + i (i < 8) or 16 + 8*hh + (i - 8) (i >= 8).
__device__ inline int keymap(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// Exchange with the lane 32 apart; returns {value of lane l, value of lane l^32}
// in an order that makes max/sum of the pair symmetric across the halves.
__device__ inline float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// A keep-mask word (two 16-bit values: 0 masks the key, anything else keeps
// it) rewritten as the additive form: a half equal to +-0 becomes `neg` (the
// type's -inf pattern), any other half +0. Packed 16-bit integer arithmetic:
// |x| - 1 wraps to 0xffff only for x = +-0.
__device__ inline uint32_t keep_to_additive(uint32_t w, uint16_t neg) {
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  const u16x2 mag = __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
  const u16x2 one = {1, 1}, n2 = {neg, neg};
  const u16x2 zero = (u16x2)(mag - one) >> (u16x2){15, 15};
  return __builtin_bit_cast(uint32_t, (u16x2)(zero * n2));
}
__device__ inline uint4 keep_to_additive(uint4 u, uint16_t neg) {
  return make_uint4(keep_to_additive(u.x, neg), keep_to_additive(u.y, neg),
                    keep_to_additive(u.z, neg), keep_to_additive(u.w, neg));
}

// s_waitcnt immediate that waits until at most n vector-memory loads of this
// wave are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt at their "no wait" maxima). Loads complete in issue order.
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | 0x0F70; }

template <typename T>
__device__ inline Frag8<T> ld_global8(const char* p) {
  Frag8<T> f;
#pragma unroll
  for (int w = 0; w < Frag8<T>::W; ++w) f.u[w] = *reinterpret_cast<const uint4*>(p + 16 * w);
  return f;
}
template <typename T>
__device__ inline Frag8<T> zero8() {
  Frag8<T> f;
#pragma unroll
  for (int w = 0; w < Frag8<T>::W; ++w) f.u[w] = make_uint4(0u, 0u, 0u, 0u);
  return f;
}

// LDS address space pointer, for the builtins that take one.
#define MHA_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Raw buffer over [base, base + bytes): loads beyond it return zeros.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

}  // namespace mha
