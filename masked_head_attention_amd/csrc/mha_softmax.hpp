// mha_softmax.hpp -- row softmax over a materialised score tensor for gfx950
// (CDNA4): float32, float16, bfloat16.
//
// Source (web page, cited by title and section):
//   [MAX] "Why attention must compute the max first" (gsyq.cn/news/340375):
//         the row-softmax workload (2.1), the online max/sum update (2.3) and
//         the fused one-pass kernel (4.2).
//
// Each row is p_j = exp(c*s_j - max) / sum exp(c*s - max). The work is bound
// by HBM: one read and one write of the tensor. One wave owns a row.
//   * rows that are 16-byte aligned and at most 64 * NV vectors long stay in
//     registers: each lane loads its 16-byte vectors once, the row maximum and
//     the sum of exponentials are wave reductions, and the weights are
//     written once [MAX 4.2];
//   * any other row takes two passes: an online maximum and rescaled sum per
//     lane [MAX 2.3], merged across the wave, then a normalising pass.
// An entry equal to -inf is a masked position (weight 0 whatever the scale);
// a row with every entry masked is written as zeros and raises
// F_FULLY_MASKED_ROW; a NaN score makes the row's unmasked weights NaN, and
// any non-finite weight raises F_NONFINITE.
#pragma once

#include "mha_common.hpp"

namespace mha {

struct SoftmaxParams {
  const void* s;
  void* p;
  int64_t rows;
  int cols;
  float c;  // scale * log2(e)
  uint32_t* flags;
};

__device__ inline float wave_max64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ inline float wave_sum64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <typename T>
__device__ inline float load_elem(const char* row, int j) {
  if constexpr (sizeof(T) == 4) return reinterpret_cast<const float*>(row)[j];
  else if constexpr (std::is_same<T, _Float16>::value)
    return (float)reinterpret_cast<const _Float16*>(row)[j];
  else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[j] << 16);
}
// Stores v rounded to T (nearest even) and returns the stored value.
template <typename T>
__device__ inline float store_elem(char* row, int j, float v) {
  if constexpr (sizeof(T) == 4) {
    reinterpret_cast<float*>(row)[j] = v;
    return v;
  } else {
    const T h = (T)v;
    reinterpret_cast<T*>(row)[j] = h;
    return (float)h;
  }
}

// The elements of one 16-byte vector as floats.
template <typename T>
__device__ inline void vec_to_f32(const uint4 u, float (&x)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 4) {
    x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
  } else {
    T* tag = nullptr;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = lo_f(w[i], tag);
      x[2 * i + 1] = hi_f(w[i], tag);
    }
  }
}
template <typename T>
__device__ inline uint4 f32_to_vec(const float (&x)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 4) {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                      __float_as_uint(x[3]));
  } else {
    T* tag = nullptr;
    return make_uint4(pack2(x[0], x[1], tag), pack2(x[2], x[3], tag), pack2(x[4], x[5], tag),
                      pack2(x[6], x[7], tag));
  }
}

// Register path: a 16-byte aligned row of at most 64 * NV vectors.
template <typename T, int NV>
__global__ __launch_bounds__(256) void softmax_rows_vec(const SoftmaxParams p) {
  constexpr int EPV = 16 / sizeof(T);  // elements per vector
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= p.rows) return;  // whole waves only
  const int nvec = p.cols / EPV;
  const char* src = static_cast<const char*>(p.s) + r * (int64_t)p.cols * sizeof(T);
  char* dst = static_cast<char*>(p.p) + r * (int64_t)p.cols * sizeof(T);

  static_assert(NV * EPV <= 64, "one mask bit per element held by a lane");
  float x[NV][EPV];
  uint64_t masked = 0;  // bit k*EPV + e: that element is -inf (or past the row)
  float m = -INFINITY;
  bool nan = false;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int j = lane + 64 * k;
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    // each score is read once: non-temporal loads (cache-policy bit `nt`)
    if (j < nvec)
      u = __builtin_bit_cast(
          uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + 16 * (int64_t)j)));
    vec_to_f32<T>(u, x[k]);
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      if (j >= nvec) x[k][e] = -INFINITY;  // past the row: masked
      if (x[k][e] == -INFINITY) masked |= 1ull << (k * EPV + e);
      m = fmaxf(m, x[k][e]);
      nan |= x[k][e] != x[k][e];
    }
  }
  m = wave_max64(m);
  const bool any_nan = __ballot(nan) != 0;
  if (m == -INFINITY && !any_nan) {  // every entry masked
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int j = lane + 64 * k;
      if (j < nvec) *reinterpret_cast<uint4*>(dst + 16 * (int64_t)j) = make_uint4(0u, 0u, 0u, 0u);
    }
    if (lane == 0) atomicOr(p.flags, F_FULLY_MASKED_ROW);
    return;
  }
  const float mc = m * p.c;
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const float t = x[k][e];
      x[k][e] = (t == -INFINITY) ? 0.f : exp2_fast(__builtin_fmaf(t, p.c, -mc));
      sum += x[k][e];
    }
  sum = wave_sum64(sum);
  const float inv = any_nan ? __builtin_nanf("") : 1.0f / sum;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int j = lane + 64 * k;
    if (j >= nvec) continue;
    float y[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) y[e] = ((masked >> (k * EPV + e)) & 1) ? 0.f : x[k][e] * inv;
    const uint4 o = f32_to_vec<T>(y);
    float back[EPV];
    vec_to_f32<T>(o, back);
#pragma unroll
    for (int e = 0; e < EPV; ++e) bad |= !__builtin_isfinite(back[e]);
    *reinterpret_cast<uint4*>(dst + 16 * (int64_t)j) = o;
  }
  if (__ballot(bad) != 0 && lane == 0) atomicOr(p.flags, F_NONFINITE);
}

// General path: any length and alignment, element by element, two passes.
template <typename T>
__global__ __launch_bounds__(256) void softmax_rows_gen(const SoftmaxParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= p.rows) return;
  const char* src = static_cast<const char*>(p.s) + r * (int64_t)p.cols * sizeof(T);
  char* dst = static_cast<char*>(p.p) + r * (int64_t)p.cols * sizeof(T);
  // pass 1: online maximum and rescaled sum per lane [MAX 2.3], log2 units
  float m = -INFINITY, l = 0.f;
  bool nan = false;
  for (int j = lane; j < p.cols; j += 64) {
    const float t = load_elem<T>(src, j);
    if (t == -INFINITY) continue;
    nan |= t != t;
    const float u = t * p.c;
    if (u > m) {
      l = l * exp2_fast(m - u) + 1.f;  // exp2(-inf) = 0 on the first legal entry
      m = u;
    } else {
      l += exp2_fast(u - m);
    }
  }
  const float M = wave_max64(m);
  const bool any_nan = __ballot(nan) != 0;
  if (M == -INFINITY && !any_nan) {
    for (int j = lane; j < p.cols; j += 64) store_elem<T>(dst, j, 0.f);
    if (lane == 0) atomicOr(p.flags, F_FULLY_MASKED_ROW);
    return;
  }
  const float L = wave_sum64(m == -INFINITY ? 0.f : l * exp2_fast(m - M));
  const float inv = any_nan ? __builtin_nanf("") : 1.0f / L;
  // pass 2: weights
  bool bad = false;
  for (int j = lane; j < p.cols; j += 64) {
    const float t = load_elem<T>(src, j);
    const float y = (t == -INFINITY) ? 0.f : exp2_fast(t * p.c - M) * inv;
    bad |= !__builtin_isfinite(store_elem<T>(dst, j, y));
  }
  if (__ballot(bad) != 0 && lane == 0) atomicOr(p.flags, F_NONFINITE);
}

template <typename T>
hipError_t launch_softmax(const SoftmaxParams& p, bool vec_ok, hipStream_t stream) {
  constexpr int EPV = 16 / sizeof(T);
  const long long grid = (p.rows + 3) / 4;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int nvec = p.cols / EPV;
  if (vec_ok && nvec <= 64 * 4)
    hipLaunchKernelGGL((softmax_rows_vec<T, 4>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  else if (vec_ok && nvec <= 64 * 8)
    hipLaunchKernelGGL((softmax_rows_vec<T, 8>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((softmax_rows_gen<T>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mha
