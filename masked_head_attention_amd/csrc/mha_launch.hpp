// mha_launch.hpp -- host-side launch of one kernel instantiation per
// (dtype, D, additive, pre-LN). Included by one translation unit per dtype.
#pragma once

#include "mha_kernel_f32.hpp"
#include "mha_kernel_half.hpp"

namespace mha {

// Query rows per workgroup, and the rows x keys tile of the skip decision.
//   16-bit types: 128 rows (4 waves x 32), tiles of 32 rows x 64 keys;
//   float32: 16 rows (NK key-split waves), tiles of 16 rows x 16 keys.
template <typename T, int D>
constexpr int block_rows() { return sizeof(T) == 2 ? 128 : F32Cfg<D>::BM; }
template <typename T, int D>
constexpr int skip_rows() { return sizeof(T) == 2 ? 32 : F32Cfg<D>::BM; }
template <typename T, int D>
constexpr int skip_keys() { return sizeof(T) == 2 ? 64 : F32Cfg<D>::SUB; }

// 16-bit types: 8 waves with two key splits under a causal mask, else 4
template <typename T, int D, int AM, bool PRE, bool KV16 = false>
hipError_t launch_half(const Params& p, long long grid, hipStream_t stream,
                       KvPre kp = KvPre{nullptr, 0, 0, nullptr}) {
  if (p.kind & K_CAUSAL)
    hipLaunchKernelGGL((mha_half_kernel<T, D, AM, PRE, 2, KV16>), dim3((unsigned)grid), dim3(512),
                       0, stream, p, kp);
  else
    hipLaunchKernelGGL((mha_half_kernel<T, D, AM, PRE, 1, KV16>), dim3((unsigned)grid), dim3(256),
                       0, stream, p, kp);
  return hipGetLastError();
}

// Workgroups per head of the float16 copy kernel.
constexpr int kKvCopySub = 4;

// bfloat16 pre-LN without a mask tensor, with a workspace: the copy kernel
// (float16 K and V, and every token's LayerNorm statistics), then the
// attention kernel on the copies (the heads whose flags are clear), then on
// the bfloat16 tensors (the heads with a flag set). k16, v16: [B,H,Lk,D]
// float16; flags: [B*H*kKvCopySub] int32; stats: [B*Lq] float2.
template <int D>
hipError_t launch_prenorm_kv16(Params p, void* k16, void* v16, int* flags, float2* stats,
                               hipStream_t stream) {
  p.nqblk = (p.Lq + block_rows<__bf16, D>() - 1) / block_rows<__bf16, D>();
  p.hg = p.H % 4 == 0 ? 4 : (p.H % 2 == 0 ? 2 : 1);
  const long long grid = (long long)p.B * (p.H / p.hg) * p.nqblk;
  const long long ncopy = (long long)p.B * p.H * kKvCopySub;
  const long long ntok = (long long)p.B * p.Lq;
  const long long nstat = std::min((ntok + 15) / 16, 2048LL);  // 16 tokens per workgroup pass
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL || ncopy + nstat > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const KvConvParams c{p.k, p.v, k16, v16, flags, (int64_t)p.Lk * D / 8, kKvCopySub, (int)nstat,
                       p.x, stats, (int64_t)ntok, p.H * D, p.eps};
  hipLaunchKernelGGL(mha_half_kernel_kv16_copy<__bf16>, dim3((unsigned)(ncopy + nstat)), dim3(256),
                     0, stream, c);
  Params pc = p;
  pc.k = k16;
  pc.v = v16;
  hipError_t e = launch_half<__bf16, D, 0, true, true>(pc, grid, stream,
                                                       KvPre{flags, kKvCopySub, 1, stats});
  if (e != hipSuccess) return e;
  return launch_half<__bf16, D, 0, true, false>(p, grid, stream,
                                                KvPre{flags, kKvCopySub, 2, nullptr});
}

template <typename T, int D, bool ADD, bool PRE>
hipError_t launch_one(Params p, hipStream_t stream) {
  p.nqblk = (p.Lq + block_rows<T, D>() - 1) / block_rows<T, D>();
  // pre-LN, 16-bit types: one workgroup serves a group of heads of the same
  // query block, so the token statistics are computed once for the group
  p.hg = (sizeof(T) == 2 && PRE) ? (p.H % 4 == 0 ? 4 : (p.H % 2 == 0 ? 2 : 1)) : 1;
  const long long grid = (long long)p.B * (p.H / p.hg) * p.nqblk;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if constexpr (sizeof(T) == 2) {
    if constexpr (ADD) {
      if (p.add_vec) return launch_half<T, D, 1, PRE>(p, grid, stream);
      return launch_half<T, D, 2, PRE>(p, grid, stream);
    } else {
      return launch_half<T, D, 0, PRE>(p, grid, stream);
    }
  } else {
    hipLaunchKernelGGL((mha_f32_kernel<D, ADD, PRE>), dim3((unsigned)grid),
                       dim3(64 * F32Cfg<D>::NK), 0, stream, p);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const Params& p, bool add, bool pre, hipStream_t s) {
  if (add) return pre ? launch_one<T, D, true, true>(p, s) : launch_one<T, D, true, false>(p, s);
  return pre ? launch_one<T, D, false, true>(p, s) : launch_one<T, D, false, false>(p, s);
}

template <typename T>
hipError_t launch_dtype(const Params& p, int D, bool add, bool pre, hipStream_t s) {
  switch (D) {
    case 16: return launch_d<T, 16>(p, add, pre, s);
    case 32: return launch_d<T, 32>(p, add, pre, s);
    case 64: return launch_d<T, 64>(p, add, pre, s);
    case 128: return launch_d<T, 128>(p, add, pre, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
void tile_shape(int D, int* rows_per_block, int* tile_rows, int* tile_keys) {
  switch (D) {
#define MHA_TILE_CASE(DD)                                     \
  case DD:                                                    \
    *rows_per_block = block_rows<T, DD>();                    \
    *tile_rows = skip_rows<T, DD>();                          \
    *tile_keys = skip_keys<T, DD>();                          \
    return;
    MHA_TILE_CASE(16)
    MHA_TILE_CASE(32)
    MHA_TILE_CASE(64)
    MHA_TILE_CASE(128)
#undef MHA_TILE_CASE
    default: *rows_per_block = *tile_rows = *tile_keys = 0;
  }
}

// Entry points defined per dtype.
hipError_t launch_f32(const Params& p, int D, bool add, bool pre, hipStream_t s);
hipError_t launch_f16(const Params& p, int D, bool add, bool pre, hipStream_t s);
hipError_t launch_bf16(const Params& p, int D, bool add, bool pre, hipStream_t s);
void tile_shape_f32(int D, int* bm, int* rows, int* keys);
void tile_shape_f16(int D, int* bm, int* rows, int* keys);
void tile_shape_bf16(int D, int* bm, int* rows, int* keys);
hipError_t launch_bf16_prenorm_kv16(const Params& p, int D, void* k16, void* v16, int* flags,
                                    float2* stats, hipStream_t s);

}  // namespace mha
