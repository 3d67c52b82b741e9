// mha_api.hip -- the C ABI of libmha: argument validation, the per-device
// flag word, dispatch to a kernel instantiation, launch on the caller's stream.
//
// Validation is synchronous and completes before the first HIP call, so an
// invalid call enqueues nothing -- the launch-configuration check of
// [MMHA 4.3] ("masked multi head attention" CUDA notes, 2kiu.com/news/6063113),
// made a status code instead of a printf.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "mha.h"
#include "mha_launch.hpp"
#include "mha_bwd.hpp"
#include "mha_decode.hpp"
#include "mha_softmax.hpp"

namespace mha {
hipError_t launch_softmax_rows(const SoftmaxParams& p, int dtype, bool vec_ok, hipStream_t s);
void decode_plan(int B, int H, int Lk, int D, int esize, int* chunk, int* nsplit);
hipError_t launch_decode(const DecodeParams& p, int dtype, int D, hipStream_t s);
hipError_t launch_bwd(const BwdParams& p, int dtype, int D, hipStream_t s);
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint32_t* g_flags[kMaxDevices] = {};
std::atomic<unsigned long long*> g_counters{nullptr};

// Scratch of the allocation-free entry points: a file-scope device array, one
// copy per GPU, held for the life of the process. In host code its name is a
// host-side stand-in, never a device address: the device address of each
// GPU's copy is looked up once (mha_init, with that device current) and kept
// in g_scratch; kernels and copies only ever see that pointer.
static __device__ __align__(256) char scratch[MHA_NOALLOC_SCRATCH_BYTES];
void* g_scratch[kMaxDevices] = {};

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool mul_ok(int64_t a, int64_t b, int64_t* r) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *r = a * b;
  return true;
}

bool count_ok(std::initializer_list<int64_t> dims, int64_t esize) {
  int64_t r = esize;
  for (int64_t d : dims)
    if (!mul_ok(r, d, &r)) return false;
  return true;
}

int elem_size(mha_dtype t) { return t == MHA_F32 ? 4 : 2; }

// The current device's flag word, allocated (and zeroed) on first use.
mha_status device_flags(uint32_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MHA_E_NO_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_flags[dev]) {
    void* p = nullptr;
    if (hipMalloc(&p, 256) != hipSuccess) return MHA_E_NO_DEVICE;
    if (hipMemset(p, 0, 256) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
      (void)hipFree(p);
      return MHA_E_NO_DEVICE;
    }
    g_flags[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_flags[dev];
  return MHA_OK;
}

// Look up (once per device, with that device current) the device address of
// this device's copy of `scratch`. No allocation.
mha_status device_scratch_setup() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MHA_E_NO_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return MHA_E_NO_DEVICE;
    g_scratch[dev] = ptr;
  }
  return MHA_OK;
}

// The current device's flag word and scratch address, both set up earlier by
// mha_init; nothing is allocated or looked up here.
mha_status device_noalloc_state(uint32_t** flags, void** scr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MHA_E_NO_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_flags[dev] || !g_scratch[dev]) return MHA_E_NOT_INITIALIZED;
  *flags = g_flags[dev];
  *scr = g_scratch[dev];
  return MHA_OK;
}

struct Call {
  const void* q;
  const void* x;
  const void* k;
  const void* v;
  const void* mask;
  unsigned kind;
  const void* gamma;
  const void* beta;
  float eps;
  const void* residual;
  int B, H, Lq, Lk, D;
  float scale;
  mha_dtype dtype;
  void* stream;
  void* out;
  bool prenorm;
  bool with_ws = false;      // mha_prenorm_cross_fwd_ws
  void* ws = nullptr;
  size_t ws_bytes = 0;
};

// Workspace of mha_prenorm_cross_fwd_ws: float16 copies of K and V, the copy
// kernel's flags, then each token's LayerNorm statistics, each part 256-byte
// aligned. Zero where the call does not use one (every dtype but bfloat16,
// no queries or no keys).
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
struct PrenormWs {
  size_t kv, flags, stats, total;  // part sizes (aligned) and the sum
};
PrenormWs prenorm_ws(int B, int H, int Lq, int Lk, int D, mha_dtype dtype) {
  if (dtype != MHA_BF16 || B == 0 || H == 0 || Lq == 0 || Lk == 0) return PrenormWs{0, 0, 0, 0};
  PrenormWs w;
  w.kv = align256((size_t)B * H * Lk * D * 2);
  w.flags = align256((size_t)B * H * mha::kKvCopySub * 4);
  w.stats = align256((size_t)B * Lq * 8);
  w.total = 2 * w.kv + w.flags + w.stats;
  return w;
}

mha_status validate(const Call& c) {
  if (c.dtype != MHA_F32 && c.dtype != MHA_F16 && c.dtype != MHA_BF16) return MHA_E_DTYPE;
  if (c.kind & ~31u) return MHA_E_MASK;
  const unsigned tensor = c.kind & (MHA_MASK_ADDITIVE | MHA_MASK_KEEP);
  const unsigned pointer_kinds = c.kind & (MHA_MASK_PADDING | MHA_MASK_ADDITIVE | MHA_MASK_KEEP);
  if (pointer_kinds & (pointer_kinds - 1)) return MHA_E_MASK;  // one mask argument
  if ((c.kind & MHA_MASK_PER_HEAD) && !tensor) return MHA_E_MASK;
  const bool wants_mask = pointer_kinds != 0;
  if (!wants_mask && c.mask) return MHA_E_MASK;
  if (c.B < 0 || c.H < 0 || c.Lq < 0 || c.Lk < 0) return MHA_E_SHAPE;
  if (c.D != 16 && c.D != 32 && c.D != 64 && c.D != 128) return MHA_E_UNSUPPORTED;
  if (!std::isfinite(c.scale) || c.scale < 0.f) return MHA_E_ARG;
  if (c.prenorm) {
    if (!std::isfinite(c.eps) || c.eps < 0.f) return MHA_E_ARG;
    if ((int64_t)c.H * c.D > 65536) return MHA_E_SHAPE;
  }
  if (c.B == 0 || c.H == 0 || c.Lq == 0) return MHA_OK;  // empty call
  if (wants_mask && !c.mask) return MHA_E_NULL;
  if (!c.out || (c.prenorm ? !c.x : !c.q)) return MHA_E_NULL;
  if (c.Lk > 0 && (!c.k || !c.v)) return MHA_E_NULL;
  if (c.prenorm && (!c.gamma || !c.beta)) return MHA_E_NULL;
  const void* ptrs16[] = {c.q, c.x, c.k, c.v, c.out, c.gamma, c.beta, c.residual,
                          tensor ? c.mask : nullptr};
  for (const void* p : ptrs16)
    if (p && !aligned(p, 16)) return MHA_E_ALIGN;
  if ((c.kind & MHA_MASK_PADDING) && !aligned(c.mask, 4)) return MHA_E_ALIGN;
  const int64_t E = elem_size(c.dtype);
  if (!count_ok({c.B, c.H, c.Lq, c.D}, E) || !count_ok({c.B, c.H, c.Lk, c.D}, E) ||
      !count_ok({c.B, (c.kind & MHA_MASK_PER_HEAD) ? c.H : 1, c.Lq, c.Lk}, E))
    return MHA_E_OVERFLOW;
  // one head's K/V, and the additive-mask rows of one wave (at most 32), are
  // addressed through 32-bit buffer offsets, including a tile of overshoot
  if (((int64_t)c.Lk + 256) * c.D * E > 0xFFFFFFFFLL) return MHA_E_OVERFLOW;
  if (tensor && 32 * ((int64_t)c.Lk + 256) * E > 0xFFFFFFFFLL)
    return MHA_E_OVERFLOW;
  int bm = 0, tr = 0, tk = 0;
  if (c.dtype == MHA_F32) mha::tile_shape_f32(c.D, &bm, &tr, &tk);
  else if (c.dtype == MHA_F16) mha::tile_shape_f16(c.D, &bm, &tr, &tk);
  else mha::tile_shape_bf16(c.D, &bm, &tr, &tk);
  const int64_t grid = (int64_t)c.B * c.H * ((c.Lq + bm - 1) / bm);
  if (grid > 0x7fffffffLL) return MHA_E_OVERFLOW;
  return MHA_OK;
}

mha_status run(const Call& c) {
  mha_status st = validate(c);
  if (st != MHA_OK) return st;
  if (c.B == 0 || c.H == 0 || c.Lq == 0) return MHA_OK;
  if (c.with_ws && (c.kind & (MHA_MASK_ADDITIVE | MHA_MASK_KEEP)) == 0) {
    const size_t need = prenorm_ws(c.B, c.H, c.Lq, c.Lk, c.D, c.dtype).total;
    if (need > 0 && (!c.ws || !aligned(c.ws, 16) || c.ws_bytes < need)) return MHA_E_WORKSPACE;
  }
  uint32_t* flags = nullptr;
  st = device_flags(&flags);
  if (st != MHA_OK) return st;
  mha::Params p{};
  p.q = c.q;
  p.k = c.k;
  p.v = c.v;
  p.lens = (c.kind & MHA_MASK_PADDING) ? static_cast<const int32_t*>(c.mask) : nullptr;
  p.add = (c.kind & (MHA_MASK_ADDITIVE | MHA_MASK_KEEP)) ? c.mask : nullptr;
  p.x = c.x;
  p.gamma = c.gamma;
  p.beta = c.beta;
  p.residual = c.residual;
  p.out = c.out;
  p.B = c.B;
  p.H = c.H;
  p.Lq = c.Lq;
  p.Lk = c.Lk;
  p.kind = c.kind & (MHA_MASK_CAUSAL | MHA_MASK_PADDING | MHA_MASK_KEEP | MHA_MASK_PER_HEAD);
  p.c = (float)((double)c.scale * 1.4426950408889634);  // log2(e): exp(x) = 2^(x log2 e)
  p.scale = c.scale;
  p.eps = c.eps;
  p.add_vec = ((int64_t)c.Lk * elem_size(c.dtype)) % 16 == 0;
  p.flags = flags;
  p.counters = g_counters.load(std::memory_order_acquire);
  const bool add = (c.kind & (MHA_MASK_ADDITIVE | MHA_MASK_KEEP)) != 0;  // a mask tensor
  hipStream_t s = static_cast<hipStream_t>(c.stream);
  hipError_t e;
  if (c.with_ws && c.dtype == MHA_BF16 && !add && c.Lk > 0) {
    const PrenormWs ws = prenorm_ws(c.B, c.H, c.Lq, c.Lk, c.D, c.dtype);
    char* w = static_cast<char*>(c.ws);
    e = mha::launch_bf16_prenorm_kv16(p, c.D, w, w + ws.kv, reinterpret_cast<int*>(w + 2 * ws.kv),
                                      reinterpret_cast<float2*>(w + 2 * ws.kv + ws.flags), s);
    return e == hipSuccess ? MHA_OK : MHA_E_LAUNCH;
  }
  if (c.dtype == MHA_F32) e = mha::launch_f32(p, c.D, add, c.prenorm, s);
  else if (c.dtype == MHA_F16) e = mha::launch_f16(p, c.D, add, c.prenorm, s);
  else e = mha::launch_bf16(p, c.D, add, c.prenorm, s);
  return e == hipSuccess ? MHA_OK : MHA_E_LAUNCH;
}

// Decode: shape checks shared by the workspace query and the call. On success
// *chunk, *nsplit hold the split plan and *ws the workspace bytes it needs.
mha_status decode_check(int B, int H, int Lk, int D, mha_dtype dtype, int* chunk, int* nsplit,
                        size_t* ws) {
  if (dtype != MHA_F32 && dtype != MHA_F16 && dtype != MHA_BF16) return MHA_E_DTYPE;
  if (B < 0 || H < 0 || Lk < 0) return MHA_E_SHAPE;
  if (D != 16 && D != 32 && D != 64 && D != 128) return MHA_E_UNSUPPORTED;
  const int64_t E = elem_size(dtype);
  if (!count_ok({B, H, Lk, D}, E)) return MHA_E_OVERFLOW;
  if (((int64_t)Lk + 256) * D * E > 0xFFFFFFFFLL) return MHA_E_OVERFLOW;
  mha::decode_plan(B, H, Lk, D, (int)E, chunk, nsplit);
  const int64_t waves = (int64_t)B * H * *nsplit;
  if (waves > 0x7fffffffLL) return MHA_E_OVERFLOW;
  *ws = *nsplit > 1 ? (size_t)waves * (size_t)(D + 2) * sizeof(float) : 0;
  return MHA_OK;
}

}  // namespace

extern "C" {

mha_status mha_bwd_workspace_size(int B, int H, int Lq, mha_dtype dtype, size_t* bytes) {
  if (!bytes) return MHA_E_NULL;
  if (dtype != MHA_F32 && dtype != MHA_F16 && dtype != MHA_BF16) return MHA_E_DTYPE;
  if (B < 0 || H < 0 || Lq < 0) return MHA_E_SHAPE;
  if (!count_ok({B, H, Lq}, 8)) return MHA_E_OVERFLOW;
  *bytes = (size_t)B * H * Lq * 8;  // each row's log-sum-exp and sum_j P dP, float32
  return MHA_OK;
}

mha_status mha_bwd(const void* q, const void* k, const void* v, const void* dout,
                   const void* mask, unsigned mask_kind, int B, int H, int Lq,
                   int Lk, int D, float scale, mha_dtype dtype, void* workspace,
                   size_t workspace_bytes, void* stream, void* dq, void* dk, void* dv) {
  if (dtype != MHA_F32 && dtype != MHA_F16 && dtype != MHA_BF16) return MHA_E_DTYPE;
  if (mask_kind & ~31u) return MHA_E_MASK;
  const unsigned tensor = mask_kind & (MHA_MASK_ADDITIVE | MHA_MASK_KEEP);
  const unsigned ptr_kinds = mask_kind & (MHA_MASK_PADDING | MHA_MASK_ADDITIVE | MHA_MASK_KEEP);
  if (ptr_kinds & (ptr_kinds - 1)) return MHA_E_MASK;  // one mask argument
  if ((mask_kind & MHA_MASK_PER_HEAD) && !tensor) return MHA_E_MASK;
  const bool pad = (mask_kind & MHA_MASK_PADDING) != 0;
  if (!ptr_kinds && mask) return MHA_E_MASK;
  if (B < 0 || H < 0 || Lq < 0 || Lk < 0) return MHA_E_SHAPE;
  if (D != 16 && D != 32 && D != 64 && D != 128) return MHA_E_UNSUPPORTED;
  if (!std::isfinite(scale) || scale < 0.f) return MHA_E_ARG;
  if (B == 0 || H == 0 || (Lq == 0 && Lk == 0)) return MHA_OK;  // empty call
  if (ptr_kinds && !mask) return MHA_E_NULL;
  if (Lk > 0 && (!k || !v || !dk || !dv)) return MHA_E_NULL;
  if (Lq > 0 && (!q || !dout || !dq)) return MHA_E_NULL;
  const void* ptrs16[] = {q, k, v, dout, dq, dk, dv};
  for (const void* p : ptrs16)
    if (p && !aligned(p, 16)) return MHA_E_ALIGN;
  if ((pad && !aligned(mask, 4)) || (tensor && !aligned(mask, 16))) return MHA_E_ALIGN;
  if (!count_ok({B, H, Lq, D}, 2) || !count_ok({B, H, Lk, D}, 2) ||
      !count_ok({B, (mask_kind & MHA_MASK_PER_HEAD) ? H : 1, Lq, Lk}, 2))
    return MHA_E_OVERFLOW;
  if (((int64_t)Lq + 256) * D * 2 > 0xFFFFFFFFLL || ((int64_t)Lk + 256) * D * 2 > 0xFFFFFFFFLL)
    return MHA_E_OVERFLOW;
  const int64_t nq = (Lq + 31) / 32, nk = (Lk + 31) / 32;
  if ((int64_t)B * H * nq > 0x7fffffffLL || (int64_t)B * H * nk > 0x7fffffffLL)
    return MHA_E_OVERFLOW;
  const size_t ws = (size_t)B * H * Lq * 8;
  if (ws > 0 && (!workspace || !aligned(workspace, 16) || workspace_bytes < ws))
    return MHA_E_WORKSPACE;
  uint32_t* flags = nullptr;
  mha_status st = device_flags(&flags);
  if (st != MHA_OK) return st;
  mha::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.dout = dout;
  p.lens = pad ? static_cast<const int32_t*>(mask) : nullptr;
  p.mask = tensor ? mask : nullptr;
  p.mask_heads = (mask_kind & MHA_MASK_PER_HEAD) ? H : 1;
  p.keep = (mask_kind & MHA_MASK_KEEP) != 0;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.lse2 = static_cast<float*>(workspace);
  p.delta = p.lse2 ? p.lse2 + (int64_t)B * H * Lq : nullptr;
  p.B = B;
  p.H = H;
  p.Lq = Lq;
  p.Lk = Lk;
  p.nqblk = (int)nq;
  p.nkblk = (int)nk;
  p.causal = (mask_kind & MHA_MASK_CAUSAL) != 0;
  p.c = (float)((double)scale * 1.4426950408889634);
  p.scale = scale;
  p.flags = flags;
  const hipError_t e = mha::launch_bwd(p, (int)dtype, D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MHA_OK : MHA_E_LAUNCH;
}

mha_status mha_decode_workspace_size(int B, int H, int Lk, int D, mha_dtype dtype,
                                     size_t* bytes) {
  if (!bytes) return MHA_E_NULL;
  int chunk = 0, nsplit = 0;
  size_t ws = 0;
  mha_status st = decode_check(B, H, Lk, D, dtype, &chunk, &nsplit, &ws);
  if (st != MHA_OK) return st;
  *bytes = ws;
  return MHA_OK;
}

}  // extern "C"

namespace {

// Decode argument checks shared by both decode entry points (everything but
// the workspace). *empty is set for a call that has nothing to do.
mha_status decode_args(const void* q, const void* k, const void* v, const int32_t* lens,
                       int B, int H, int Lk, int D, float scale, mha_dtype dtype, void* out,
                       float* lse, int* chunk, int* nsplit, size_t* ws, bool* empty) {
  mha_status st = decode_check(B, H, Lk, D, dtype, chunk, nsplit, ws);
  if (st != MHA_OK) return st;
  if (!std::isfinite(scale) || scale < 0.f) return MHA_E_ARG;
  *empty = B == 0 || H == 0;
  if (*empty) return MHA_OK;
  if (!q || !out) return MHA_E_NULL;
  if (Lk > 0 && (!k || !v)) return MHA_E_NULL;
  const void* ptrs16[] = {q, k, v, out};
  for (const void* p : ptrs16)
    if (p && !aligned(p, 16)) return MHA_E_ALIGN;
  if ((lens && !aligned(lens, 4)) || (lse && !aligned(lse, 4))) return MHA_E_ALIGN;
  return MHA_OK;
}

// Enqueue the decode kernels with a validated workspace (ws bytes at `work`).
mha_status decode_launch(const void* q, const void* k, const void* v, const int32_t* lens,
                         int B, int H, int Lk, int D, float scale, mha_dtype dtype,
                         int chunk, int nsplit, size_t ws, void* work, uint32_t* flags,
                         void* stream, void* out, float* lse) {
  float* workspace = static_cast<float*>(work);
  mha::DecodeParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.lens = lens;
  p.out = out;
  p.lse = lse;
  const int64_t slots = (int64_t)B * H * nsplit;
  p.part_o = ws > 0 ? workspace : nullptr;
  p.part_ml = ws > 0 ? workspace + slots * D : nullptr;
  p.B = B;
  p.H = H;
  p.Lk = Lk;
  p.chunk = chunk;
  p.nsplit = nsplit;
  p.c = (float)((double)scale * 1.4426950408889634);  // log2(e): exp(x) = 2^(x log2 e)
  p.flags = flags;
  const hipError_t e = mha::launch_decode(p, (int)dtype, D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MHA_OK : MHA_E_LAUNCH;
}

}  // namespace

extern "C" {

mha_status mha_decode_fwd(const void* q, const void* k, const void* v, const int32_t* lens,
                          int B, int H, int Lk, int D, float scale, mha_dtype dtype,
                          void* workspace, size_t workspace_bytes, void* stream, void* out,
                          float* lse) {
  int chunk = 0, nsplit = 0;
  size_t ws = 0;
  bool empty = false;
  mha_status st = decode_args(q, k, v, lens, B, H, Lk, D, scale, dtype, out, lse, &chunk,
                              &nsplit, &ws, &empty);
  if (st != MHA_OK || empty) return st;
  if (ws > 0 && (!workspace || !aligned(workspace, 16) || workspace_bytes < ws))
    return MHA_E_WORKSPACE;
  uint32_t* flags = nullptr;
  st = device_flags(&flags);
  if (st != MHA_OK) return st;
  return decode_launch(q, k, v, lens, B, H, Lk, D, scale, dtype, chunk, nsplit, ws, workspace,
                       flags, stream, out, lse);
}

mha_status mha_decode_fwd_noalloc(const void* q, const void* k, const void* v,
                                  const int32_t* lens, int B, int H, int Lk, int D, float scale,
                                  mha_dtype dtype, void* stream, void* out, float* lse) {
  int chunk = 0, nsplit = 0;
  size_t ws = 0;
  bool empty = false;
  mha_status st = decode_args(q, k, v, lens, B, H, Lk, D, scale, dtype, out, lse, &chunk,
                              &nsplit, &ws, &empty);
  if (st != MHA_OK || empty) return st;
  if (ws > (size_t)MHA_NOALLOC_SCRATCH_BYTES) return MHA_E_SCRATCH;
  uint32_t* flags = nullptr;
  void* scr = nullptr;
  st = device_noalloc_state(&flags, &scr);
  if (st != MHA_OK) return st;
  // the split kernel writes every partial result the merge kernel reads, so
  // the scratch needs no clearing between calls
  return decode_launch(q, k, v, lens, B, H, Lk, D, scale, dtype, chunk, nsplit, ws, scr, flags,
                       stream, out, lse);
}

mha_status mha_noalloc_scratch_bytes(size_t* bytes) {
  if (!bytes) return MHA_E_NULL;
  *bytes = MHA_NOALLOC_SCRATCH_BYTES;
  return MHA_OK;
}

mha_status mha_init(void) {
  uint32_t* f = nullptr;
  const mha_status st = device_flags(&f);
  if (st != MHA_OK) return st;
  return device_scratch_setup();
}

mha_status mha_fwd(const void* q, const void* k, const void* v, const void* mask,
                   unsigned mask_kind, int B, int H, int Lq, int Lk, int D, float scale,
                   mha_dtype dtype, void* stream, void* out) {
  Call c{q, nullptr, k, v, mask, mask_kind, nullptr, nullptr, 0.f, nullptr,
         B, H, Lq, Lk, D, scale, dtype, stream, out, false};
  return run(c);
}

mha_status mha_prenorm_cross_fwd(const void* x, const void* k, const void* v, const void* mask,
                                 unsigned mask_kind, const void* gamma, const void* beta,
                                 float eps, const void* residual, int B, int H, int Lq, int Lk,
                                 int D, float scale, mha_dtype dtype, void* stream, void* out) {
  Call c{nullptr, x, k, v, mask, mask_kind, gamma, beta, eps, residual,
         B, H, Lq, Lk, D, scale, dtype, stream, out, true};
  return run(c);
}

mha_status mha_prenorm_cross_fwd_ws(const void* x, const void* k, const void* v, const void* mask,
                                    unsigned mask_kind, const void* gamma, const void* beta,
                                    float eps, const void* residual, int B, int H, int Lq, int Lk,
                                    int D, float scale, mha_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* stream, void* out) {
  Call c{nullptr, x, k, v, mask, mask_kind, gamma, beta, eps, residual,
         B, H, Lq, Lk, D, scale, dtype, stream, out, true};
  c.with_ws = true;
  c.ws = workspace;
  c.ws_bytes = workspace_bytes;
  return run(c);
}

mha_status mha_prenorm_cross_workspace_size(int B, int H, int Lq, int Lk, int D, mha_dtype dtype,
                                            size_t* bytes) {
  if (!bytes) return MHA_E_NULL;
  if (dtype != MHA_F32 && dtype != MHA_F16 && dtype != MHA_BF16) return MHA_E_DTYPE;
  if (B < 0 || H < 0 || Lq < 0 || Lk < 0) return MHA_E_SHAPE;
  if (D != 16 && D != 32 && D != 64 && D != 128) return MHA_E_UNSUPPORTED;
  if (!count_ok({B, H, Lk, D}, 2) || !count_ok({B, Lq, 8}, 1)) return MHA_E_OVERFLOW;
  *bytes = prenorm_ws(B, H, Lq, Lk, D, dtype).total;
  return MHA_OK;
}

mha_status mha_softmax_rows(const void* s, void* p, int64_t rows, int cols, float scale,
                            mha_dtype dtype, void* stream) {
  if (dtype != MHA_F32 && dtype != MHA_F16 && dtype != MHA_BF16) return MHA_E_DTYPE;
  if (rows < 0 || cols < 0) return MHA_E_SHAPE;
  if (!std::isfinite(scale) || scale < 0.f) return MHA_E_ARG;
  if (rows == 0 || cols == 0) return MHA_OK;  // empty call
  if (!s || !p) return MHA_E_NULL;
  const int64_t E = elem_size(dtype);
  if (!aligned(s, (uintptr_t)E) || !aligned(p, (uintptr_t)E)) return MHA_E_ALIGN;
  if (!count_ok({rows, cols}, E) || (rows + 3) / 4 > 0x7fffffffLL) return MHA_E_OVERFLOW;
  uint32_t* flags = nullptr;
  mha_status st = device_flags(&flags);
  if (st != MHA_OK) return st;
  mha::SoftmaxParams sp{};
  sp.s = s;
  sp.p = p;
  sp.rows = rows;
  sp.cols = cols;
  sp.c = scale * 1.4426950408889634f;
  sp.flags = flags;
  const bool vec_ok = aligned(s, 16) && aligned(p, 16) && ((int64_t)cols * E) % 16 == 0;
  const hipError_t e =
      mha::launch_softmax_rows(sp, (int)dtype, vec_ok, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MHA_OK : MHA_E_LAUNCH;
}

mha_status mha_get_flags(void* stream, uint32_t* flags, int clear) {
  if (!flags) return MHA_E_NULL;
  uint32_t* dflags = nullptr;
  mha_status st = device_flags(&dflags);
  if (st != MHA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return MHA_E_NO_DEVICE;
  if (hipMemcpy(flags, dflags, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return MHA_E_NO_DEVICE;
  if (clear) {
    if (hipMemsetAsync(dflags, 0, sizeof(uint32_t), s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return MHA_E_NO_DEVICE;
  }
  return MHA_OK;
}

mha_status mha_set_debug_counters(uint64_t* dev_counters) {
  if (dev_counters && !aligned(dev_counters, 8)) return MHA_E_ALIGN;
  g_counters.store(reinterpret_cast<unsigned long long*>(dev_counters), std::memory_order_release);
  return MHA_OK;
}

mha_status mha_tile_config(mha_dtype dtype, int D, unsigned mask_kind, int* rows, int* keys) {
  if (!rows || !keys) return MHA_E_NULL;
  if (dtype != MHA_F32 && dtype != MHA_F16 && dtype != MHA_BF16) return MHA_E_DTYPE;
  if (mask_kind & ~31u) return MHA_E_MASK;
  if (D != 16 && D != 32 && D != 64 && D != 128) return MHA_E_UNSUPPORTED;
  int bm = 0;
  if (dtype == MHA_F32) mha::tile_shape_f32(D, &bm, rows, keys);
  else if (dtype == MHA_F16) mha::tile_shape_f16(D, &bm, rows, keys);
  else mha::tile_shape_bf16(D, &bm, rows, keys);
  return MHA_OK;
}

const char* mha_status_str(mha_status s) {
  switch (s) {
    case MHA_OK: return "MHA_OK";
    case MHA_E_NULL: return "MHA_E_NULL: a required pointer is NULL";
    case MHA_E_SHAPE: return "MHA_E_SHAPE: invalid dimension";
    case MHA_E_DTYPE: return "MHA_E_DTYPE: unknown dtype";
    case MHA_E_MASK: return "MHA_E_MASK: invalid mask kind or mask pointer";
    case MHA_E_UNSUPPORTED: return "MHA_E_UNSUPPORTED: D must be 16, 32, 64 or 128";
    case MHA_E_ALIGN: return "MHA_E_ALIGN: a tensor pointer is misaligned";
    case MHA_E_OVERFLOW: return "MHA_E_OVERFLOW: sizes overflow";
    case MHA_E_NO_DEVICE: return "MHA_E_NO_DEVICE: no usable HIP device";
    case MHA_E_LAUNCH: return "MHA_E_LAUNCH: kernel launch failed";
    case MHA_E_ARG: return "MHA_E_ARG: scale or eps out of range";
    case MHA_E_WORKSPACE: return "MHA_E_WORKSPACE: workspace missing, misaligned or too small";
    case MHA_E_NOT_INITIALIZED:
      return "MHA_E_NOT_INITIALIZED: call mha_init on this device before an allocation-free entry point";
    case MHA_E_SCRATCH:
      return "MHA_E_SCRATCH: the call needs more scratch than MHA_NOALLOC_SCRATCH_BYTES";
  }
  return "unknown mha_status";
}

}  // extern "C"
