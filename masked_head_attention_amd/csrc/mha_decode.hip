// Decode kernels (one query row per head against a key/value cache), one
// instantiation per element type and head size, and the host-side split plan.
#include "mha_decode.hpp"

namespace mha {

// Keys per split: at most 32 KiB of K rows per wave (128 keys at D = 128 in
// 16-bit types), halved while the launch would hold fewer than 8192
// (head, split) waves (32 per CU), down to 64 keys or one iteration. A single
// split stores the row directly. Measured on the float16 H = 32, D = 128
// decode workload (cache lengths 256..4096): 128-key splits 102.7 us per call,
// 64: 106.1, 256: 107.3, 512: 117.0.
void decode_plan(int B, int H, int Lk, int D, int esize, int* chunk, int* nsplit) {
  const int rb = D * esize;
  const int kpi = decode_keys_per_iter(D, esize);
  const int cmin = kpi > 64 ? kpi : 64;
  int c = 32768 / rb > cmin ? 32768 / rb : cmin;
  const long long heads = (long long)B * H;
  while (c > cmin && heads * ((Lk + c - 1) / c) < 8192) c /= 2;
  *chunk = c;
  const int n = (Lk + c - 1) / c;
  *nsplit = n > 1 ? n : 1;
}

template <typename T>
static hipError_t launch_decode_dtype(const DecodeParams& p, int D, hipStream_t s) {
  switch (D) {
    case 16: return launch_decode_t<T, 16>(p, s);
    case 32: return launch_decode_t<T, 32>(p, s);
    case 64: return launch_decode_t<T, 64>(p, s);
    case 128: return launch_decode_t<T, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeParams& p, int dtype, int D, hipStream_t s) {
  switch (dtype) {
    case 0: return launch_decode_dtype<float>(p, D, s);
    case 1: return launch_decode_dtype<_Float16>(p, D, s);
    default: return launch_decode_dtype<__bf16>(p, D, s);
  }
}

}  // namespace mha
