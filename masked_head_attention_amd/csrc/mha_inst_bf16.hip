// Kernel instantiations for one element type.
#include "mha_launch.hpp"

namespace mha {
hipError_t launch_bf16(const Params& p, int D, bool add, bool pre, hipStream_t s) {
  return launch_dtype<__bf16>(p, D, add, pre, s);
}
void tile_shape_bf16(int D, int* bm, int* rows, int* keys) { tile_shape<__bf16>(D, bm, rows, keys); }
hipError_t launch_bf16_prenorm_kv16(const Params& p, int D, void* k16, void* v16, int* flags,
                                    float2* stats, hipStream_t s) {
  switch (D) {
    case 16: return launch_prenorm_kv16<16>(p, k16, v16, flags, stats, s);
    case 32: return launch_prenorm_kv16<32>(p, k16, v16, flags, stats, s);
    case 64: return launch_prenorm_kv16<64>(p, k16, v16, flags, stats, s);
    case 128: return launch_prenorm_kv16<128>(p, k16, v16, flags, stats, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace mha
