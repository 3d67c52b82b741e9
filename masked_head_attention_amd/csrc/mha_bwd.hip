// Backward kernels (dQ, then dK and dV), one instantiation per element type
// and head size.
#include "mha_bwd_f32.hpp"

namespace mha {

template <typename T>
static hipError_t launch_bwd_dtype(const BwdParams& p, int D, hipStream_t s) {
  switch (D) {
    case 16: return launch_bwd_t<T, 16>(p, s);
    case 32: return launch_bwd_t<T, 32>(p, s);
    case 64: return launch_bwd_t<T, 64>(p, s);
    case 128: return launch_bwd_t<T, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t launch_bwd_float(const BwdParams& p, int D, hipStream_t s) {
  switch (D) {
    case 16: return launch_bwd_f32<16>(p, s);
    case 32: return launch_bwd_f32<32>(p, s);
    case 64: return launch_bwd_f32<64>(p, s);
    case 128: return launch_bwd_f32<128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd(const BwdParams& p, int dtype, int D, hipStream_t s) {
  if (dtype == 0) return launch_bwd_float(p, D, s);
  return dtype == 1 ? launch_bwd_dtype<_Float16>(p, D, s) : launch_bwd_dtype<__bf16>(p, D, s);
}

}  // namespace mha
