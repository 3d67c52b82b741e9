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

// float32: the MFMA kernels of the 16-bit types (v_mfma_f32_32x32x2_f32) up to
// D = 64; at D = 128 their tiles and fragments would not fit a CU's LDS and a
// lane's registers, and the vector-ALU kernels run.
static hipError_t launch_bwd_float(const BwdParams& p, int D, hipStream_t s) {
  switch (D) {
    case 16: return launch_bwd_t<float, 16>(p, s);
    case 32: return launch_bwd_t<float, 32>(p, s);
    case 64: return launch_bwd_t<float, 64>(p, s);
    case 128: return launch_bwd_f32<128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd(const BwdParams& p, int dtype, int D, hipStream_t s) {
  if (dtype == 0) return launch_bwd_float(p, D, s);
  return dtype == 1 ? launch_bwd_dtype<_Float16>(p, D, s) : launch_bwd_dtype<__bf16>(p, D, s);
}

}  // namespace mha
