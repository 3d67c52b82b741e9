// Row-softmax kernel instantiations, one per element type.
#include "mha_softmax.hpp"

namespace mha {
hipError_t launch_softmax_rows(const SoftmaxParams& p, int dtype, bool vec_ok, hipStream_t s) {
  switch (dtype) {
    case 0: return launch_softmax<float>(p, vec_ok, s);
    case 1: return launch_softmax<_Float16>(p, vec_ok, s);
    default: return launch_softmax<__bf16>(p, vec_ok, s);
  }
}
}  // namespace mha
