// Kernel instantiations for one element type.
#include "mha_launch.hpp"

namespace mha {
hipError_t launch_f16(const Params& p, int D, bool add, bool pre, hipStream_t s) {
  return launch_dtype<_Float16>(p, D, add, pre, s);
}
void tile_shape_f16(int D, int* bm, int* rows, int* keys) { tile_shape<_Float16>(D, bm, rows, keys); }
}  // namespace mha
