// Kernel instantiations for one element type.
#include "mha_launch.hpp"

namespace mha {
hipError_t launch_f32(const Params& p, int D, bool add, bool pre, hipStream_t s) {
  return launch_dtype<float>(p, D, add, pre, s);
}
void tile_shape_f32(int D, int* bm, int* rows, int* keys) { tile_shape<float>(D, bm, rows, keys); }
}  // namespace mha
