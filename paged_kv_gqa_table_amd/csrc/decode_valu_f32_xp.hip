// Instances of the vector-ALU decode kernel for one (dtype, layout) pair; split into
// separate translation units so the build compiles them in parallel.
#include "decode_valu.h"

namespace pkv {
hipError_t launch_decode_valu_f32_xp(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  return launch_valu<true>(a, G, grid_parts, s);
}
}  // namespace pkv
