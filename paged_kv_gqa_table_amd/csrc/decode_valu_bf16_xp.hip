// Instances of the bf16 vector-ALU decode kernel for one layout; one translation unit per
// (dtype, layout) so the build compiles them in parallel.
#include "decode_valu_bf16.h"

namespace pkv {
hipError_t launch_decode_valu_bf16_xp(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  return launch_bf16<true>(a, G, grid_parts, s);
}
}  // namespace pkv
