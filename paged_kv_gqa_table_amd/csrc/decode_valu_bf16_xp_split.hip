// bf16 vector-ALU decode instances of one (layout, mode) pair; one translation unit per pair
// so that the build compiles them in parallel.
#include "decode_valu_bf16.h"

namespace pkv {
hipError_t launch_bf16_xp_split(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  return launch_bf16_mode<true, true, false>(a, G, grid_parts, s);
}
}  // namespace pkv
