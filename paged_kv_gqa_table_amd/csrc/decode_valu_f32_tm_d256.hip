// float32 vector-ALU decode instances, token-major layout, head dim 256, G 1 .. 8 (G 9 .. 16 in
// the _d256g16 unit, so that the build compiles the two halves in parallel).
#include "decode_valu.h"

namespace pkv {
hipError_t launch_valu_f32_tm_d256(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  if (G > 8) return launch_valu_f32_tm_d256g16(a, G, grid_parts, s);
  return launch_valu_g<false, 256, 1, 8>(a, G, grid_parts, s);
}
}  // namespace pkv
