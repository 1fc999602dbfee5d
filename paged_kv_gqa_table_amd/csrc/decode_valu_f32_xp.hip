// float32 vector-ALU decode instances, x-packed layout: head dims 64 and 128 with G <= 8
// here, head dim 256 and larger groups in the _d256 and _g16 units.
#include "decode_valu.h"

namespace pkv {
hipError_t launch_decode_valu_f32_xp(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  if (G < 1 || G > 16) return hipErrorNotSupported;
  if (a.D == 256) return launch_valu_f32_xp_d256(a, G, grid_parts, s);
  if (G > 8) return launch_valu_f32_xp_g16(a, G, grid_parts, s);
  switch (a.D) {
    case 64: return launch_valu_g<true, 64, 1, 8>(a, G, grid_parts, s);
    case 128: return launch_valu_g<true, 128, 1, 8>(a, G, grid_parts, s);
    default: return hipErrorNotSupported;
  }
}
}  // namespace pkv
