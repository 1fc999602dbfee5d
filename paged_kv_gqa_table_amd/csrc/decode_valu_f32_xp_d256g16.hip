// float32 vector-ALU decode instances, x-packed layout, head dim 256, G 9 .. 16.
#include "decode_valu.h"

namespace pkv {
hipError_t launch_valu_f32_xp_d256g16(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  return launch_valu_g<true, 256, 9, 16>(a, G, grid_parts, s);
}
}  // namespace pkv
