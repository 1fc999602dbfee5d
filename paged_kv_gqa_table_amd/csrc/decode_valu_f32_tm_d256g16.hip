// float32 vector-ALU decode instances, token-major layout, head dim 256, G 9 .. 16.
#include "decode_valu.h"

namespace pkv {
hipError_t launch_valu_f32_tm_d256g16(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  return launch_valu_g<false, 256, 9, 16>(a, G, grid_parts, s);
}
}  // namespace pkv
