// float32 vector-ALU decode instances, x-packed layout, G 9 .. 16 at head dims 64 and 128.
#include "decode_valu.h"

namespace pkv {
hipError_t launch_valu_f32_xp_g16(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_valu_g<true, 64, 9, 16>(a, G, grid_parts, s);
    case 128: return launch_valu_g<true, 128, 9, 16>(a, G, grid_parts, s);
    default: return hipErrorNotSupported;
  }
}
}  // namespace pkv
