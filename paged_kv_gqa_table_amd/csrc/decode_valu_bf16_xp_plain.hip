// bf16 vector-ALU decode instances of one (layout, mode) pair; one translation unit per pair
// so that the build compiles them in parallel.
#include "decode_valu_bf16.h"

namespace pkv {
hipError_t launch_bf16_xp_plain(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  return launch_bf16_mode<true, false, false>(a, G, grid_parts, s);
}

// Phase 1 of the bf16 vector-ALU kernel in the xp layout: the instance family of the mode.
hipError_t launch_decode_valu_bf16_xp(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  const bool fin = a.out != nullptr;
  if (a.nsplit > 0) return fin ? launch_bf16_xp_split_final(a, G, grid_parts, s) : launch_bf16_xp_split(a, G, grid_parts, s);
  return fin ? launch_bf16_xp_final(a, G, grid_parts, s) : launch_bf16_xp_plain(a, G, grid_parts, s);
}
}  // namespace pkv
