// Placeholder: groups of 8 go through the vector-ALU kernel until the MFMA kernel lands.
#include "decode_args.h"

namespace pkv {
hipError_t launch_decode_mfma_bf16_tm(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  return G <= 8 ? launch_decode_valu_bf16_tm(a, G, grid_parts, s) : hipErrorNotSupported;
}
hipError_t launch_decode_mfma_bf16_xp(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  return G <= 8 ? launch_decode_valu_bf16_xp(a, G, grid_parts, s) : hipErrorNotSupported;
}
}  // namespace pkv
