// MLA causal paged prefill (placeholder until the MFMA kernel lands).
#include "mla_args.h"

namespace pkv {
hipError_t launch_mla_prefill(const MlaArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace pkv
