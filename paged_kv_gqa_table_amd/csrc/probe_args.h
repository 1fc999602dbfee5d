// Launcher of the streaming read probe (read_probe.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace pkv {

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);

}  // namespace pkv
