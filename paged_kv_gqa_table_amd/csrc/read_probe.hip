// Plain streaming read of a device buffer, for measuring the read bandwidth the GPU
// sustains for the simplest access pattern (a reference point for the decode kernels'
// gathers; no part of the attention path uses it).
//
// Each lane reads 16 bytes per load, 8 loads in flight, grid-stride over the buffer, and
// folds what it read into one word with XOR. The word is written only if it equals a
// constant, which keeps the loads alive without a write per workgroup.
#include "common.h"
#include "probe_args.h"

namespace pkv {

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
constexpr uint32_t kReadMagic = 0x9e3779b9u;
constexpr int kReadGridPerCU = 32;  // measured best for this loop on MI355X (8 loads in flight)

__global__ __launch_bounds__(kReadThreads) void read_probe_kernel(const u32x4_t* p, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4_t v[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(p + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == kReadMagic) sink[0] = x;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t per_block = (size_t)kReadThreads * kReadUnroll;
  const size_t want = (n16 + per_block - 1) / per_block;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const size_t cap = (size_t)kReadGridPerCU * cus;
  const int grid = (int)(want < cap ? want : cap);
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kReadThreads), 0, s, reinterpret_cast<const u32x4_t*>(buf),
                     n16, sink);
  return hipGetLastError();
}

}  // namespace pkv
