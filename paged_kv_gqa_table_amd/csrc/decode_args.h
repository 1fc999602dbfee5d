// Launch arguments shared by the decode kernels and the host dispatcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct DecodePartialArgs {
  const void* q;          // [S, H, D]
  const void* kc;         // K pool (layout-dependent)
  const void* vc;         // V pool (layout-dependent)
  const int32_t* bt;      // [S, mb]
  const int32_t* lens;    // [S]
  int mb;                 // max_blocks_per_seq
  int S, H, KVH, D, NB;   // sizes; NB = pool blocks
  float scale_log2;       // scale * log2(e): scores are kept in base-2 units inside
  int ps;                 // partition size in tokens (multiple of 16)
  int ppp;                // pages per partition = ps / 16
  int P;                  // max_num_partitions: stride of the partial arrays
  float* acc;             // [S, H, P, D]
  float* m;               // [S, H, P]
  float* l;               // [S, H, P]
};

struct DecodeReduceArgs {
  const float* acc;
  const float* m;
  const float* l;
  const int32_t* lens;
  int S, H, D, ps, P;
  void* out;
  float* lse;             // may be null
};

// Launchers: return hipSuccess or the launch error. grid_parts = ceil(max_seq_len / ps).
hipError_t launch_decode_valu_f32_tm(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s);
hipError_t launch_decode_valu_f32_xp(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s);
hipError_t launch_decode_valu_bf16_tm(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s);
hipError_t launch_decode_valu_bf16_xp(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s);
hipError_t launch_decode_mfma_bf16_tm(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s);
hipError_t launch_decode_mfma_bf16_xp(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s);
hipError_t launch_decode_reduce(const DecodeReduceArgs& a, bool out_bf16, hipStream_t s);

// Workgroup cap of the dense decode launches on the current device (host side).
int dense_grid_cap();
// Workgroups of `kernel` (block_threads threads, dyn_lds bytes of dynamic LDS) that the
// current device holds at once; dense_grid_cap() if the runtime cannot tell.
int resident_grid(const void* kernel, int block_threads, size_t dyn_lds);

}  // namespace pkv
