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
  int len_cap;            // lengths are clamped to this many tokens: min(mb * 16, launched
                          // partitions * ps), or mb * 16 under NUM_SPLITS, so no partition
                          // index reaches the launched grid (or P)
  int S, H, KVH, D, NB;   // sizes; NB = pool blocks
  float scale_log2;       // scale * log2(e): scores are kept in base-2 units inside
  int ps;                 // partition size in tokens (multiple of 16); unused when nsplit > 0
  int ppp;                // pages per partition = ps / 16; unused when nsplit > 0
  int nsplit;             // > 0: NUM_SPLITS policy, ceil(pages_b / nsplit) pages per partition
  int bs;                 // block size (tokens per page) of the pools: 16 for every kernel but
                          // the generic one
  int normalize;          // != 0: store acc / l instead of acc
  const float* alibi;     // [H] ALiBi slopes (natural-log units), or null: score of key t
                          // gets -slope_h * (len - 1 - t)
  int kv_fp8;             // != 0: K/V pools hold float8 e4m3 (query and out stay bf16)
  float v_scale;          // float8 V dequantization factor (k_scale is folded into scale_log2)
  int P;                  // max_num_partitions: stride of the partial arrays
  float* acc;             // [S, H, P, D]; may be null in final mode when P == 1
  float* m;               // [S, H, P]
  float* l;               // [S, H, P]
  // Final mode (out != null): one launch computes the output. A (sequence, kv head) with a
  // single partition writes out / lse directly; otherwise its partials are written and the
  // last workgroup to finish one of its partitions (counted in counters[b * KVH + kvh],
  // which it resets to 0) combines them.
  void* out;              // [S, H, D], the query dtype
  float* lse;             // [S, H] natural log, may be null
  int* counters;          // [S * KVH], zero on entry and on exit; null when P == 1
};

// Tokens per partition of a sequence of len tokens: the fixed partition size, or under the
// NUM_SPLITS policy (flash-decode post, split-K partial kernel) ceil(ceil(len / bs) / nsplit)
// whole pages of bs tokens (at least one page, so that an empty sequence has no partitions).
__host__ __device__ inline int part_tokens(int len, int ps, int nsplit, int bs) {
  if (nsplit <= 0) return ps;
  const int pages = (len + bs - 1) / bs;
  const int ppp = (pages + nsplit - 1) / nsplit;
  return (ppp > 0 ? ppp : 1) * bs;
}

struct DecodeReduceArgs {
  const float* acc;
  const float* m;
  const float* l;
  const int32_t* lens;
  int S, H, D, ps, P;
  int nsplit, bs;         // NUM_SPLITS policy when nsplit > 0 (see part_tokens)
  int normalized;         // != 0: acc rows hold acc / l
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
// Any block size (a.bs), head dim 64/128/256, G <= 16, float32 or bf16 query, both layouts.
hipError_t launch_decode_generic(const DecodePartialArgs& a, int G, int grid_parts, bool xp, bool q_f32,
                                 hipStream_t s);

// Sets the calling thread's pkv_last_error() message (printf format) and returns `code`.
int set_last_error(int code, const char* fmt, ...);

// Workgroup cap of the dense decode launches on the current device (host side).
int dense_grid_cap();
// Workgroups of `kernel` (block_threads threads, dyn_lds bytes of dynamic LDS) that the
// current device holds at once; dense_grid_cap() if the runtime cannot tell.
int resident_grid(const void* kernel, int block_threads, size_t dyn_lds);

}  // namespace pkv
