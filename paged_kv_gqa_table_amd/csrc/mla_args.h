// Launch arguments of the MLA causal paged-prefill kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kMlaMaxBatch = 512;  // batches per chunk of the prefill kernel's LDS tile list

struct MlaArgs {
  const void* q_nope;        // [total_q, 16, 512] bf16
  const void* q_pe;          // [total_q, 16, 64] bf16
  const void* ckv;           // [num_pages, 1, 512] bf16
  const void* kpe;           // [num_pages, 1, 64] bf16
  const int32_t* qo_indptr;  // [batch + 1]
  const int32_t* kv_indptr;  // [batch + 1]
  const int32_t* kv_indices; // [kv_indptr[batch]]
  int batch, total_q, max_q_len, num_pages;
  float sm_scale_log2;       // sm_scale * log2(e)
  void* out;                 // [total_q, 16, 512] bf16
  float* lse;                // [total_q, 16] base 2
};

hipError_t launch_mla_prefill(const MlaArgs& a, hipStream_t s);

// Pages of several tokens: token-level offsets and pool rows for the prefill kernel above.
struct MlaPagesArgs {
  const int32_t* kv_indptr;         // [batch + 1] in pages
  const int32_t* kv_indices;        // [num_kv_indices] page ids
  const int32_t* last_len;          // [batch] tokens in each batch's last page, or null (full)
  int batch, num_kv_indices, num_pages, ps;
  int32_t* tok_indptr;              // [batch + 1] out: token offsets
  int32_t* tok_rows;                // [num_kv_indices * ps] out: pool row (page * ps + slot) per token
};

hipError_t launch_mla_expand_pages(const MlaPagesArgs& a, hipStream_t s);

// MLA decode (one new token per sequence), split-K over the latent cache.
struct MlaDecodeArgs {
  const void* q_nope;         // [batch, 16, 512] bf16
  const void* q_pe;           // [batch, 16, 64] bf16
  const void* ckv;            // [num_pages, 1, 512] bf16 (also V)
  const void* kpe;            // [num_pages, 1, 64] bf16
  const int32_t* kv_indptr;   // [batch + 1]
  const int32_t* kv_indices;  // [kv_indptr[batch]] token ids
  int batch, num_pages, num_kv_indices;
  int split;                  // tokens per split (multiple of 16)
  int P;                      // max_num_splits: stride of the partial arrays
  int len_cap;                // lengths are clamped to (launched splits) * split tokens
  float sm_scale_log2;        // sm_scale * log2(e)
  float* acc;                 // [batch, 16, P, 512]
  float* m;                   // [batch, 16, P] natural log
  float* l;                   // [batch, 16, P]
  int32_t* counters;          // [batch], zero; null: the combine is a second launch
  void* out;                  // [batch, 16, 512] bf16
  float* lse;                 // [batch, 16] base 2
};

hipError_t launch_mla_decode(const MlaDecodeArgs& a, int grid_parts, hipStream_t s);

// Workgroup cap for persistent-style grids on the current device (host side).
int dense_grid_cap();

}  // namespace pkv
