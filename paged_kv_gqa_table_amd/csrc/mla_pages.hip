// MLA prefill over pages of several tokens: a small index kernel that turns the page-level
// description (kv_indptr counting pages, kv_indices page ids, the last page's token count)
// into token-level offsets and pool rows, so that the one-token-per-row prefill kernel
// (mla_prefill.hip) runs unchanged on the pool viewed as [num_pages * ps, 1, dim].
//
// The page's kernel takes a PAGE_SIZE while its host wrapper asserts 1; the layout read
// here is the plainest one its page-counting kv_indptr supports: batch b owns pages
// kv_indices[kv_indptr[b] .. kv_indptr[b+1]-1] in order, each holds ps tokens except the
// last, which holds last_len[b] (ps when the array is absent), and key token j is slot
// j % ps of the batch's (j / ps)-th page. The index arrays cost 4 bytes per token against
// 1152 bytes of ckv + kpe that the prefill kernel then reads for it.
#include "common.h"
#include "mla_args.h"

namespace pkv {
namespace {

constexpr int kExpandThreads = 256;

// Every workgroup rebuilds the per-batch page and token offsets in LDS (page offsets
// clamped into [0, num_kv_indices] and made non-decreasing, last-page lengths into
// [1, ps], so every write below stays inside tok_rows whatever the device arrays hold);
// workgroup 0 also stores the token offsets. Then each page of the grid-stride range
// writes the pool rows of its tokens.
__global__ __launch_bounds__(kExpandThreads) void mla_expand_pages_kernel(MlaPagesArgs a) {
  extern __shared__ int s_idx[];
  int* s_pg = s_idx;                 // [batch + 1] page offsets
  int* s_tok = s_idx + a.batch + 1;  // [batch + 1] token offsets
  int* s_last = s_tok + a.batch + 1; // [batch] tokens in the last page
  for (int i = threadIdx.x; i <= a.batch; i += blockDim.x) {
    int v = a.kv_indptr[i];
    s_pg[i] = v < 0 ? 0 : (v > a.num_kv_indices ? a.num_kv_indices : v);
    if (i < a.batch) {
      int l = a.last_len != nullptr ? a.last_len[i] : a.ps;
      s_last[i] = l < 1 ? 1 : (l > a.ps ? a.ps : l);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // at most kMlaMaxBatch batches: a serial pass is cheap
    int run = 0;
    s_tok[0] = 0;
    for (int b = 0; b < a.batch; ++b) {
      if (s_pg[b + 1] < s_pg[b]) s_pg[b + 1] = s_pg[b];
      const int np = s_pg[b + 1] - s_pg[b];
      run += np > 0 ? (np - 1) * a.ps + s_last[b] : 0;
      s_tok[b + 1] = run;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= a.batch; i += blockDim.x) a.tok_indptr[i] = s_tok[i];
  const int lo_page = s_pg[0], hi_page = s_pg[a.batch];
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < a.num_kv_indices; i += gridDim.x * blockDim.x) {
    if (i < lo_page || i >= hi_page) continue;  // not owned by any batch
    int lo = 0, hi = a.batch;  // s_pg[lo] <= i < s_pg[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pg[mid] <= i) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int j = i - s_pg[b];  // page index within the batch
    const int cnt = (i == s_pg[b + 1] - 1) ? s_last[b] : a.ps;
    int page = a.kv_indices[i];
    page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
    int32_t* dst = a.tok_rows + s_tok[b] + j * a.ps;
    for (int t = 0; t < cnt; ++t) dst[t] = page * a.ps + t;
  }
}

}  // namespace

hipError_t launch_mla_expand_pages(const MlaPagesArgs& a, hipStream_t s) {
  const int blocks = a.num_kv_indices > 0 ? (a.num_kv_indices + kExpandThreads - 1) / kExpandThreads : 1;
  const int grid = blocks < 1024 ? blocks : 1024;
  const size_t lds = (size_t)(3 * a.batch + 2) * sizeof(int);
  hipLaunchKernelGGL(mla_expand_pages_kernel, dim3(grid), dim3(kExpandThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace pkv
