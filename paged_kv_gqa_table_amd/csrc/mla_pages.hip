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
// 1152 bytes of ckv + kpe that the prefill kernel then reads for it. Two launches: a
// one-workgroup scan of the token counts, then one workgroup per batch writing its rows,
// so nothing here grows with the batch count but the grid.
#include "common.h"
#include "mla_args.h"

namespace pkv {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanPer = 4;  // batches per thread and pass of the scan
constexpr int kExpandThreads = 256;

// Page range [lo, hi) and token count of batch b, every value clamped so that whatever the
// device arrays hold, the ranges stay inside [0, num_kv_indices] and counts are >= 0
// (for a well-formed kv_indptr these are the batch's own pages).
__device__ __forceinline__ void batch_pages(const MlaPagesArgs& a, int b, int& lo, int& hi, int& ntok) {
  int x = a.kv_indptr[b], y = a.kv_indptr[b + 1];
  lo = x < 0 ? 0 : (x > a.num_kv_indices ? a.num_kv_indices : x);
  y = y < 0 ? 0 : (y > a.num_kv_indices ? a.num_kv_indices : y);
  hi = y < lo ? lo : y;
  int last = a.last_len != nullptr ? a.last_len[b] : a.ps;
  last = last < 1 ? 1 : (last > a.ps ? a.ps : last);
  ntok = hi > lo ? (hi - lo - 1) * a.ps + last : 0;
}

// token_indptr: the exclusive prefix of the batches' token counts, capped at
// num_kv_indices * ps (the size of tok_rows). One workgroup, kScanThreads * kScanPer
// batches per pass, the running total carried between passes.
__global__ __launch_bounds__(kScanThreads) void mla_token_scan_kernel(MlaPagesArgs a) {
  __shared__ long s_wave[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const long cap = (long)a.num_kv_indices * a.ps;
  long carry = 0;
  if (tid == 0) a.tok_indptr[0] = 0;
  for (int c0 = 0; c0 < a.batch; c0 += kScanThreads * kScanPer) {
    int cnt[kScanPer];
    long local = 0;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      const int b = c0 + tid * kScanPer + k;
      int lo, hi, nt = 0;
      if (b < a.batch) batch_pages(a, b, lo, hi, nt);
      cnt[k] = nt;
      local += nt;
    }
    long x = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[w] = x;
    __syncthreads();
    long base = carry, total = carry;
    for (int v = 0; v < kScanThreads / 64; ++v) {
      base += v < w ? s_wave[v] : 0;
      total += s_wave[v];
    }
    long run = base + x - local;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      const int b = c0 + tid * kScanPer + k;
      run += cnt[k];
      if (b < a.batch) a.tok_indptr[b + 1] = (int32_t)(run < cap ? run : cap);
    }
    carry = total;
    __syncthreads();  // s_wave is rewritten by the next pass
  }
}

// One workgroup per batch (grid-stride): the pool row page * ps + slot of each of the
// batch's tokens, written inside [token_indptr[b], token_indptr[b + 1]).
__global__ __launch_bounds__(kExpandThreads) void mla_expand_pages_kernel(MlaPagesArgs a) {
  for (int b = blockIdx.x; b < a.batch; b += gridDim.x) {
    int lo, hi, ntok;
    batch_pages(a, b, lo, hi, ntok);
    const int t0 = a.tok_indptr[b];
    const int n = min(ntok, a.tok_indptr[b + 1] - t0);  // less only where the cap cut it
    for (int j = threadIdx.x; j < n; j += kExpandThreads) {
      const int pg = j / a.ps;
      int page = a.kv_indices[lo + pg];
      page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
      a.tok_rows[t0 + j] = page * a.ps + (j - pg * a.ps);
    }
  }
}

}  // namespace

hipError_t launch_mla_expand_pages(const MlaPagesArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(mla_token_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.batch == 0) return hipSuccess;
  const int grid = a.batch < 4096 ? a.batch : 4096;
  hipLaunchKernelGGL(mla_expand_pages_kernel, dim3(grid), dim3(kExpandThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
