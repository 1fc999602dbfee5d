// Dense work list for split-K decode, built redundantly by every workgroup from seq_lens.
//
// A work item is one (sequence b, kv head, partition p) with p < ceil(len_b / ps). Items of
// sequence b are numbered prefix[b] .. prefix[b+1]-1 (kv head major, partition minor), so
// a launch can map blockIdx to real work only: workgroups never spin on empty partitions,
// however skewed the batch. The prefix sums live in LDS; sequences past kMaxDenseSeqs use
// the plain (partition, kv head, sequence) grid instead.
#pragma once

#include "common.h"

namespace pkv {

constexpr int kMaxDenseSeqs = 4096;

// Partitions of one sequence, with its length clamped into [0, mb * 16].
PKV_DEVICE int partitions_of(int len, int mb_tokens, int ps) {
  len = len < 0 ? 0 : (len > mb_tokens ? mb_tokens : len);
  return (len + ps - 1) / ps;
}

// Builds s_prefix[0..S] (exclusive prefix of items per sequence) with all NT threads of
// the block; returns the total number of items. Ends with a barrier.
template <int NT>
__device__ int build_worklist(const int32_t* lens, int S, int mb_tokens, int ps, int KVH, int* s_prefix,
                              int* s_wave) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int per = (S + NT - 1) / NT;
  const int i0 = tid * per;
  int local = 0;
  for (int i = i0; i < i0 + per && i < S; ++i) local += partitions_of(lens[i], mb_tokens, ps) * KVH;
  // inclusive scan of `local` inside the wave
  int x = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wv] = x;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) base += (v < wv) ? s_wave[v] : 0;
  int run = base + x - local;  // exclusive prefix of this thread's first sequence
  for (int i = i0; i < i0 + per && i < S; ++i) {
    s_prefix[i] = run;
    run += partitions_of(lens[i], mb_tokens, ps) * KVH;
  }
  int total = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) total += s_wave[v];
  if (tid == 0) s_prefix[S] = total;
  __syncthreads();
  return total;
}

// Sequence owning `item`: the largest b with s_prefix[b] <= item (uniform search).
PKV_DEVICE int find_seq(const int* s_prefix, int S, int item) {
  int lo = 0, hi = S;  // s_prefix[lo] <= item < s_prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_prefix[mid] <= item) lo = mid; else hi = mid;
  }
  return lo;
}

// Sentinel m = -inf, l = 0 for every (b, h, p) with ceil(len_b / ps) <= p < grid_parts,
// spread over the whole grid (one pass, grid-stride).
PKV_DEVICE void write_sentinels(const int* s_prefix, int S, int H, int KVH, int grid_parts, int P,
                                float* m, float* l) {
  const long total = (long)S * H * grid_parts;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int p = (int)(idx % grid_parts);
    const long bh = idx / grid_parts;
    const int b = (int)(bh / H);
    const int nparts = (s_prefix[b + 1] - s_prefix[b]) / KVH;
    if (p >= nparts) {
      const size_t o = (size_t)bh * P + p;
      m[o] = kNegInf;
      l[o] = 0.f;
    }
  }
}

}  // namespace pkv
