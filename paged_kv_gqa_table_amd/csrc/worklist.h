// Dense work list for split-K decode, built redundantly by every workgroup from seq_lens.
//
// A work item is one (sequence b, kv head, partition p) with p < ceil(len_b / ps_b), where
// ps_b is the fixed partition size or, under the NUM_SPLITS policy, the sequence's own
// page-aligned split size (part_tokens in decode_args.h). Only
// real items are numbered, so a launch maps blockIdx to work without ever visiting an
// empty partition, however skewed the batch. Items are ordered for a short tail:
//   1. every full partition (ps tokens) of every sequence, sequence-major, then kv head,
//      then partition;
//   2. the partial last partitions (len_b % ps != 0), sequence by sequence, kv head minor.
// Workgroups take items in blockIdx order, so the items that start last, after the
// first wave of workgroups drains, are the short ones.
//
// LDS (dynamic, worklist_lds_words(S) ints): s_full[S + 1] holds, per sequence, the
// exclusive prefix of its full items shifted left by one, with bit 0 set when it has a
// partial partition; s_order[S] lists the sequences with a partial partition in the
// order their items are numbered.
#pragma once

#include "common.h"
#include "decode_args.h"

namespace pkv {

constexpr int kMaxDenseSeqs = 4096;
__host__ __device__ inline int worklist_lds_words(int S) { return 2 * S + 1; }

// The list is used when its LDS fits and item counts fit the packed prefix (< 2^30).
inline bool use_dense_worklist(int S, int KVH, int grid_parts) {
  return S <= kMaxDenseSeqs && (long)S * KVH * grid_parts < (1L << 30);
}

struct DenseItems {
  const int* full;   // s_full
  const int* order;  // s_order
  int S, KVH, n_full, n_items;
};

// Builds the list with all NT threads of the block (s_wave: 2 * NT / 64 ints). Ends with a
// barrier. Lengths are clamped into [0, mb_tokens]; partitions are ps tokens, or split per
// sequence when nsplit > 0.
template <int NT>
__device__ DenseItems build_worklist(const int32_t* lens, int S, int mb_tokens, int ps, int nsplit, int KVH,
                                     int* lds, int* s_wave) {
  constexpr int NW = NT / 64;
  int* s_full = lds;
  int* s_order = lds + S + 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int per = (S + NT - 1) / NT;
  const int i0 = tid * per;
  const int i1 = min(i0 + per, S);
  int local_f = 0, local_p = 0;
  for (int i = i0; i < i1; ++i) {
    int len = lens[i];
    len = len < 0 ? 0 : (len > mb_tokens ? mb_tokens : len);
    const int psb = part_tokens(len, ps, nsplit, 16);
    const int nf = len / psb;
    const int rem = len - nf * psb;
    s_full[i] = len;  // this thread's own slots: read back below without a barrier
    local_f += nf * KVH;
    local_p += rem > 0;
  }
  // inclusive scans of both counts inside the wave
  int xf = local_f, xp = local_p;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int yf = __shfl_up(xf, off, 64);
    const int yp = __shfl_up(xp, off, 64);
    if (lane >= off) {
      xf += yf;
      xp += yp;
    }
  }
  if (lane == 63) {
    s_wave[wv] = xf;
    s_wave[NW + wv] = xp;
  }
  __syncthreads();
  int base_f = 0, base_p = 0, n_full = 0, n_pseq = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    base_f += (v < wv) ? s_wave[v] : 0;
    base_p += (v < wv) ? s_wave[NW + v] : 0;
    n_full += s_wave[v];
    n_pseq += s_wave[NW + v];
  }
  int run_f = base_f + xf - local_f;  // exclusive prefixes at this thread's first sequence
  int run_p = base_p + xp - local_p;
  for (int i = i0; i < i1; ++i) {
    const int len = s_full[i];
    const int psb = part_tokens(len, ps, nsplit, 16);
    const int nf = len / psb;
    const bool has_p = len - nf * psb > 0;
    s_full[i] = (run_f << 1) | (has_p ? 1 : 0);
    run_f += nf * KVH;
    if (has_p) s_order[run_p++] = i;
  }
  if (tid == 0) s_full[S] = n_full << 1;
  __syncthreads();
  return DenseItems{s_full, s_order, S, KVH, n_full, n_full + n_pseq * KVH};
}

PKV_DEVICE int full_prefix(const DenseItems& it, int b) { return it.full[b] >> 1; }

// Number of partitions (full and partial) of sequence b.
PKV_DEVICE int seq_parts(const DenseItems& it, int b) {
  return (full_prefix(it, b + 1) - full_prefix(it, b)) / it.KVH + (it.full[b] & 1);
}

// (b, kv head, p) of `item` (uniform across the workgroup).
PKV_DEVICE void decode_item(const DenseItems& it, int item, int& b, int& kvh, int& p) {
  if (item < it.n_full) {
    int lo = 0, hi = it.S;  // full_prefix(lo) <= item < full_prefix(hi)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (full_prefix(it, mid) <= item) lo = mid; else hi = mid;
    }
    const int r = item - full_prefix(it, lo);
    const int nf = (full_prefix(it, lo + 1) - full_prefix(it, lo)) / it.KVH;
    b = lo;
    kvh = r / nf;
    p = r - kvh * nf;
  } else {
    const int r = item - it.n_full;
    const int j = r / it.KVH;
    b = it.order[j];
    b = b < 0 ? 0 : (b >= it.S ? it.S - 1 : b);  // always a valid row, whatever the list holds
    kvh = r - j * it.KVH;
    p = (full_prefix(it, b + 1) - full_prefix(it, b)) / it.KVH;  // the partition after the full ones
  }
}

// The k-th item of workgroup s in a grid of R workgroups, or -1 past its last one. Full
// items go round-robin (s + k R); the partial items then go first to the workgroups that
// got one full item fewer, so that no workgroup carries a whole extra item.
PKV_DEVICE int wg_item(const DenseItems& it, int s, int R, int k) {
  const int F = it.n_full;
  const int nf = s < F ? (F - s + R - 1) / R : 0;  // full items of workgroup s
  if (k < nf) return s + k * R;
  const int first = F % R;  // the first workgroup with one full item fewer
  const int item = F + ((s - first) % R + R) % R + (k - nf) * R;
  return item < it.n_items ? item : -1;
}

// Sentinel m = -inf, l = 0 for every (b, h, p) with ceil(len_b / ps_b) <= p < grid_parts,
// spread over the whole grid (one pass, grid-stride). Nothing when m is null (the final
// mode with a single partition keeps no partials).
PKV_DEVICE void write_sentinels(const DenseItems& it, int H, int grid_parts, int P, float* m, float* l) {
  if (m == nullptr) return;
  const long total = (long)it.S * H * grid_parts;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int p = (int)(idx % grid_parts);
    const long bh = idx / grid_parts;
    const int b = (int)(bh / H);
    if (p >= seq_parts(it, b)) {
      const size_t o = (size_t)bh * P + p;
      m[o] = kNegInf;
      l[o] = 0.f;
    }
  }
}

}  // namespace pkv
