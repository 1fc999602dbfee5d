// Split-K decode: the cross-partition combine of one (sequence, head) row by one wave, and
// the end-of-item pieces that let phase 1 produce the final output in the same launch.
//
// The combine is the flash-decode post's _flash_decode_combine_kernel (M = max m_p,
// w_p = exp(m_p - M), out = sum w_p acc_p / sum w_p l_p) over the P_b partitions of the
// sequence (PagedAttention V2 page, _reduce_partitions_kernel: partitions past P_b are
// never read), plus the natural-log LSE M + ln(sum w_p l_p). With normalized partials
// (acc_p already divided by l_p, the PagedAttention V2 page's tmp_output) each row
// weighs w_p l_p instead.
#pragma once

#include <type_traits>

#include "common.h"
#include "decode_args.h"
#include "worklist.h"

namespace pkv {

// One wave combines row `row` (= b * H + h) of the partial arrays (stride P partitions)
// over its first np partitions and writes out[row, :] (and lse[row] when lse is not null).
// Each lane owns D / 64 contiguous output dims, so every acc row is one coalesced read;
// m and l of the first 64 partitions and 8 acc rows go out before anything waits.
// Eight floats (a lane's share of a 512-wide row) as one 32-byte access.
struct alignas(32) Float8 {
  float4 a, b;
};

// lse_scale multiplies the written LSE (1 for natural log, 1 / ln 2 for base 2).
template <int D, bool OUT_BF16>
PKV_DEVICE void reduce_row_wave(const float* acc, const float* pm, const float* pl, int P, int np,
                                bool normalized, size_t row, void* out, float* lse, float lse_scale = 1.f) {
  constexpr int DPL = D / 64;  // output dims per lane
  constexpr int CH = 8;        // partition rows of acc in flight per lane
  const int lane = threadIdx.x & 63;
  np = uniform(np > P ? P : np);
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = 0.f;
  float M = kNegInf, Z = 0.f;

  if (np > 0) {
    const float* mrow = pm + row * P;
    const float* lrow = pl + row * P;
    const float* arow = acc + row * P * D + lane * DPL;
    using VecT = typename std::conditional<
        DPL == 8, Float8,
        typename std::conditional<DPL == 4, float4, typename std::conditional<DPL == 2, float2, float>::type>::type>::type;
    const float m0 = lane < np ? mrow[lane] : kNegInf;  // partition `lane`
    const float l0 = lane < np ? lrow[lane] : 0.f;
    VecT buf[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u)
      if (u < np) buf[u] = *reinterpret_cast<const VecT*>(arow + (size_t)u * D);
    float mv = m0;
    for (int i = lane + 64; i < np; i += 64) mv = fmaxf(mv, mrow[i]);  // more than 64 partitions
    M = uniform(strided_max<1>(mv));
    const float wl = __expf(m0 - M);  // weight of partition `lane` (0 past np)
    const float cl = normalized ? wl * l0 : wl;  // coefficient of acc row `lane`
    float zl = wl * l0;
    for (int i = lane + 64; i < np; i += 64) zl += __expf(mrow[i] - M) * lrow[i];
    Z = strided_sum<1>(zl);
    for (int c0 = 0; c0 < np; c0 += CH) {
      if (c0 > 0) {
#pragma unroll
        for (int u = 0; u < CH; ++u)
          if (c0 + u < np) buf[u] = *reinterpret_cast<const VecT*>(arow + (size_t)(c0 + u) * D);
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int pidx = c0 + u;
        if (pidx < np) {
          float cf;
          if (pidx < 64) {
            cf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), pidx));
          } else {
            cf = __expf(mrow[pidx] - M);
            if (normalized) cf *= lrow[pidx];
          }
          const float* f = reinterpret_cast<const float*>(&buf[u]);
#pragma unroll
          for (int i = 0; i < DPL; ++i) o[i] = fmaf(cf, f[i], o[i]);
        }
      }
    }
    const float inv = 1.f / Z;
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] *= inv;
  }

  const size_t ob = row * D + lane * DPL;
  if constexpr (OUT_BF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(out) + ob;
    if constexpr (DPL == 8) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                                  pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
    } else if constexpr (DPL == 4) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    } else if constexpr (DPL == 2) {
      *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(o[0], o[1]);
    } else {
      dst[0] = (uint16_t)f32_to_bf16_bits(o[0]);
    }
  } else {
    float* dst = reinterpret_cast<float*>(out) + ob;
#pragma unroll
    for (int i = 0; i < DPL; ++i) dst[i] = o[i];
  }
  if (lse != nullptr && lane == 0) lse[row] = (np > 0) ? (M + __logf(Z)) * lse_scale : kNegInf;
}

// Number of partitions of a sequence of len tokens under the launch's partition map.
PKV_DEVICE int item_parts(const DecodePartialArgs& a, int len) {
  const int pt = part_tokens(len, a.ps, a.nsplit, 16);
  return (len + pt - 1) / pt;
}

// The result of one merged (head, dim) of an item: o and L relative to the base-2 max M2.
// Writes the final output when the sequence has a single partition and the launch is in
// final mode, else the partial row (acc divided by L when the launch asks for normalized
// partials).
template <int D, bool OUT_BF16>
PKV_DEVICE void store_item_value(const DecodePartialArgs& a, size_t bh, int p, int d, float o, float M2, float L,
                                 bool single) {
  if (single) {
    const float v = o / L;
    if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(a.out)[bh * D + d] = (uint16_t)f32_to_bf16_bits(v);
    else reinterpret_cast<float*>(a.out)[bh * D + d] = v;
    if (d == 0 && a.lse != nullptr) a.lse[bh] = M2 * kLn2 + __logf(L);
    return;
  }
  const size_t si = bh * a.P + p;
  a.acc[si * D + d] = a.normalize ? o / L : o;
  if (d == 0) {
    a.m[si] = M2 * kLn2;
    a.l[si] = L;
  }
}

// End of an item in final mode with np > 1 partitions: after every thread's partial
// stores, the workgroup counts itself in counters[b * KVH + kvh]; the workgroup that
// completes the count combines the G rows (one wave per head) and resets the counter.
// Every thread of the workgroup calls this (it holds barriers).
//
// Ordering, with the fewest cache operations (each XCD has its own L2, not coherent with
// the others'): every wave waits until its own partial stores have reached L2, the
// barrier then orders all of them before thread 0's agent-scope release fence (which writes
// the L2 back) and its relaxed count; the combining workgroup's thread 0 takes an
// agent-scope acquire fence (which invalidates the stale cached copies) before a barrier
// lets its waves read. One release per item and one acquire per (sequence, kv head); a
// fence in every thread instead made the one-launch decode five times slower.
template <int D, bool OUT_BF16, int W>
__device__ void finish_item_fused(const DecodePartialArgs& a, int b, int kvh, int G, int np) {
  __shared__ int s_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial rows are in L2
  __syncthreads();
  int* ctr = a.counters + (size_t)b * a.KVH + kvh;
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    s_last = atomicAdd(ctr, 1) == np - 1;
  }
  __syncthreads();
  if (s_last) {
    if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();
    const int w = threadIdx.x >> 6;
    for (int g = w; g < G; g += W)
      reduce_row_wave<D, OUT_BF16>(a.acc, a.m, a.l, a.P, np, a.normalize != 0,
                                   (size_t)b * a.H + (size_t)kvh * G + g, a.out, a.lse);
    if (threadIdx.x == 0) atomicExch(ctr, 0);
  }
  __syncthreads();  // s_last is read before any later item's count overwrites it
}

// Final mode: out = 0 and lse = -inf for every sequence without partitions (len_b = 0),
// grid-stride over the whole launch.
template <int D, bool OUT_BF16>
PKV_DEVICE void write_empty_outputs(const DenseItems& it, const DecodePartialArgs& a) {
  const long total = (long)a.S * a.H * D;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const long bh = idx / D;
    const int b = (int)(bh / a.H);
    if (seq_parts(it, b) == 0) {
      if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(a.out)[idx] = 0;
      else reinterpret_cast<float*>(a.out)[idx] = 0.f;
      if (a.lse != nullptr && idx % D == 0) a.lse[bh] = kNegInf;
    }
  }
}

// Final mode on the plain (b, kvh, p) grid: the workgroup of partition 0 of an empty
// sequence writes its G rows of zeros and -inf.
template <int D, bool OUT_BF16>
PKV_DEVICE void write_empty_rows(const DecodePartialArgs& a, int b, int kvh, int G) {
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const size_t bh = (size_t)b * a.H + (size_t)kvh * G + idx / D;
    const int d = idx % D;
    if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(a.out)[bh * D + d] = 0;
    else reinterpret_cast<float*>(a.out)[bh * D + d] = 0.f;
    if (a.lse != nullptr && d == 0) a.lse[bh] = kNegInf;
  }
}

}  // namespace pkv
