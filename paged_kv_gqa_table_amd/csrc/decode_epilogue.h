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

// Partial rows handed between workgroups of one launch (the one-launch decode) are written
// and read with agent-scope relaxed atomics: on gfx950 these carry the sc1 bit, so a store
// writes through the XCD's own L2 to the point where every XCD sees it and a load does not
// take a stale copy from its L2. That hands over exactly the rows concerned; an agent-scope
// fence instead writes back or invalidates the whole L2 of the XCD it runs on.
template <bool COHERENT>
PKV_DEVICE float ld_f32(const float* p) {
  if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool COHERENT>
PKV_DEVICE void st_f32(float* p, float v) {
  if constexpr (COHERENT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
// A lane's VecT share (4, 8, 16 or 32 bytes) of an acc row; 64-bit words when coherent.
template <bool COHERENT, typename VecT>
PKV_DEVICE VecT ld_vec(const float* p) {
  if constexpr (!COHERENT) {
    return *reinterpret_cast<const VecT*>(p);
  } else if constexpr (sizeof(VecT) == 4) {
    VecT v;
    *reinterpret_cast<float*>(&v) = ld_f32<true>(p);
    return v;
  } else {
    VecT v;
    uint64_t* w = reinterpret_cast<uint64_t*>(&v);
    const uint64_t* src = reinterpret_cast<const uint64_t*>(p);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(VecT) / 8); ++i)
      w[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return v;
  }
}

// One wave combines row `row` (= b * H + h) of the partial arrays (stride P partitions)
// over its first np partitions and writes out[row, :] (and lse[row] when lse is not null).
// Each lane owns D / 64 contiguous output dims, so every acc row is one coalesced read;
// m and l of the first 64 partitions and 8 acc rows go out before anything waits.
// Eight floats (a lane's share of a 512-wide row) as one 32-byte access.
struct alignas(32) Float8 {
  float4 a, b;
};

// lse_scale multiplies the written LSE (1 for natural log, 1 / ln 2 for base 2). COHERENT:
// the partials were written by other workgroups of the same launch (see ld_vec).
template <int D, bool OUT_BF16, bool COHERENT = false>
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
    const float m0 = lane < np ? ld_f32<COHERENT>(mrow + lane) : kNegInf;  // partition `lane`
    const float l0 = lane < np ? ld_f32<COHERENT>(lrow + lane) : 0.f;
    VecT buf[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u)
      if (u < np) buf[u] = ld_vec<COHERENT, VecT>(arow + (size_t)u * D);
    float mv = m0;
    for (int i = lane + 64; i < np; i += 64) mv = fmaxf(mv, ld_f32<COHERENT>(mrow + i));  // more than 64 partitions
    M = uniform(strided_max<1>(mv));
    const float wl = __expf(m0 - M);  // weight of partition `lane` (0 past np)
    const float cl = normalized ? wl * l0 : wl;  // coefficient of acc row `lane`
    float zl = wl * l0;
    for (int i = lane + 64; i < np; i += 64) zl += __expf(ld_f32<COHERENT>(mrow + i) - M) * ld_f32<COHERENT>(lrow + i);
    Z = strided_sum<1>(zl);
    for (int c0 = 0; c0 < np; c0 += CH) {
      if (c0 > 0) {
#pragma unroll
        for (int u = 0; u < CH; ++u)
          if (c0 + u < np) buf[u] = ld_vec<COHERENT, VecT>(arow + (size_t)(c0 + u) * D);
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int pidx = c0 + u;
        if (pidx < np) {
          float cf;
          if (pidx < 64) {
            cf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), pidx));
          } else {
            cf = __expf(ld_f32<COHERENT>(mrow + pidx) - M);
            if (normalized) cf *= ld_f32<COHERENT>(lrow + pidx);
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

// ALiBi bias (Press, Smith and Lewis, "Train Short, Test Long", ICLR 2022): the score of key
// t of a sequence of len tokens gets -slope * (len - 1 - t). Inside a partition the kernels
// add only the partition-relative part -slope * (t_last - t), t_last being the partition's
// last token, which keeps the scores small and their float32 rounding error relative to
// them small; the constant rest, -slope * (len - 1 - t_last), shifts the partition's max
// and nothing else (l and acc are taken relative to that max), so it is added to the
// stored max once. In base-2 units (the kernels' internal scale).
PKV_DEVICE float alibi_shift2(const DecodePartialArgs& a, int h, int len, int t_last) {
  return -a.alibi[h] * kLog2e * (float)(len - 1 - t_last);
}

// Number of partitions of a sequence of len tokens under the launch's partition map.
PKV_DEVICE int item_parts(const DecodePartialArgs& a, int len) {
  const int pt = part_tokens(len, a.ps, a.nsplit, a.bs);
  return (len + pt - 1) / pt;
}

// The result of one merged (head, dim) of an item: o and L relative to the base-2 max M2.
// Writes the final output when the sequence has a single partition and the launch is in
// final mode, else the partial row (acc divided by L when the launch asks for normalized
// partials).
// COHERENT (the one-launch decode): the partial row is written for another workgroup of the
// same launch to combine, with stores every XCD sees (st_f32).
template <int D, bool OUT_BF16, bool COHERENT = false>
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
  st_f32<COHERENT>(a.acc + si * D + d, a.normalize ? o / L : o);
  if (d == 0) {
    st_f32<COHERENT>(a.m + si, M2 * kLn2);
    st_f32<COHERENT>(a.l + si, L);
  }
}

// End of an item in final mode with np > 1 partitions: after every thread's partial
// stores, the workgroup counts itself in counters[b * KVH + kvh]; the workgroup that
// completes the count combines the G rows (one wave per head) and resets the counter.
// Every thread of the workgroup calls this (it holds barriers).
//
// Ordering: the partial rows were stored coherently (store_item_value<.., true>); every wave
// waits until its own stores have completed, which for these stores means they are visible
// to every XCD; the barrier orders all of them before thread 0's count (a device-scope
// atomic, performed where every XCD sees it). The workgroup that completes the count reads
// the rows back with coherent loads, issued only after the count returned. No cache is
// written back or invalidated as a whole (an agent-scope fence pair per item made the
// one-launch decode twice as slow as two launches).
template <int D, bool OUT_BF16, int W>
__device__ void finish_item_fused(const DecodePartialArgs& a, int b, int kvh, int G, int np) {
  __shared__ int s_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial rows are visible device-wide
  __syncthreads();
  int* ctr = a.counters + (size_t)b * a.KVH + kvh;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == np - 1;
  __syncthreads();
  if (s_last) {
    const int w = threadIdx.x >> 6;
    for (int g = w; g < G; g += W)
      reduce_row_wave<D, OUT_BF16, true>(a.acc, a.m, a.l, a.P, np, a.normalize != 0,
                                         (size_t)b * a.H + (size_t)kvh * G + g, a.out, a.lse);
    if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
