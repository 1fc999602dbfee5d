// Split-K paged decode, phase 2: log-sum-exp weighted combine of the partials.
//
// Computes what the flash-decode post's _flash_decode_combine_kernel computes
// (M = max m_p, w_p = exp(m_p - M), out = sum w_p acc_p / sum w_p l_p, zeros for an
// empty sequence), over ceil(len / ps) partitions per sequence as in the PagedAttention
// V2 Triton page's _reduce_partitions_kernel (or the sequence's non-empty NUM_SPLITS
// splits). The optional natural-log LSE M + ln(sum w_p l_p) is written as well. With
// normalized partials (acc_p = acc / l, that page's tmp_output) each row weighs w_p l_p.
//
// Two forms, chosen by the caller's partition bound P:
//  * P <= 16: one wave per (sequence, head) (reduce_row_wave in decode_epilogue.h, shared
//    with the one-launch decode); each lane owns D / 64 contiguous output dims, so every
//    partition row of acc is one coalesced 256 B - 1 KiB read, 8 rows in flight.
//  * P > 16: one workgroup of 4 waves per (sequence, head). A row of more than 8
//    partitions: wave w combines its quarter of them the same way (16 rows in flight),
//    then the four waves' (max, sum, accumulator) merge through LDS with the same
//    weighting, so a sequence of 128 partitions takes two memory round trips instead of
//    sixteen. A row of at most 8 in such a batch takes the one-wave path (one round trip)
//    and the other three waves leave at once. (For batches of short contexts only, the
//    four-fold launch costs more than it saves.)
// Partitions past P_b are never read (their acc rows are not even written by phase 1).
#include <type_traits>

#include "common.h"
#include "decode_args.h"
#include "decode_epilogue.h"

namespace pkv {

// Partitions of sequence b under the launch's partition map (capped at P).
PKV_DEVICE int reduce_parts(const DecodeReduceArgs& a, int b) {
  int len = a.lens[b];
  len = len < 0 ? 0 : len;
  const int pt = part_tokens(len, a.ps, a.nsplit, a.bs);
  const int np = (len + pt - 1) / pt;
  return uniform(np > a.P ? a.P : np);
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeReduceArgs a) {
  const int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6);  // b * H + h
  if (row >= a.S * a.H) return;
  const int np = reduce_parts(a, row / a.H);
  reduce_row_wave<D, OUT_BF16>(a.acc, a.m, a.l, a.P, np, a.normalized != 0, (size_t)row, a.out, a.lse);
}

constexpr int kReduceWaves = 4;
constexpr int kReduceSplitP = 16;  // partition bound above which a row gets 4 waves
constexpr int kReduceOneWaveP = 8;  // rows reduce_row_wave combines in one memory round trip

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(64 * kReduceWaves) void decode_reduce_split_kernel(DecodeReduceArgs a) {
  constexpr int DPL = D / 64;  // output dims per lane
  constexpr int CH = 16;       // partition rows of acc in flight per lane
  __shared__ float s_o[kReduceWaves][D];
  __shared__ float s_m[kReduceWaves], s_z[kReduceWaves];
  const int lane = threadIdx.x & 63;
  const int w = uniform((int)(threadIdx.x >> 6));
  const int row = blockIdx.x;  // b * H + h
  if (row >= a.S * a.H) return;  // uniform over the workgroup
  const int np = reduce_parts(a, row / a.H);
  if (np <= kReduceOneWaveP) {  // a short row: one wave, as in decode_reduce_kernel; the
    if (w == 0)                 // others leave at once and free their slots for other rows
      reduce_row_wave<D, OUT_BF16>(a.acc, a.m, a.l, a.P, np, a.normalized != 0, (size_t)row, a.out, a.lse);
    return;  // uniform over the workgroup: no barrier follows for it
  }
  // this wave's partitions [p0, p1)
  const int per = (np + kReduceWaves - 1) / kReduceWaves;
  const int p0 = min(np, w * per), p1 = min(np, p0 + per);
  const int nw = p1 - p0;

  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = 0.f;
  float M = kNegInf, Z = 0.f;

  if (nw > 0) {
    const float* mrow = a.m + (size_t)row * a.P + p0;
    const float* lrow = a.l + (size_t)row * a.P + p0;
    const float* arow = a.acc + ((size_t)row * a.P + p0) * D + lane * DPL;
    using VecT = typename std::conditional<DPL == 4, float4, typename std::conditional<DPL == 2, float2, float>::type>::type;
    // m, l of the first 64 partitions (one per lane) and the first CH acc rows all go out
    // before anything waits on them: one memory round trip for the common case.
    const float m0 = lane < nw ? mrow[lane] : kNegInf;  // partition p0 + lane
    const float l0 = lane < nw ? lrow[lane] : 0.f;
    VecT buf[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u)
      if (u < nw) buf[u] = *reinterpret_cast<const VecT*>(arow + (size_t)u * D);
    float mv = m0;
    for (int i = lane + 64; i < nw; i += 64) mv = fmaxf(mv, mrow[i]);  // more than 64 partitions
    M = uniform(strided_max<1>(mv));
    const float wl = __expf(m0 - M);  // weight of partition p0 + lane (0 past the range)
    const float cl = a.normalized ? wl * l0 : wl;  // coefficient of acc row p0 + lane
    float zl = wl * l0;
    for (int i = lane + 64; i < nw; i += 64) zl += __expf(mrow[i] - M) * lrow[i];
    Z = strided_sum<1>(zl);
    for (int c0 = 0; c0 < nw; c0 += CH) {
      if (c0 > 0) {
#pragma unroll
        for (int u = 0; u < CH; ++u)
          if (c0 + u < nw) buf[u] = *reinterpret_cast<const VecT*>(arow + (size_t)(c0 + u) * D);
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int pidx = c0 + u;
        if (pidx < nw) {
          float wgt;
          if (pidx < 64) {
            wgt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), pidx));
          } else {
            wgt = __expf(mrow[pidx] - M);
            if (a.normalized) wgt *= lrow[pidx];
          }
          const float* f = reinterpret_cast<const float*>(&buf[u]);
#pragma unroll
          for (int i = 0; i < DPL; ++i) o[i] = fmaf(wgt, f[i], o[i]);
        }
      }
    }
  }
  // ---- merge the waves: out = sum_w e_w o_w / sum_w e_w Z_w with e_w = exp(M_w - max M)
#pragma unroll
  for (int i = 0; i < DPL; ++i) s_o[w][lane * DPL + i] = o[i];
  if (lane == 0) {
    s_m[w] = M;
    s_z[w] = Z;
  }
  __syncthreads();
  float Mt = s_m[0];
#pragma unroll
  for (int v = 1; v < kReduceWaves; ++v) Mt = fmaxf(Mt, s_m[v]);
  float e[kReduceWaves], Zt = 0.f;
#pragma unroll
  for (int v = 0; v < kReduceWaves; ++v) {
    e[v] = s_m[v] == kNegInf ? 0.f : __expf(s_m[v] - Mt);  // a wave with no partitions weighs 0
    Zt = fmaf(e[v], s_z[v], Zt);
  }
  const float inv = np > 0 ? 1.f / Zt : 0.f;
  for (int d = threadIdx.x; d < D; d += 64 * kReduceWaves) {
    float od = 0.f;
#pragma unroll
    for (int v = 0; v < kReduceWaves; ++v) od = fmaf(e[v], s_o[v][d], od);
    od *= inv;
    const size_t ob = (size_t)row * D + d;
    if constexpr (OUT_BF16) {
      reinterpret_cast<uint16_t*>(a.out)[ob] = (uint16_t)f32_to_bf16_bits(od);
    } else {
      reinterpret_cast<float*>(a.out)[ob] = od;
    }
  }
  if (a.lse != nullptr && threadIdx.x == 0) a.lse[row] = (np > 0) ? Mt + __logf(Zt) : kNegInf;
}

template <int D>
static hipError_t launch_reduce_d(const DecodeReduceArgs& a, bool out_bf16, hipStream_t s) {
  const int rows = a.S * a.H;
  if (rows <= 0) return hipSuccess;
  if (a.P > kReduceSplitP) {
    if (out_bf16)
      hipLaunchKernelGGL((decode_reduce_split_kernel<D, true>), dim3(rows), dim3(64 * kReduceWaves), 0, s, a);
    else
      hipLaunchKernelGGL((decode_reduce_split_kernel<D, false>), dim3(rows), dim3(64 * kReduceWaves), 0, s, a);
    return hipGetLastError();
  }
  dim3 grid((rows + 3) / 4);
  if (out_bf16)
    hipLaunchKernelGGL((decode_reduce_kernel<D, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<D, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_reduce(const DecodeReduceArgs& a, bool out_bf16, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_reduce_d<64>(a, out_bf16, s);
    case 128: return launch_reduce_d<128>(a, out_bf16, s);
    case 256: return launch_reduce_d<256>(a, out_bf16, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
