// Split-K paged decode, phase 1, on the vector ALUs (query-head groups G <= 8).
//
// What it computes is the per-partition online softmax of the PagedAttention V2 Triton
// page (_partition_attn_kernel) with the unnormalized accumulator of the flash-decode
// post (_flash_decode_partial_kernel): for one (sequence b, kv head, partition p) it
// produces, for each of the G query heads of that kv head, m = max score, l = sum of
// exp(score - m) and acc = sum of exp(score - m) * V over the partition's tokens.
//
// gfx950 design (not the pages'):
//  * One workgroup per (partition, kv head, sequence), W waves. Each page of 16 tokens
//    is read from HBM exactly once and used for all G heads. Waves take the partition's
//    pages round-robin and keep independent softmax states, merged once through LDS.
//  * K is read straight into registers with 16-byte loads. A token's row is split over
//    LPT lanes (LPT * 16 B >= 128 B, so every load instruction consumes whole 128-byte
//    lines in both layouts). Scores are reduced across those LPT lanes with DPP.
//  * The running max is wave-uniform per head (readfirstlane), so the rescale of l and
//    acc is a scalar branch that is skipped whenever a page does not raise the max.
//  * Scores live in base 2 (scale * log2 e folded once) so exp is a single v_exp_f32;
//    the stored m is converted back to natural-log units.
//  * bf16: q.K uses v_dot2c_f32_bf16 on raw bf16 pairs (no unpacking); P.V uses the same
//    instruction on P rounded to bf16 (as both decode pages do before their P.V product).
//    f32: plain FMAs, P stays f32.
//  * Token-major V has the same lane layout as K, so P never leaves the lane. x-packed V
//    ([D, 16] per page) is read linearly (lane i takes 16-byte chunk i, i.e. one d and
//    8 (bf16) or 4 (f32) consecutive tokens) and P reaches it through a small per-wave
//    LDS row.
//  * Page ids of a partition are cached one per lane and broadcast with readlane.
//  * Single register buffer with early re-issue: the next page's K loads go out as soon
//    as the current scores are formed, its V loads as soon as P.V is done.
#pragma once

#include "common.h"
#include "decode_args.h"

namespace pkv {

template <bool BF16, int D, int G, bool XP, int LPT, int W>
__global__ __launch_bounds__(64 * W) void decode_partial_valu_kernel(DecodePartialArgs a) {
  constexpr int BS = 16;
  constexpr int E = BF16 ? 8 : 4;      // elements per 16-byte chunk
  constexpr int EB = BF16 ? 2 : 4;     // bytes per element
  constexpr int ROWB = D * EB;         // bytes of one token's K (or V) row
  constexpr int NC = ROWB / 16;        // chunks per token row
  constexpr int CPL = NC / LPT;        // chunks per lane per token
  constexpr int TPI = 64 / LPT;        // tokens covered by one load instruction
  constexpr int TPL = BS / TPI;        // tokens per lane per page
  constexpr int PAGEB = BS * ROWB;     // bytes of one (page, kv head) block of K (or V)
  // x-packed V: [D][16] per page; 16-byte chunk = one d, TPC consecutive tokens.
  constexpr int TPC = 16 / EB;         // tokens per V chunk
  constexpr int CPD = BS / TPC;        // chunks per d
  constexpr int NVC = D * CPD / 64;    // V chunks per lane per page (x-packed)
  static_assert(NC % LPT == 0 && CPL >= 1, "row must split evenly over LPT lanes");
  static_assert(TPL >= 1 && (!BF16 || XP || TPL % 2 == 0), "token pairs for bf16 P.V");
  static_assert(!XP || NVC >= 1, "x-packed V needs at least one chunk per lane");

  __shared__ float red_acc[W][G][D];
  __shared__ float red_m[W][G];
  __shared__ float red_l[W][G];
  __shared__ __attribute__((aligned(16))) float p_lds[XP ? W : 1][G][BS];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int c = lane % LPT;   // chunk column of the token row
  const int tg = lane / LPT;  // token group (token index within a load row)

  const int p = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int H = a.H;

  int len = a.lens[b];
  len = len < 0 ? 0 : len;
  len = len > a.mb * BS ? a.mb * BS : len;
  const int tok0 = p * a.ps;
  const size_t stat_base = ((size_t)b * H + (size_t)kvh * G) * a.P + p;  // + g * P

  if (tok0 >= len) {  // empty partition: sentinel (PagedAttention V2, unused-partition branch)
    if (threadIdx.x < G) {
      a.m[stat_base + (size_t)threadIdx.x * a.P] = kNegInf;
      a.l[stat_base + (size_t)threadIdx.x * a.P] = 0.f;
    }
    return;
  }

  const int npages_seq = (len + BS - 1) / BS;
  const int pg_begin = p * a.ppp;
  const int pg_end = min(pg_begin + a.ppp, npages_seq);
  const int32_t* bt_row = a.bt + (size_t)b * a.mb;

  // Page ids of this partition, one per lane (the common case ps <= 1024 tokens).
  int pid_cache = 0;
  if (pg_begin + lane < pg_end) pid_cache = bt_row[pg_begin + lane];
  auto page_id = [&](int pg) -> int {
    int rel = pg - pg_begin;
    int id = rel < 64 ? __builtin_amdgcn_readlane(pid_cache, rel) : bt_row[pg];
    id = id < 0 ? 0 : id;
    return id >= a.NB ? a.NB - 1 : id;
  };

  // ---- query registers: lane holds dims of chunk columns c + LPT*k
  uint32_t qv[G][CPL][4];
  {
    const char* qb = reinterpret_cast<const char*>(a.q) + ((size_t)b * H + (size_t)kvh * G) * ROWB;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        uint4 v = ld16(qb + (size_t)g * ROWB + (c + LPT * k) * 16);
        qv[g][k][0] = v.x; qv[g][k][1] = v.y; qv[g][k][2] = v.z; qv[g][k][3] = v.w;
      }
  }

  constexpr int NACC = XP ? NVC : CPL * E;  // accumulator floats per lane per head
  float acc[G][NACC];
  float m2[G], lsum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m2[g] = kNegInf;
    lsum[g] = 0.f;
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[g][i] = 0.f;
  }

  const size_t head_off = (size_t)kvh * PAGEB;
  const size_t block_stride = (size_t)a.KVH * PAGEB;
  const char* kbase = reinterpret_cast<const char*>(a.kc) + head_off;
  const char* vbase = reinterpret_cast<const char*>(a.vc) + head_off;

  // Byte offset of (token-in-page t, chunk column cc) inside a (page, head) K block.
  auto k_off = [&](int t, int cc) -> int {
    if constexpr (XP) return (cc * BS + t) * 16;   // [D/x][16][x]
    else return t * ROWB + cc * 16;                // [16][D]
  };

  constexpr int NVREG = XP ? NVC : TPL * CPL;
  uint4 kr[TPL][CPL];
  uint4 vr[NVREG];

  auto issue_k = [&](int pg) {
    const char* kp = kbase + (size_t)page_id(pg) * block_stride;
#pragma unroll
    for (int j = 0; j < TPL; ++j)
#pragma unroll
      for (int k = 0; k < CPL; ++k) kr[j][k] = ld16(kp + k_off(tg + TPI * j, c + LPT * k));
  };
  auto issue_v = [&](int pg) {
    const char* vp = vbase + (size_t)page_id(pg) * block_stride;
    if constexpr (XP) {
#pragma unroll
      for (int i = 0; i < NVC; ++i) vr[i] = ld16(vp + (size_t)(64 * i + lane) * 16);
    } else {
#pragma unroll
      for (int j = 0; j < TPL; ++j)
#pragma unroll
        for (int k = 0; k < CPL; ++k) vr[j * CPL + k] = ld16(vp + k_off(tg + TPI * j, c + LPT * k));
    }
  };

  int pg = pg_begin + w;
  if (pg < pg_end) {
    issue_k(pg);
    issue_v(pg);
  }
  while (pg < pg_end) {
    const int nxt = pg + W;
    const int ntok = min(BS, len - pg * BS);  // valid tokens in this page

    // ---- scores s[g][j] for this lane's tokens, summed over the LPT lanes of the row
    float s[G][TPL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          const uint4 kv = kr[j][k];
          if constexpr (BF16) {
            d0 = dot2_bf16(qv[g][k][0], kv.x, d0);
            d1 = dot2_bf16(qv[g][k][1], kv.y, d1);
            d0 = dot2_bf16(qv[g][k][2], kv.z, d0);
            d1 = dot2_bf16(qv[g][k][3], kv.w, d1);
          } else {
            d0 = fmaf(__uint_as_float(qv[g][k][0]), __uint_as_float(kv.x), d0);
            d1 = fmaf(__uint_as_float(qv[g][k][1]), __uint_as_float(kv.y), d1);
            d0 = fmaf(__uint_as_float(qv[g][k][2]), __uint_as_float(kv.z), d0);
            d1 = fmaf(__uint_as_float(qv[g][k][3]), __uint_as_float(kv.w), d1);
          }
        }
        s[g][j] = d0 + d1;
      }
    if (nxt < pg_end) issue_k(nxt);  // K registers are free again

#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        const float v = group_sum<LPT>(s[g][j]);
        s[g][j] = (tg + TPI * j < ntok) ? v * a.scale_log2 : kNegInf;
      }

    // ---- online softmax with a wave-uniform running max per head
    float pr[G][TPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float pm = s[g][0];
#pragma unroll
      for (int j = 1; j < TPL; ++j) pm = fmaxf(pm, s[g][j]);
      pm = uniform(strided_max<LPT>(pm));
      if (pm > m2[g]) {  // uniform branch: only when this page raises the max
        const float alpha = fast_exp2(m2[g] - pm);
        lsum[g] *= alpha;
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[g][i] *= alpha;
        m2[g] = pm;
      }
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        pr[g][j] = fast_exp2(s[g][j] - m2[g]);
        ps += pr[g][j];
      }
      lsum[g] += ps;
    }

    // ---- tail page: zero V of invalid tokens (their slots may hold anything, even NaN)
    const bool tail = ntok < BS;

    if constexpr (!XP) {
      if (tail) {
#pragma unroll
        for (int j = 0; j < TPL; ++j)
          if (tg + TPI * j >= ntok)
#pragma unroll
            for (int k = 0; k < CPL; ++k) vr[j * CPL + k] = make_uint4(0, 0, 0, 0);
      }
      if constexpr (BF16) {
        // token pairs (j, j+1): pair elements of the two tokens and use dot2 over them
#pragma unroll
        for (int j = 0; j < TPL; j += 2) {
          uint32_t pp[G];
#pragma unroll
          for (int g = 0; g < G; ++g) pp[g] = pack_bf16x2(pr[g][j], pr[g][j + 1]);
#pragma unroll
          for (int k = 0; k < CPL; ++k) {
            const uint4 va = vr[j * CPL + k], vb = vr[(j + 1) * CPL + k];
            const uint32_t ua[4] = {va.x, va.y, va.z, va.w};
            const uint32_t ub[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t lo = pair_lo(ua[e], ub[e]);
              const uint32_t hi = pair_hi(ua[e], ub[e]);
#pragma unroll
              for (int g = 0; g < G; ++g) {
                acc[g][k * E + 2 * e] = dot2_bf16(pp[g], lo, acc[g][k * E + 2 * e]);
                acc[g][k * E + 2 * e + 1] = dot2_bf16(pp[g], hi, acc[g][k * E + 2 * e + 1]);
              }
            }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < TPL; ++j)
#pragma unroll
          for (int k = 0; k < CPL; ++k) {
            const uint4 v = vr[j * CPL + k];
            const float f[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                                __uint_as_float(v.w)};
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int g = 0; g < G; ++g) acc[g][k * E + e] = fmaf(pr[g][j], f[e], acc[g][k * E + e]);
          }
      }
    } else {
      // publish P to the wave's LDS row: p_lds[w][g][token]
      if (c == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int j = 0; j < TPL; ++j) p_lds[w][g][tg + TPI * j] = pr[g][j];
      }
      wave_lds_fence();
      const int u = lane % CPD;  // which TPC-token slice of the page this lane's chunks hold
      if (tail) {
#pragma unroll
        for (int i = 0; i < NVC; ++i) {
          uint32_t x[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (BF16) {
              const int t = u * TPC + 2 * e;
              x[e] = (t >= ntok) ? 0u : (t + 1 >= ntok ? (x[e] & 0xffffu) : x[e]);
            } else {
              const int t = u * TPC + e;
              x[e] = (t >= ntok) ? 0u : x[e];
            }
          }
          vr[i] = make_uint4(x[0], x[1], x[2], x[3]);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float4 pf = *reinterpret_cast<const float4*>(&p_lds[w][g][u * TPC]);
        if constexpr (BF16) {
          const float4 pf2 = *reinterpret_cast<const float4*>(&p_lds[w][g][u * TPC + 4]);
          const uint32_t p01 = pack_bf16x2(pf.x, pf.y), p23 = pack_bf16x2(pf.z, pf.w);
          const uint32_t p45 = pack_bf16x2(pf2.x, pf2.y), p67 = pack_bf16x2(pf2.z, pf2.w);
#pragma unroll
          for (int i = 0; i < NVC; ++i) {
            float t0 = dot2_bf16(p01, vr[i].x, acc[g][i]);
            float t1 = dot2_bf16(p23, vr[i].y, 0.f);
            t0 = dot2_bf16(p45, vr[i].z, t0);
            t1 = dot2_bf16(p67, vr[i].w, t1);
            acc[g][i] = t0 + t1;
          }
        } else {
#pragma unroll
          for (int i = 0; i < NVC; ++i) {
            float t = acc[g][i];
            t = fmaf(pf.x, __uint_as_float(vr[i].x), t);
            t = fmaf(pf.y, __uint_as_float(vr[i].y), t);
            t = fmaf(pf.z, __uint_as_float(vr[i].z), t);
            t = fmaf(pf.w, __uint_as_float(vr[i].w), t);
            acc[g][i] = t;
          }
        }
      }
      wave_lds_fence();  // reads of this page's P finish before the next page overwrites it
    }
    if (nxt < pg_end) issue_v(nxt);  // V registers are free again
    pg = nxt;
  }

  // ---- merge this wave's lanes, then the waves, through LDS
#pragma unroll
  for (int g = 0; g < G; ++g) {
    lsum[g] = strided_sum<LPT>(lsum[g]);  // over token groups (lanes of a group agree)
    if constexpr (XP) {
#pragma unroll
      for (int i = 0; i < NVC; ++i) acc[g][i] = group_sum<CPD>(acc[g][i]);
    } else {
#pragma unroll
      for (int i = 0; i < NACC; ++i) acc[g][i] = strided_sum<LPT>(acc[g][i]);
    }
  }
  if constexpr (XP) {
    if (lane % CPD == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < NVC; ++i) red_acc[w][g][(64 * i + lane) / CPD] = acc[g][i];
    }
  } else {
    if (tg == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < CPL; ++k)
#pragma unroll
          for (int e = 0; e < E; ++e) red_acc[w][g][(c + LPT * k) * E + e] = acc[g][k * E + e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      red_m[w][g] = m2[g];
      red_l[w][g] = lsum[g];
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += 64 * W) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = red_m[0][g];
#pragma unroll
    for (int v = 1; v < W; ++v) M = fmaxf(M, red_m[v][g]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const float f = fast_exp2(red_m[v][g] - M);  // waves without pages carry -inf: f = 0
      o = fmaf(f, red_acc[v][g][d], o);
      L = fmaf(f, red_l[v][g], L);
    }
    const size_t si = stat_base + (size_t)g * a.P;
    a.acc[si * D + d] = o;
    if (d == 0) {
      a.m[si] = M * kLn2;
      a.l[si] = L;
    }
  }
}

// Instantiation helper: picks LPT / W for a (dtype, D) pair and launches.
template <bool BF16, bool XP, int D, int G>
hipError_t launch_valu_one(const DecodePartialArgs& a, int grid_parts, hipStream_t s) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int LPT = (D * EB >= 512) ? 16 : 8;
  constexpr int W = 4;
  dim3 grid(grid_parts, a.KVH, a.S);
  hipLaunchKernelGGL((decode_partial_valu_kernel<BF16, D, G, XP, LPT, W>), grid, dim3(64 * W), 0, s, a);
  return hipGetLastError();
}

template <bool BF16, bool XP, int D>
hipError_t launch_valu_d(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  switch (G) {
    case 1: return launch_valu_one<BF16, XP, D, 1>(a, grid_parts, s);
    case 2: return launch_valu_one<BF16, XP, D, 2>(a, grid_parts, s);
    case 3: return launch_valu_one<BF16, XP, D, 3>(a, grid_parts, s);
    case 4: return launch_valu_one<BF16, XP, D, 4>(a, grid_parts, s);
    case 5: return launch_valu_one<BF16, XP, D, 5>(a, grid_parts, s);
    case 6: return launch_valu_one<BF16, XP, D, 6>(a, grid_parts, s);
    case 7: return launch_valu_one<BF16, XP, D, 7>(a, grid_parts, s);
    case 8: return launch_valu_one<BF16, XP, D, 8>(a, grid_parts, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16, bool XP>
hipError_t launch_valu(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_valu_d<BF16, XP, 64>(a, G, grid_parts, s);
    case 128: return launch_valu_d<BF16, XP, 128>(a, G, grid_parts, s);
    case 256:
      if constexpr (BF16) return launch_valu_d<BF16, XP, 256>(a, G, grid_parts, s);
      else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
