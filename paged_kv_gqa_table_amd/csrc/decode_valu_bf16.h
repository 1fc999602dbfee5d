// Split-K paged decode, phase 1, bf16, vector ALUs (query-head groups G <= 8).
//
// Same computation as decode_valu.h (per-partition m, l and unnormalized acc for the G
// heads of one kv head; PagedAttention V2 Triton page, _partition_attn_kernel, with the
// flash-decode post's unnormalized accumulator), with a layout tuned for bf16:
//  * K and V use different lane layouts. For q.K a token's row is split over 8 lanes (so
//    each score needs only 3 DPP steps); for P.V over 16 lanes in the token-major layout
//    (so each lane owns fewer dims and the accumulator is small), or the linear 16-byte
//    chunk order of the x-packed V layout.
//  * P crosses between the two layouts through a per-wave LDS row of bf16 values, stored
//    in the order each V lane reads them: one 4-, 8- or 16-byte read gives a lane its
//    token pairs, ready for v_dot2c_f32_bf16.
//  * Everything else follows decode_valu.h: dense work list, page ids broadcast with
//    v_readlane, q rows in LDS, single register buffer with early re-issue, wave-uniform
//    running max with lazy re-basing, base-2 exponent, LDS merge of the waves.
#pragma once

#include "common.h"
#include "decode_args.h"
#include "worklist.h"

namespace pkv {

constexpr float kRebaseBf16 = 8.f;  // log2 headroom of the lazy softmax re-basing

template <int D, bool XP>
struct Bf16Cfg {
  static constexpr int BS = 16;
  static constexpr int ROWB = D * 2;                 // bytes of a token row
  static constexpr int NC = ROWB / 16;               // 16-byte chunks per row (8, 16, 32)
  // q.K layout: 8 lanes per token, 2 tokens per lane per page
  static constexpr int KCPL = NC / 8;                // chunks per lane per token
  // P.V layout (token-major): LV lanes per token, VT tokens per lane
  static constexpr int LV = NC >= 16 ? 16 : 8;
  static constexpr int VT = BS * LV / 64;            // 4 or 2
  static constexpr int VCPL = NC / LV;               // chunks per lane per token
  // x-packed V: chunk = one dim x 8 tokens; 2 chunks per dim; NVC chunks per lane
  static constexpr int NVC = D * 2 / 64;
  static constexpr int NACC = XP ? NVC : VCPL * 8;   // accumulator floats per lane per head
  static constexpr int NVREG = XP ? NVC : VT * VCPL;
};

// Position of token t's bf16 P in a wave's LDS row, so that a V lane reads its tokens
// contiguously: token-major 16-lane rows read tokens (r, r+4, r+8, r+12), 8-lane rows
// (r, r+8), x-packed chunks 8 consecutive tokens.
template <int LV, bool XP>
PKV_DEVICE int p_slot(int t) {
  if constexpr (XP) return t;
  else if constexpr (LV == 16) return (t & 3) * 4 + (t >> 2);
  else return (t & 7) * 2 + (t >> 3);
}

template <int W, int G, int D>
struct Bf16Smem {
  __attribute__((aligned(16))) uint32_t q_lds[G][D / 2];   // bf16 query rows
  float red_acc[W][G][D];
  float red_m[W][G];
  float red_mref[W][G];
  float red_l[W][G];
  __attribute__((aligned(16))) uint16_t p_lds[W][G][16];  // bf16 P of the current page
};

template <int D, int G, bool XP, int W>
__device__ __forceinline__ void bf16_partition(const DecodePartialArgs& a, const int b, const int kvh, const int p,
                                               int len, Bf16Smem<W, G, D>& sm) {
  using C = Bf16Cfg<D, XP>;
  constexpr int BS = C::BS, ROWB = C::ROWB, KCPL = C::KCPL, LV = C::LV, VT = C::VT, VCPL = C::VCPL;
  constexpr int NVC = C::NVC, NACC = C::NACC;
  constexpr int PAGEB = BS * ROWB;

  const int lane = threadIdx.x & 63;
  const int w = uniform((int)(threadIdx.x >> 6));
  const int kc = lane & 7;    // q.K: chunk column
  const int kt = lane >> 3;   // q.K: token (and kt + 8)
  const int vc = lane % LV;   // P.V token-major: chunk column
  const int vt = lane / LV;   // P.V token-major: first token
  const int H = a.H;
  const int pg_begin = p * a.ppp;
  const int32_t* bt_row = a.bt + (size_t)b * a.mb;

  // Page ids and the query rows are requested before the length is known (ids only
  // inside the table row; unused ones are never dereferenced), so the item's first
  // memory round trip fetches length, ids and q together.
  int pid_cache = 0;
  auto load_ids = [&](int i0) {  // lane j <- id of this wave's page i0 + j
    const int pg = pg_begin + w + W * (i0 + lane);
    int id = (pg < a.mb && pg < pg_begin + a.ppp) ? bt_row[pg] : 0;
    id = id < 0 ? 0 : id;
    pid_cache = id >= a.NB ? a.NB - 1 : id;
  };
  load_ids(0);
  constexpr int QCH = G * (ROWB / 16);                 // 16-byte chunks of the G query rows
  constexpr int QPT = (QCH + 64 * W - 1) / (64 * W);   // per thread
  uint4 qreg[QPT];
  {
    const char* qb = reinterpret_cast<const char*>(a.q) + ((size_t)b * H + (size_t)kvh * G) * ROWB;
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int i = threadIdx.x + u * 64 * W;
      qreg[u] = i < QCH ? ld16(qb + (size_t)i * 16) : make_uint4(0, 0, 0, 0);
    }
  }
  len = len < 0 ? 0 : (len > a.mb * BS ? a.mb * BS : len);
  len = uniform(len);
  if (p * a.ps >= len) {  // empty partition (PagedAttention V2 page, unused-partition branch)
    if ((int)threadIdx.x < G) {
      const size_t si = ((size_t)b * H + (size_t)kvh * G + threadIdx.x) * a.P + p;
      a.m[si] = kNegInf;
      a.l[si] = 0.f;
    }
    return;  // uniform across the workgroup
  }
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int i = threadIdx.x + u * 64 * W;
    if (i < QCH) *reinterpret_cast<uint4*>(&sm.q_lds[0][0] + i * 4) = qreg[u];
  }
  const int npages_seq = (len + BS - 1) / BS;
  const int pg_end = min(pg_begin + a.ppp, npages_seq);
  const int n_my = pg_end - pg_begin - w > 0 ? (pg_end - pg_begin - w + W - 1) / W : 0;
  __syncthreads();

  float acc[G][NACC];
  float m_ref[G], m_true[G], lsum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_ref[g] = kNegInf;
    m_true[g] = kNegInf;
    lsum[g] = 0.f;
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[g][i] = 0.f;
  }

  const size_t block_stride = (size_t)a.KVH * PAGEB;
  const char* kbase = reinterpret_cast<const char*>(a.kc) + (size_t)kvh * PAGEB;
  const char* vbase = reinterpret_cast<const char*>(a.vc) + (size_t)kvh * PAGEB;
  auto page_ptr = [&](const char* base, int rel) -> const char* {  // rel = index into pid_cache
    const int id = __builtin_amdgcn_readlane(pid_cache, rel & 63);
    return base + (size_t)id * block_stride;
  };
  auto k_off = [&](int t, int cc) -> int {
    if constexpr (XP) return (cc * BS + t) * 16;
    else return t * ROWB + cc * 16;
  };

#ifndef PKV_BF16_DEPTH
#define PKV_BF16_DEPTH 1
#endif
  // DEPTH pages of K and V are in flight per wave: page i's registers are refilled with
  // page i + DEPTH as soon as they are consumed (K after the scores, V after P.V).
  constexpr int DEPTH = PKV_BF16_DEPTH;
  uint4 kr[DEPTH][2][KCPL];
  uint4 vr[DEPTH][C::NVREG];
  int cache_base = 0;  // first page (in this wave's order) whose id is in pid_cache
  auto ensure_ids = [&](int i) {  // uniform; refreshes the lane cache every 64 pages
    if (i >= cache_base + 64) {
      cache_base = i & ~63;
      load_ids(cache_base);
    }
  };
  auto issue_k = [&](int d, int i) {
    const char* kp = page_ptr(kbase, i - cache_base);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int k = 0; k < KCPL; ++k) kr[d][j][k] = ld16(kp + k_off(kt + 8 * j, kc + 8 * k));
  };
  auto issue_v = [&](int d, int i) {
    const char* vp = page_ptr(vbase, i - cache_base);
    if constexpr (XP) {
#pragma unroll
      for (int q = 0; q < NVC; ++q) vr[d][q] = ld16(vp + (size_t)(64 * q + lane) * 16);
    } else {
#pragma unroll
      for (int j = 0; j < VT; ++j)
#pragma unroll
        for (int k = 0; k < VCPL; ++k)
          vr[d][j * VCPL + k] = ld16(vp + (vt + (64 / LV) * j) * ROWB + (vc + LV * k) * 16);
    }
  };

#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (d < n_my) {
      issue_k(d, d);
      issue_v(d, d);
    }
  for (int i0 = 0; i0 < n_my; i0 += DEPTH) {
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    const int i = i0 + d;
    if (i >= n_my) break;
    const int pg = pg_begin + w + W * i;
    const int ntok = min(BS, len - pg * BS);
    // refill target: DEPTH pages ahead, or this page again past the end (an L2 hit; keeps
    // the loads unconditional so the registers need no merge copies)
    const int nx = i + DEPTH < n_my ? i + DEPTH : i;
    ensure_ids(nx);
    // ---- scores of tokens kt and kt + 8, summed over the 8 lanes of a row
    asm volatile("" ::: "memory");  // q is re-read from LDS every page (registers are scarce)
    float s[G][2];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint4 qv[KCPL];
#pragma unroll
      for (int k = 0; k < KCPL; ++k) qv[k] = *reinterpret_cast<const uint4*>(&sm.q_lds[g][(kc + 8 * k) * 4]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int k = 0; k < KCPL; ++k) {
          d0 = dot2_bf16(qv[k].x, kr[d][j][k].x, d0);
          d1 = dot2_bf16(qv[k].y, kr[d][j][k].y, d1);
          d0 = dot2_bf16(qv[k].z, kr[d][j][k].z, d0);
          d1 = dot2_bf16(qv[k].w, kr[d][j][k].w, d1);
        }
        s[g][j] = d0 + d1;
      }
    }
    issue_k(d, nx);

#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float v = group_sum<8>(s[g][j]);
        s[g][j] = (kt + 8 * j < ntok) ? v * a.scale_log2 : kNegInf;
      }

    // ---- softmax: wave-uniform max per head, lazy re-basing (branch-free)
    float pr[G][2];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pm = wave_max_uniform<8>(fmaxf(s[g][0], s[g][1]));
      m_true[g] = fmaxf(m_true[g], pm);
      const float new_ref = (m_true[g] > m_ref[g] + kRebaseBf16) ? m_true[g] : m_ref[g];
      const float alpha = fast_exp2(m_ref[g] - new_ref);  // 0 on the first page, else 1 unless re-based
      m_ref[g] = new_ref;
      lsum[g] *= alpha;
#pragma unroll
      for (int q = 0; q < NACC; ++q) acc[g][q] *= alpha;
      pr[g][0] = fast_exp2(s[g][0] - m_ref[g]);
      pr[g][1] = fast_exp2(s[g][1] - m_ref[g]);
      lsum[g] += pr[g][0] + pr[g][1];
    }

    // ---- P to the wave's LDS row (bf16), in the order the V lanes read it
    if (kc == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t pk = pack_bf16x2(pr[g][0], pr[g][1]);
        sm.p_lds[w][g][p_slot<LV, XP>(kt)] = (uint16_t)(pk & 0xffffu);
        sm.p_lds[w][g][p_slot<LV, XP>(kt + 8)] = (uint16_t)(pk >> 16);
      }
    }
    wave_lds_fence();

    // ---- tail page: zero V of invalid tokens (their slots may hold anything, even NaN)
    if (ntok < BS) {
      if constexpr (XP) {
        const int u = lane & 1;
#pragma unroll
        for (int q = 0; q < NVC; ++q) {
          uint32_t x[4] = {vr[d][q].x, vr[d][q].y, vr[d][q].z, vr[d][q].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 8 * u + 2 * e;
            x[e] = (t >= ntok) ? 0u : (t + 1 >= ntok ? (x[e] & 0xffffu) : x[e]);
          }
          vr[d][q] = make_uint4(x[0], x[1], x[2], x[3]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < VT; ++j)
          if (vt + (64 / LV) * j >= ntok)
#pragma unroll
            for (int k = 0; k < VCPL; ++k) vr[d][j * VCPL + k] = make_uint4(0, 0, 0, 0);
      }
    }

    // ---- P.V
    if constexpr (XP) {
      const int u = lane & 1;  // this lane's chunks hold tokens 8u .. 8u+7
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint4 pp = *reinterpret_cast<const uint4*>(&sm.p_lds[w][g][8 * u]);
#pragma unroll
        for (int q = 0; q < NVC; ++q) {
          float t0 = dot2_bf16(pp.x, vr[d][q].x, acc[g][q]);
          float t1 = dot2_bf16(pp.y, vr[d][q].y, 0.f);
          t0 = dot2_bf16(pp.z, vr[d][q].z, t0);
          t1 = dot2_bf16(pp.w, vr[d][q].w, t1);
          acc[g][q] = t0 + t1;
        }
      }
    } else {
      // token pairs (j, j+1) of this lane: pair their elements and use dot2 over them
      uint32_t pp[G][VT / 2];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if constexpr (VT == 4) {
          const uint2 v2 = *reinterpret_cast<const uint2*>(&sm.p_lds[w][g][4 * vt]);
          pp[g][0] = v2.x;
          pp[g][1] = v2.y;
        } else {
          pp[g][0] = *reinterpret_cast<const uint32_t*>(&sm.p_lds[w][g][2 * vt]);
        }
      }
#pragma unroll
      for (int j = 0; j < VT; j += 2)
#pragma unroll
        for (int k = 0; k < VCPL; ++k) {
          const uint4 va = vr[d][j * VCPL + k], vb = vr[d][(j + 1) * VCPL + k];
          const uint32_t ua[4] = {va.x, va.y, va.z, va.w};
          const uint32_t ub[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = pair_lo(ua[e], ub[e]);
            const uint32_t hi = pair_hi(ua[e], ub[e]);
#pragma unroll
            for (int g = 0; g < G; ++g) {
              acc[g][k * 8 + 2 * e] = dot2_bf16(pp[g][j / 2], lo, acc[g][k * 8 + 2 * e]);
              acc[g][k * 8 + 2 * e + 1] = dot2_bf16(pp[g][j / 2], hi, acc[g][k * 8 + 2 * e + 1]);
            }
          }
        }
    }
    wave_lds_fence();  // this page's P reads finish before the next page overwrites it
    issue_v(d, nx);
  }
  }

  // ---- merge: l over the q.K token groups; acc over the P.V token groups; then waves
#pragma unroll
  for (int g = 0; g < G; ++g) {
    lsum[g] = strided_sum<8>(lsum[g]);
#pragma unroll
    for (int q = 0; q < NACC; ++q) {
      if constexpr (XP) acc[g][q] = group_sum<2>(acc[g][q]);
      else acc[g][q] = strided_sum<LV>(acc[g][q]);
    }
  }
  if constexpr (XP) {
    if ((lane & 1) == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int q = 0; q < NVC; ++q) sm.red_acc[w][g][(64 * q + lane) >> 1] = acc[g][q];
    }
  } else {
    if (vt == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < VCPL; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e) sm.red_acc[w][g][(vc + LV * k) * 8 + e] = acc[g][k * 8 + e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm.red_m[w][g] = m_true[g];
      sm.red_mref[w][g] = m_ref[g];
      sm.red_l[w][g] = lsum[g];
    }
  }
  __syncthreads();

  const size_t stat_base = ((size_t)b * H + (size_t)kvh * G) * a.P + p;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * W) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = sm.red_m[0][g];
#pragma unroll
    for (int v = 1; v < W; ++v) M = fmaxf(M, sm.red_m[v][g]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const float f = fast_exp2(sm.red_mref[v][g] - M);
      o = fmaf(f, sm.red_acc[v][g][d], o);
      L = fmaf(f, sm.red_l[v][g], L);
    }
    const size_t si = stat_base + (size_t)g * a.P;
    a.acc[si * D + d] = o;
    if (d == 0) {
      a.m[si] = M * kLn2;
      a.l[si] = L;
    }
  }
  __syncthreads();
}

// Waves per SIMD the register allocator must leave room for: 4 where the kernel fits in
// 128 VGPRs without spilling, else no constraint.
constexpr int bf16_min_waves(int D, int G) { return (D == 64 && G <= 5) || (D == 128 && G <= 4) ? 4 : 1; }

template <int D, int G, bool XP, int W, bool DENSE>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(bf16_min_waves(D, G), 8))) void decode_partial_bf16_kernel(DecodePartialArgs a, int grid_parts) {
  __shared__ Bf16Smem<W, G, D> sm;
  if constexpr (DENSE) {
    extern __shared__ int s_worklist[];
    __shared__ int s_wave[2 * W];
    const DenseItems it = build_worklist<64 * W>(a.lens, a.S, a.mb * 16, a.ps, a.KVH, s_worklist, s_wave);
    write_sentinels(it, a.H, grid_parts, a.P, a.m, a.l);
    for (int item = blockIdx.x; item < it.n_items; item += gridDim.x) {
      int b, kvh, p;
      decode_item(it, item, b, kvh, p);
      bf16_partition<D, G, XP, W>(a, uniform(b), uniform(kvh), uniform(p), a.lens[b], sm);
    }
  } else {
    // direct map, partition-major: workgroup i handles partition i / (S * KVH) of
    // (sequence, kv head) i % (S * KVH). Empty partitions sit at high partition indices,
    // so they are dispatched last. The length load goes out with the item's other first
    // loads; the empty-partition check comes after them.
    const int sk = a.S * a.KVH;
    const int p = blockIdx.x / sk;
    const int r = blockIdx.x - p * sk;
    const int b = r / a.KVH;
    bf16_partition<D, G, XP, W>(a, uniform(b), uniform(r - b * a.KVH), uniform(p), a.lens[b], sm);
  }
}

#ifndef PKV_BF16_WAVES
#define PKV_BF16_WAVES 4
#endif
#ifndef PKV_DENSE_RATIO
#define PKV_DENSE_RATIO 0
#endif
template <bool XP, int D, int G>
hipError_t launch_bf16_one(const DecodePartialArgs& a, int grid_parts, hipStream_t s) {
  constexpr int W = PKV_BF16_WAVES;
  const long upper = (long)a.S * a.KVH * grid_parts;
  // The dense work list costs one extra memory round trip per workgroup but keeps every
  // workgroup busy and balanced; on MI355X it was faster than the plain partition grid even
  // for uniform lengths, so the plain grid (ratio > 0) is kept only for very large batches.
  if (use_dense_worklist(a.S, a.KVH, grid_parts) && upper > (long)PKV_DENSE_RATIO * dense_grid_cap() / 4) {
    const int grid = (int)(upper < dense_grid_cap() ? upper : dense_grid_cap());
    hipLaunchKernelGGL((decode_partial_bf16_kernel<D, G, XP, W, true>), dim3(grid), dim3(64 * W),
                       worklist_lds_words(a.S) * sizeof(int), s, a, grid_parts);
  } else {
    hipLaunchKernelGGL((decode_partial_bf16_kernel<D, G, XP, W, false>), dim3((unsigned)upper), dim3(64 * W), 0, s,
                       a, grid_parts);
  }
  return hipGetLastError();
}

template <bool XP, int D>
hipError_t launch_bf16_d(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  switch (G) {
    case 1: return launch_bf16_one<XP, D, 1>(a, grid_parts, s);
    case 2: return launch_bf16_one<XP, D, 2>(a, grid_parts, s);
    case 3: return launch_bf16_one<XP, D, 3>(a, grid_parts, s);
    case 4: return launch_bf16_one<XP, D, 4>(a, grid_parts, s);
    case 5: return launch_bf16_one<XP, D, 5>(a, grid_parts, s);
    case 6: return launch_bf16_one<XP, D, 6>(a, grid_parts, s);
    case 7: return launch_bf16_one<XP, D, 7>(a, grid_parts, s);
    case 8: return launch_bf16_one<XP, D, 8>(a, grid_parts, s);
    default: return hipErrorNotSupported;
  }
}

template <bool XP>
hipError_t launch_bf16(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_bf16_d<XP, 64>(a, G, grid_parts, s);
    case 128: return launch_bf16_d<XP, 128>(a, G, grid_parts, s);
    case 256: return launch_bf16_d<XP, 256>(a, G, grid_parts, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace pkv
