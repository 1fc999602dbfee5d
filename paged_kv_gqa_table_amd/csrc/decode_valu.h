// Split-K paged decode, phase 1, float32, on the vector ALUs (query-head groups G <= 16).
//
// What it computes is the per-partition online softmax of the PagedAttention V2 Triton
// page (_partition_attn_kernel) with the unnormalized accumulator of the flash-decode
// post (_flash_decode_partial_kernel): for one (sequence b, kv head, partition p) it
// produces, for each of the G query heads of that kv head, m = max score, l = sum of
// exp(score - m) and acc = sum of exp(score - m) * V over the partition's tokens.
//
// gfx950 design (not the pages'):
//  * Work items are (sequence, kv head, partition) triples with real tokens, taken from a
//    dense list (worklist.h) so no workgroup is spent on empty partitions; the empty ones
//    get their sentinel from a grid-stride pass. Each workgroup has W waves; every page of
//    16 tokens is read from HBM exactly once and used for all G heads. Waves take the
//    partition's pages round-robin with independent softmax states, merged through LDS.
//  * K goes straight into registers with 16-byte loads. A token's row is split over LPT
//    lanes (LPT * 16 B >= 128 B, so each load instruction consumes whole 128-byte lines in
//    both layouts); scores are summed across those lanes with DPP.
//  * The running max is wave-uniform per head (readfirstlane), so the rescale of l and acc
//    is a scalar branch, skipped whenever a page does not raise the max.
//  * Scores are kept in base 2 (scale * log2 e folded once), so exp is one v_exp_f32; the
//    stored m is converted back to natural-log units.
//  * Plain float32 FMAs and float32 P (no rounding of P, so the 1e-5 bound holds).
//  * Token-major V has K's lane layout, so P never leaves the lane. x-packed V ([D][16] per
//    page) is read linearly (lane i takes 16-byte chunk i: one d, 4 consecutive tokens)
//    and P reaches it through a per-wave LDS row.
//  * Page ids are cached one per lane (lane j: the wave's j-th page) and broadcast with
//    v_readlane, so the page loop issues no dependent vector loads. Single register buffer
//    with early re-issue: the next page's K loads leave as soon as the current scores are
//    formed, its V loads as soon as P.V is done.
#pragma once

#include <type_traits>

#include "common.h"
#include "decode_args.h"
#include "decode_epilogue.h"
#include "worklist.h"

namespace pkv {

constexpr float kRebase = 8.f;  // log2 headroom of the lazy softmax rescale

template <int D, int G, bool XP, int LPT, int W>
struct ValuCfg {
  static constexpr int BS = 16;
  static constexpr int E = 4;                 // float32 elements per 16-byte chunk
  static constexpr int EB = 4;                // bytes per element
  static constexpr int ROWB = D * EB;         // bytes of one token's K (or V) row
  static constexpr int NC = ROWB / 16;        // chunks per token row
  static constexpr int CPL = NC / LPT;        // chunks per lane per token
  static constexpr int TPI = 64 / LPT;        // tokens covered by one load instruction
  static constexpr int TPL = BS / TPI;        // tokens per lane per page
  static constexpr int PAGEB = BS * ROWB;     // bytes of one (page, kv head) block of K or V
  static constexpr int TPC = 16 / EB;         // x-packed V: tokens per chunk
  static constexpr int CPD = BS / TPC;        // x-packed V: chunks per d
  static constexpr int NVC = D * CPD / 64;    // x-packed V: chunks per lane per page
  static constexpr int NACC = XP ? NVC : CPL * E;
  static constexpr int NVREG = XP ? NVC : TPL * CPL;
  static_assert(NC % LPT == 0 && CPL >= 1, "row must split evenly over LPT lanes");
  static_assert(TPL >= 1, "at least one token per lane and page");
  static_assert(!XP || NVC >= 1, "x-packed V needs at least one chunk per lane");
};

template <int W, int G, int D, bool XP>
struct ValuSmem {
  __attribute__((aligned(16))) uint32_t q_lds[G][D];  // query rows of the item (D*4 bytes >= a row)
  float red_acc[W][G][D];
  float red_m[W][G];     // exact max of the wave's scores (base 2)
  float red_mref[W][G];  // reference max that the wave's l and acc are relative to
  float red_l[W][G];
  __attribute__((aligned(16))) float p_lds[XP ? W : 1][G][16];
};

// One work item: partials of (b, kvh, p) for the G heads of kv head kvh.
template <int D, int G, bool XP, int LPT, int W, bool FINAL, bool ALIBI>
__device__ __forceinline__ void valu_partition(const DecodePartialArgs& a, const int b, const int kvh,
                                               const int p, const int len, ValuSmem<W, G, D, XP>& sm) {
  using C = ValuCfg<D, G, XP, LPT, W>;
  constexpr int BS = C::BS, E = C::E, ROWB = C::ROWB, CPL = C::CPL, TPI = C::TPI, TPL = C::TPL;
  constexpr int PAGEB = C::PAGEB, TPC = C::TPC, CPD = C::CPD, NVC = C::NVC, NACC = C::NACC;

  const int lane = threadIdx.x & 63;
  const int w = uniform((int)(threadIdx.x >> 6));
  const int c = lane % LPT;   // chunk column of the token row
  const int tg = lane / LPT;  // token group (token index within a load row)
  const int H = a.H;

  const int npages_seq = (len + BS - 1) / BS;
  const int ppp = uniform(part_tokens(len, a.ps, a.nsplit, BS) / BS);
  const int pg_begin = p * ppp;
  const int pg_end = min(pg_begin + ppp, npages_seq);
  // pages of this wave: pg_begin + w + W * i, i < n_my
  const int n_my = pg_end - pg_begin - w > 0 ? (pg_end - pg_begin - w + W - 1) / W : 0;
  const int t_last = min(pg_end * BS, len) - 1;  // the partition's last token (ALiBi reference)
  const int32_t* bt_row = a.bt + (size_t)b * a.mb;

  int pid_cache = 0;
  auto load_ids = [&](int i0) {  // lane j <- id of the wave's page i0 + j
    const int i = i0 + lane;
    int id = (i < n_my) ? bt_row[pg_begin + w + W * i] : 0;
    id = id < 0 ? 0 : id;
    pid_cache = id >= a.NB ? a.NB - 1 : id;
  };
  load_ids(0);

  // ---- the G query rows go to LDS once per item; lanes re-read their chunks per page
  // (broadcast reads), which keeps them out of the register budget.
  {
    const char* qb = reinterpret_cast<const char*>(a.q) + ((size_t)b * H + (size_t)kvh * G) * ROWB;
    for (int i = threadIdx.x; i < G * (ROWB / 16); i += 64 * W) {
      const int g = i / (ROWB / 16), ch = i - g * (ROWB / 16);
      *reinterpret_cast<uint4*>(&sm.q_lds[g][ch * 4]) = ld16(qb + (size_t)g * ROWB + ch * 16);
    }
  }
  __syncthreads();

  // Softmax state per head: l and acc are relative to m_ref (base 2); m_true is the exact
  // running max. m_ref is re-based only when m_true outgrows it by kRebase, so p stays
  // below 2^kRebase and the rescale of acc is rare; the exact max is what gets stored.
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

  // Byte offset of (token-in-page t, chunk column cc) inside a (page, head) K block.
  auto k_off = [&](int t, int cc) -> int {
    if constexpr (XP) return (cc * BS + t) * 16;   // [D/x][16][x]
    else return t * ROWB + cc * 16;                // [16][D]
  };

  uint4 kr[TPL][CPL];
  uint4 vr[C::NVREG];

  auto page_ptr = [&](const char* base, int i) -> const char* {
    const int id = __builtin_amdgcn_readlane(pid_cache, i & 63);
    return base + (size_t)id * block_stride;
  };
  // Pages are loaded non-temporally, except each wave's last page: the loop refills the
  // registers past the end by re-reading that page (so the loads stay unconditional and
  // need no merge copies), which must then be an L2 hit, not HBM.
  auto ldkv = [&](auto nt, const char* p) -> uint4 {
    if constexpr (decltype(nt)::value) return ld16_kv(p);
    else return ld16(p);
  };
  auto issue_k = [&](auto nt, int i) {
    const char* kp = page_ptr(kbase, i);
#pragma unroll
    for (int j = 0; j < TPL; ++j)
#pragma unroll
      for (int k = 0; k < CPL; ++k) kr[j][k] = ldkv(nt, kp + k_off(tg + TPI * j, c + LPT * k));
  };
  auto issue_v = [&](auto nt, int i) {
    const char* vp = page_ptr(vbase, i);
    if constexpr (XP) {
#pragma unroll
      for (int q = 0; q < NVC; ++q) vr[q] = ldkv(nt, vp + (size_t)(64 * q + lane) * 16);
    } else {
#pragma unroll
      for (int j = 0; j < TPL; ++j)
#pragma unroll
        for (int k = 0; k < CPL; ++k) vr[j * CPL + k] = ldkv(nt, vp + k_off(tg + TPI * j, c + LPT * k));
    }
  };

  using Streaming = std::true_type;  // non-temporal loads
  using Cached = std::false_type;    // ordinary loads (kept in L2)
  if (n_my > 1) {
    issue_k(Streaming{}, 0);
    issue_v(Streaming{}, 0);
  } else if (n_my == 1) {
    issue_k(Cached{}, 0);
    issue_v(Cached{}, 0);
  }
  // one page; `nt` is the cache policy of the loads it issues for the next page
  auto page = [&](auto nt, int i) {
    const int pg = pg_begin + w + W * i;
    const int ntok = min(BS, len - pg * BS);  // valid tokens in this page (uniform)
    const bool more = i + 1 < n_my;
    if (more && ((i + 1) & 63) == 0) load_ids(i + 1);  // next 64 pages of this wave (rare)

    // ---- scores for this lane's tokens, summed over the LPT lanes of the row
    asm volatile("" ::: "memory");  // keep the q reads inside the loop (registers are scarce)
    float s[G][TPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint4 qv[CPL];
#pragma unroll
      for (int k = 0; k < CPL; ++k) qv[k] = *reinterpret_cast<const uint4*>(&sm.q_lds[g][(c + LPT * k) * 4]);
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          const uint4 kv = kr[j][k];
          d0 = fmaf(__uint_as_float(qv[k].x), __uint_as_float(kv.x), d0);
          d1 = fmaf(__uint_as_float(qv[k].y), __uint_as_float(kv.y), d1);
          d0 = fmaf(__uint_as_float(qv[k].z), __uint_as_float(kv.z), d0);
          d1 = fmaf(__uint_as_float(qv[k].w), __uint_as_float(kv.w), d1);
        }
        s[g][j] = d0 + d1;
      }
    }
    // K registers are free again: the next page's loads leave now (unconditionally: the
    // last iteration re-reads its own page, see issue_k).
    issue_k(nt, more ? i + 1 : i);

#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        const float v = group_sum<LPT>(s[g][j]);
        float x = v * a.scale_log2;
        if constexpr (ALIBI)
          x = fmaf(a.alibi[kvh * G + g] * kLog2e, (float)(pg * BS + tg + TPI * j - t_last), x);
        s[g][j] = (tg + TPI * j < ntok) ? x : kNegInf;
      }

    // ---- online softmax with a wave-uniform running max per head
    float pr[G][TPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float pm = s[g][0];
#pragma unroll
      for (int j = 1; j < TPL; ++j) pm = fmaxf(pm, s[g][j]);
      pm = wave_max_uniform<LPT>(pm);
      m_true[g] = fmaxf(m_true[g], pm);
      // Re-base when the max outgrows the reference by kRebase (and on the wave's first
      // page, where l = acc = 0). Branch-free: alpha is exactly 1 when nothing changes, and
      // a uniform multiply costs less than the register copies a branch would force.
      const float new_ref = (m_true[g] > m_ref[g] + kRebase) ? m_true[g] : m_ref[g];
      const float alpha = fast_exp2(m_ref[g] - new_ref);  // -inf - x -> 0 on the first page
      m_ref[g] = new_ref;
      lsum[g] *= alpha;
#pragma unroll
      for (int q = 0; q < NACC; ++q) acc[g][q] *= alpha;
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        pr[g][j] = fast_exp2(s[g][j] - m_ref[g]);
        psum += pr[g][j];
      }
      lsum[g] += psum;
    }

    const bool tail = ntok < BS;  // uniform
    if constexpr (!XP) {
      // ---- tail page: zero V of invalid tokens (their slots may hold anything, even NaN)
      if (tail) {
#pragma unroll
        for (int j = 0; j < TPL; ++j)
          if (tg + TPI * j >= ntok)
#pragma unroll
            for (int k = 0; k < CPL; ++k) vr[j * CPL + k] = make_uint4(0, 0, 0, 0);
      }
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
    } else {
      // publish P to the wave's LDS row: p_lds[w][g][token]
      if (c == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int j = 0; j < TPL; ++j) sm.p_lds[w][g][tg + TPI * j] = pr[g][j];
      }
      wave_lds_fence();
      const int u = lane % CPD;  // which TPC-token slice of the page this lane's chunks hold
      if (tail) {
#pragma unroll
        for (int q = 0; q < NVC; ++q) {
          uint32_t x[4] = {vr[q].x, vr[q].y, vr[q].z, vr[q].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = u * TPC + e;
            x[e] = (t >= ntok) ? 0u : x[e];
          }
          vr[q] = make_uint4(x[0], x[1], x[2], x[3]);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float4 pf = *reinterpret_cast<const float4*>(&sm.p_lds[w][g][u * TPC]);
#pragma unroll
        for (int q = 0; q < NVC; ++q) {
          float t = acc[g][q];
          t = fmaf(pf.x, __uint_as_float(vr[q].x), t);
          t = fmaf(pf.y, __uint_as_float(vr[q].y), t);
          t = fmaf(pf.z, __uint_as_float(vr[q].z), t);
          t = fmaf(pf.w, __uint_as_float(vr[q].w), t);
          acc[g][q] = t;
        }
      }
      wave_lds_fence();  // this page's P reads finish before the next page overwrites it
    }
    issue_v(nt, more ? i + 1 : i);  // V registers are free again (unconditional, as for K)
  };
  int i = 0;
  for (; i + 2 < n_my; ++i) page(Streaming{}, i);    // refills pages 1 .. n_my-2
  for (; i < n_my; ++i) page(Cached{}, i);  // refills the last page, then re-reads it

  // ---- merge this wave's lanes, then the waves, through LDS
#pragma unroll
  for (int g = 0; g < G; ++g) {
    lsum[g] = strided_sum<LPT>(lsum[g]);  // over token groups (lanes of a group agree)
    if constexpr (XP) {
#pragma unroll
      for (int q = 0; q < NVC; ++q) acc[g][q] = group_sum<CPD>(acc[g][q]);
    } else {
#pragma unroll
      for (int q = 0; q < NACC; ++q) acc[g][q] = strided_sum<LPT>(acc[g][q]);
    }
  }
  if constexpr (XP) {
    if (lane % CPD == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int q = 0; q < NVC; ++q) sm.red_acc[w][g][(64 * q + lane) / CPD] = acc[g][q];
    }
  } else {
    if (tg == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < CPL; ++k)
#pragma unroll
          for (int e = 0; e < E; ++e) sm.red_acc[w][g][(c + LPT * k) * E + e] = acc[g][k * E + e];
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

  const int nparts = FINAL ? item_parts(a, len) : 0;
  const bool single = FINAL && nparts == 1;  // final output straight from the merge
  const size_t bh0 = (size_t)b * H + (size_t)kvh * G;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * W) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = sm.red_m[0][g];
#pragma unroll
    for (int v = 1; v < W; ++v) M = fmaxf(M, sm.red_m[v][g]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const float f = fast_exp2(sm.red_mref[v][g] - M);  // waves without pages carry -inf: f = 0
      o = fmaf(f, sm.red_acc[v][g][d], o);
      L = fmaf(f, sm.red_l[v][g], L);
    }
    if constexpr (ALIBI) M += alibi_shift2(a, kvh * G + g, len, t_last);  // after the weights
    store_item_value<D, false, FINAL>(a, bh0 + g, p, d, o, M, L, single);
  }
  __syncthreads();  // LDS is reused by the next item
  if constexpr (FINAL)
    if (nparts > 1) finish_item_fused<D, false, W>(a, b, kvh, G, nparts);
}

template <int D, int G, bool XP, int LPT, int W, bool DENSE, int WPE, bool FINAL, bool ALIBI>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(WPE, 8))) void decode_partial_valu_kernel(DecodePartialArgs a, int grid_parts) {
  __shared__ ValuSmem<W, G, D, XP> sm;
  if constexpr (DENSE) {
    extern __shared__ int s_worklist[];
    __shared__ int s_wave[2 * W];
    const DenseItems it = build_worklist<64 * W>(a.lens, a.S, a.len_cap, a.ps, a.nsplit, a.KVH, s_worklist, s_wave);
    write_sentinels(it, a.H, grid_parts, a.P, a.m, a.l);
    if constexpr (FINAL) write_empty_outputs<D, false>(it, a);
    for (int item = blockIdx.x; item < it.n_items; item += gridDim.x) {
      int b, kvh, p;
      decode_item(it, item, b, kvh, p);
      b = uniform(b);
      kvh = uniform(kvh);
      p = uniform(p);
      int len = a.lens[b];
      len = len > a.len_cap ? a.len_cap : len;
      valu_partition<D, G, XP, LPT, W, FINAL, ALIBI>(a, b, kvh, p, uniform(len), sm);
    }
  } else {  // partition-major: empty partitions sit at high indices and are dispatched last
    const int sk = a.S * a.KVH;
    const int p = (int)(blockIdx.x / sk);
    const int r = (int)(blockIdx.x - p * sk);
    const int b = r / a.KVH, kvh = r - b * a.KVH;
    int len = a.lens[b];
    len = len < 0 ? 0 : (len > a.len_cap ? a.len_cap : len);
    if (p * part_tokens(len, a.ps, a.nsplit, 16) >= len) {
      // empty partition: sentinel (PagedAttention V2, unused-partition branch)
      if (threadIdx.x < G && a.m != nullptr) {
        const size_t si = ((size_t)b * a.H + (size_t)kvh * G + threadIdx.x) * a.P + p;
        a.m[si] = kNegInf;
        a.l[si] = 0.f;
      }
      if constexpr (FINAL)
        if (p == 0) write_empty_rows<D, false>(a, b, kvh, G);
      return;
    }
    valu_partition<D, G, XP, LPT, W, FINAL, ALIBI>(a, b, kvh, p, len, sm);
  }
}

template <bool XP, int D, int G, bool FINAL, bool ALIBI>
hipError_t launch_valu_fin(const DecodePartialArgs& a, int grid_parts, hipStream_t s) {
  constexpr int EB = 4;
#ifndef PKV_VALU_ROW_BYTES_LPT16
#define PKV_VALU_ROW_BYTES_LPT16 256
#endif
#ifndef PKV_VALU_WPE
#define PKV_VALU_WPE 1
#endif
  // Token rows of >= 256 bytes are split over 16 lanes, shorter ones over 8.
  constexpr int LPT = (D * EB >= PKV_VALU_ROW_BYTES_LPT16) ? 16 : 8;
  constexpr int W = 4;
  constexpr int WPE = PKV_VALU_WPE;  // target waves per SIMD (4 caps VGPRs at 128)
  // The work list pays off on skewed batches; the float32 instances at head dim 256 or
  // with more than 8 heads per group (a parity path) keep to the plain grid, which halves
  // what they compile.
  constexpr bool kListed = D != 256 && G <= 8;
  bool listed = false;
  if constexpr (kListed) listed = use_dense_worklist(a.S, a.KVH, grid_parts);
  if (listed) {
    if constexpr (kListed) {
      const long upper = (long)a.S * a.KVH * grid_parts;
      const int grid = (int)(upper < dense_grid_cap() ? upper : dense_grid_cap());
      hipLaunchKernelGGL((decode_partial_valu_kernel<D, G, XP, LPT, W, true, WPE, FINAL, ALIBI>), dim3(grid),
                         dim3(64 * W), worklist_lds_words(a.S) * sizeof(int), s, a, grid_parts);
    }
  } else {
    const long upper = (long)a.S * a.KVH * grid_parts;
    if (upper > INT32_MAX) return hipErrorNotSupported;
    hipLaunchKernelGGL((decode_partial_valu_kernel<D, G, XP, LPT, W, false, WPE, FINAL, ALIBI>), dim3((unsigned)upper),
                       dim3(64 * W), 0, s, a, grid_parts);
  }
  return hipGetLastError();
}

template <bool XP, int D, int G>
hipError_t launch_valu_one(const DecodePartialArgs& a, int grid_parts, hipStream_t s) {
  if (a.kv_fp8) return hipErrorNotSupported;  // float8 caches are read with a bf16 query
  if (a.alibi != nullptr)
    return a.out != nullptr ? launch_valu_fin<XP, D, G, true, true>(a, grid_parts, s)
                            : launch_valu_fin<XP, D, G, false, true>(a, grid_parts, s);
  return a.out != nullptr ? launch_valu_fin<XP, D, G, true, false>(a, grid_parts, s)
                          : launch_valu_fin<XP, D, G, false, false>(a, grid_parts, s);
}

// Group sizes GLO .. GHI of one head dim (the instances of one translation unit).
template <bool XP, int D, int GLO, int GHI>
hipError_t launch_valu_g(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  if constexpr (GLO > GHI) {
    return hipErrorNotSupported;
  } else {
    if (G == GLO) return launch_valu_one<XP, D, GLO>(a, grid_parts, s);
    return launch_valu_g<XP, D, GLO + 1, GHI>(a, G, grid_parts, s);
  }
}

// The float32 instances are split over four translation units per layout so that the
// build compiles them in parallel: head dims 64 and 128 with G <= 8 (decode_valu_f32_<l>),
// G 9 .. 16 at head dims 64 and 128 (decode_valu_f32_<l>_g16), head dim 256 with G <= 8
// (decode_valu_f32_<l>_d256) and with G 9 .. 16 (decode_valu_f32_<l>_d256g16).
#define PKV_F32_PART_LAUNCHERS(L)                                                                       \
  hipError_t launch_valu_f32_##L##_d256(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s);    \
  hipError_t launch_valu_f32_##L##_d256g16(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s); \
  hipError_t launch_valu_f32_##L##_g16(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s);
PKV_F32_PART_LAUNCHERS(tm)
PKV_F32_PART_LAUNCHERS(xp)
#undef PKV_F32_PART_LAUNCHERS

}  // namespace pkv
