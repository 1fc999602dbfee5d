// Split-K paged decode, phase 1, bf16, vector ALUs (query-head groups G <= 8).
//
// Same computation as decode_valu.h (per-partition m, l and unnormalized acc for the G
// heads of one kv head; PagedAttention V2 Triton page, _partition_attn_kernel, with the
// flash-decode post's unnormalized accumulator), with a layout tuned for bf16:
//  * K and V use different lane layouts. For q.K a token's row is split over 8 lanes; the
//    2G partial scores of a lane are reduce-scattered over those 8 lanes (a few DPP adds,
//    lane-permuted registers, see bf16_items), so each lane ends with whole scores and the
//    softmax runs once per (head, token) instead of once per lane of the row. For P.V a
//    token row is split over 16 lanes in the token-major layout (so each lane owns fewer
//    dims and the accumulator is small), or read in the linear 16-byte chunk order of the
//    x-packed V layout.
//  * P crosses between the two layouts through a per-wave LDS row of bf16 values, stored
//    in the order each V lane reads them: one 4-, 8- or 16-byte read gives a lane its
//    token pairs, ready for v_dot2c_f32_bf16.
//  * Softmax with a lane-local running max: each page costs one max per head and lane, and
//    a single ballot asks whether any score passed the wave-uniform exponent reference by
//    more than the headroom; only then (the first page, and rarely later) is the max
//    reduced over the wave and the accumulators rescaled. The exact max is reduced once
//    per item, at the merge. (Reducing it over the wave and rescaling every page cost
//    about 80 more instructions per page: 58.4 against 56.3 us per llama_gqa4 step.)
//  * Everything else follows decode_valu.h: dense work list, page ids broadcast with
//    v_readlane, q rows in LDS, single register buffer with early re-issue, base-2
//    exponent, LDS merge of the waves.
#pragma once

#include <type_traits>

#include "common.h"
#include "decode_args.h"
#include "decode_epilogue.h"
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
  __attribute__((aligned(16))) uint32_t q_lds[2][G][D / 2];  // bf16 query rows: current, next item
  float red_acc[W][G][D];
  float red_m[W][G];
  float red_mref[W][G];
  float red_l[W][G];
  __attribute__((aligned(16))) uint16_t p_lds[W][G][16];  // bf16 P of the current page
};

// Processes the workgroup's work items (DENSE: wg_item(.., blockIdx.x, gridDim.x, k) for
// k = 0, 1, ... of the work list; otherwise the single partition-major item first_item). While an item runs,
// the page ids and length of the workgroup's next item are fetched, and its query rows go
// to the other LDS buffer by DMA while the waves merge, so moving to the next item costs no
// memory round trip before its first K/V pages go out. SPLIT: partitions follow the
// NUM_SPLITS policy, so an item's first page depends on its sequence's length and the
// page ids of the next item are fetched after its length (one more round trip per item).
// FINAL: the launch produces the output (final mode of DecodePartialArgs); compiled
// separately so that the plain partial kernel carries none of its code. ALIBI: scores
// carry the ALiBi bias (alibi_shift2). FP8: the K/V pools hold
// float8 e4m3 values (one byte each, same element order; x-packed keys in 16-element
// chunks), loaded 8 bytes where bf16 loads 16 and converted exactly to bf16 right before
// use; k_scale is folded into scale_log2 and v_scale multiplies the merged accumulator.
template <int D, int G, bool XP, int W, bool DENSE, bool SPLIT, bool FINAL, bool ALIBI, bool FP8 = false>
__device__ __forceinline__ void bf16_items(const DecodePartialArgs& a, const DenseItems& wl, int first_item,
                                           Bf16Smem<W, G, D>& sm) {
  using C = Bf16Cfg<D, XP>;
  constexpr int BS = C::BS, ROWB = C::ROWB, KCPL = C::KCPL, LV = C::LV, VT = C::VT, VCPL = C::VCPL;
  constexpr int NVC = C::NVC, NACC = C::NACC, NVREG = C::NVREG;
  constexpr int KVROWB = FP8 ? D : ROWB;       // bytes of a K/V token row (the query stays bf16)
  constexpr int PAGEB = BS * KVROWB;
  constexpr int QCH = G * (ROWB / 16);          // 16-byte chunks of the G query rows

  const int lane = threadIdx.x & 63;
  const int w = uniform((int)(threadIdx.x >> 6));
  const int kc = lane & 7;    // q.K: chunk column
  const int kt = lane >> 3;   // q.K: token (and kt + 8)
  // Scores in the reduce-scatter layout. The 2G (head, token half) scores a token row needs
  // are cut into blocks of 8 values (4 heads), then at most one block of 4 (2 heads) and one
  // of 2 (1 head). In a block of n values a lane keeps its partial scores in a lane-permuted
  // register order (register r holds value r ^ (kc & (n - 2)): the head bits follow the lane
  // through the q addresses it reads, the K registers keep their token order), so a few DPP
  // adds over the 8 lanes of the row leave every lane with whole scores: in a block of 8,
  // lane kc holds head (kc >> 1), token half kc & 1, each value once; in a block of 4 each
  // value sits in two lanes (kc, kc ^ 4), in a block of 2 in four. The exponent, running
  // max and sum are then computed once per value instead of once per lane of the row.
  constexpr int NB8 = 2 * G / 8;            // blocks of 4 heads
  constexpr bool HAS4 = (2 * G) % 8 >= 4;   // a block of 2 heads
  constexpr bool HAS2 = G % 2 == 1;         // a block of 1 head
  constexpr int NLV = NB8 + HAS4 + HAS2;    // scores per lane
  constexpr int H4 = 4 * NB8;               // first head of the 2-head block
  constexpr int H2 = 4 * NB8 + 2 * HAS4;    // the head of the 1-head block
  const bool odd = (kc & 1) != 0;
  // the lane's (head, token) of its k-th score, and whether it is the lane that publishes it
  auto lv_head = [&](int k) -> int {
    if (k < NB8) return 4 * k + (kc >> 1);
    if (HAS4 && k == NB8) return H4 + ((kc >> 1) & 1);
    return H2;
  };
  auto lv_owner = [&](int k) -> bool {
    if (k < NB8) return true;
    if (HAS4 && k == NB8) return (kc & 4) == 0;
    return (kc & 6) == 0;
  };
  const int rs_t = kt + 8 * (kc & 1);  // the lane's token within the page (every block)
  // a lane holding head g's k-th score, for reading head-uniform values back
  auto lv_src_lane = [&](int g) -> int {
    if (g < H4) return 2 * (g & 3);
    if (HAS4 && g < H2) return 2 * (g - H4);
    return 0;
  };
  auto lv_of_head = [&](int g) -> int {
    if (g < H4) return g >> 2;
    if (HAS4 && g < H2) return NB8;
    return NB8 + (HAS4 ? 1 : 0);
  };
  const int vc = lane % LV;   // P.V token-major: chunk column
  const int vt = lane / LV;   // P.V token-major: first token
  const int H = a.H;
  const size_t block_stride = (size_t)a.KVH * PAGEB;

  auto item_of = [&](int item, int& b, int& kvh, int& p) {
    if constexpr (DENSE) {
      decode_item(wl, item, b, kvh, p);
    } else {  // partition-major: empty partitions sit at high indices and are dispatched last
      const int sk = a.S * a.KVH;
      p = item / sk;
      const int r = item - p * sk;
      b = r / a.KVH;
      kvh = r - b * a.KVH;
    }
    b = uniform(b);
    kvh = uniform(kvh);
    p = uniform(p);
  };
  // lane j <- table entry of this wave's page i0 + j of partition p of sequence b. The load
  // is unconditional (a page past the partition or the table row reads the row's last
  // entry of the partition instead) and the value is clamped into the pool only when a
  // page address is formed, so nothing waits for it until it is used.
  auto page_ids = [&](int b, int p, int ppp, int i0) -> int {
    const int pg_begin = p * ppp;
    const int pg_last = min(a.mb, pg_begin + ppp) - 1;
    const int pg = min(pg_begin + w + W * (i0 + lane), pg_last);
    return a.bt[(size_t)b * a.mb + pg];
  };
  auto clamp_len = [&](int len) {
    len = len < 0 ? 0 : (len > a.len_cap ? a.len_cap : len);
    return uniform(len);
  };
  // pages per partition of a sequence of (clamped) length len
  auto ppp_of = [&](int len) -> int {
    if constexpr (SPLIT) return uniform(part_tokens(len, a.ps, a.nsplit, BS) / BS);
    else return a.ppp;
  };
  // sequence length through the scalar cache: only the use waits for it
  auto len_of = [&](int b) { return ((const __attribute__((address_space(4))) int32_t*)a.lens)[b]; };
  // the G query rows of (b, kvh) into q_lds[slot] by LDS DMA (no registers held)
  auto fetch_q = [&](int b, int kvh, int slot) {
    const char* qb = reinterpret_cast<const char*>(a.q) + ((size_t)b * H + (size_t)kvh * G) * ROWB;
#pragma unroll
    for (int c0 = 64 * w; c0 < QCH; c0 += 64 * W) {
      if (c0 + lane < QCH)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(qb + (size_t)(c0 + lane) * 16),
            (__attribute__((address_space(3))) void*)(&sm.q_lds[slot][0][0] + c0 * 4), 16, 0, 0);
    }
  };
  // byte offset of the 8 key elements 8 cc .. 8 cc + 7 of token t within a page
  auto k_off = [&](int t, int cc) -> int {
    if constexpr (XP && FP8) return ((cc >> 1) * BS + t) * 16 + (cc & 1) * 8;
    else if constexpr (XP) return (cc * BS + t) * 16;
    else if constexpr (FP8) return t * KVROWB + cc * 8;
    else return t * ROWB + cc * 16;
  };
  constexpr int CHB = FP8 ? 8 : 16;  // bytes of 8 K/V elements

  // ---- the first item: ids, length and q in one memory round trip
  int nb, nkvh, np;
  item_of(first_item, nb, nkvh, np);
  int npid;
  int nlen;
  if constexpr (SPLIT) {
    nlen = len_of(nb);
    npid = page_ids(nb, np, ppp_of(clamp_len(nlen)), 0);
  } else {
    npid = page_ids(nb, np, a.ppp, 0);
  }
  fetch_q(nb, nkvh, 0);
  if constexpr (!SPLIT) nlen = len_of(nb);
  if (!DENSE && np * ppp_of(clamp_len(nlen)) * BS >= clamp_len(nlen)) {
    // empty partition (PagedAttention V2 page, unused-partition branch)
    if ((int)threadIdx.x < G && a.m != nullptr) {
      const size_t si = ((size_t)nb * H + (size_t)nkvh * G + threadIdx.x) * a.P + np;
      a.m[si] = kNegInf;
      a.l[si] = 0.f;
    }
    if constexpr (FINAL)
      if (np == 0) write_empty_rows<D, true>(a, nb, nkvh, G);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS DMA may outlive the workgroup
    return;  // uniform across the workgroup
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // q of the first item is visible

  int k_item = 0;
  int slot = 0;
  for (;;) {
    // ---- the prefetched item becomes current
    const int b = nb, kvh = nkvh, p = np, len = clamp_len(nlen);
    int pid_cache = npid;
    const int ppp = ppp_of(len);
    const int pg_begin = p * ppp;
    const int pg_end = min(pg_begin + ppp, (len + BS - 1) / BS);
    const int n_my = pg_end - pg_begin - w > 0 ? (pg_end - pg_begin - w + W - 1) / W : 0;
    const int t_last = min(pg_end * BS, len) - 1;  // the partition's last token (ALiBi reference)
    const char* kbase = reinterpret_cast<const char*>(a.kc) + (size_t)kvh * PAGEB;
    const char* vbase = reinterpret_cast<const char*>(a.vc) + (size_t)kvh * PAGEB;
    int cache_base = 0;  // first page (in this wave's order) whose id is in pid_cache
    auto page_ptr = [&](const char* base, int i) -> const char* {
      int id = __builtin_amdgcn_readlane(pid_cache, (i - cache_base) & 63);
      id = id < 0 ? 0 : (id >= a.NB ? a.NB - 1 : id);
      return base + (size_t)id * block_stride;
    };
    auto ensure_ids = [&](int i) {  // uniform; refreshes the lane cache every 64 pages
      if (i >= cache_base + 64) {
        cache_base = i & ~63;
        // used at once (the clamp), so the wait for it stays inside this rare branch
        const int id = page_ids(b, p, ppp, cache_base);
        pid_cache = id < 0 ? 0 : (id >= a.NB ? a.NB - 1 : id);
      }
    };
    using KVReg = typename std::conditional<FP8, uint2, uint4>::type;  // 8 elements as loaded
    KVReg kr[2][KCPL];
    KVReg vraw[NVREG];
    // Pages are loaded non-temporally, except each wave's last page of the item: the loop
    // refills the registers past the end by re-reading that page (so the loads stay
    // unconditional and need no merge copies), which must then be an L2 hit, not HBM.
    auto ldkv = [&](auto nt, const char* p) -> KVReg {
      if constexpr (FP8) {
        if constexpr (decltype(nt)::value) return ld8_nt(p);
        else return *reinterpret_cast<const uint2*>(p);
      } else {
        if constexpr (decltype(nt)::value) return ld16_kv(p);
        else return ld16(p);
      }
    };
    auto issue_k = [&](auto nt, int i) {
      const char* kp = page_ptr(kbase, i);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int k = 0; k < KCPL; ++k) kr[j][k] = ldkv(nt, kp + k_off(kt + 8 * j, kc + 8 * k));
    };
    auto issue_v = [&](auto nt, int i) {
      const char* vp = page_ptr(vbase, i);
      if constexpr (XP) {
#pragma unroll
        for (int q = 0; q < NVC; ++q) vraw[q] = ldkv(nt, vp + (size_t)(64 * q + lane) * CHB);
      } else {
#pragma unroll
        for (int j = 0; j < VT; ++j)
#pragma unroll
          for (int k = 0; k < VCPL; ++k)
            vraw[j * VCPL + k] = ldkv(nt, vp + (vt + (64 / LV) * j) * KVROWB + (vc + LV * k) * CHB);
      }
    };
    using Streaming = std::true_type;  // non-temporal loads
    using Cached = std::false_type;    // ordinary loads (kept in L2)
    // first page (a valid page of the pool even when this wave has none in the item)
    if (n_my > 1) {
      issue_k(Streaming{}, 0);
      issue_v(Streaming{}, 0);
    } else {
      issue_k(Cached{}, 0);
      issue_v(Cached{}, 0);
    }

    // ---- prefetch of the workgroup's next item
    ++k_item;
    const int next_item = DENSE ? wg_item(wl, blockIdx.x, gridDim.x, k_item) : -1;
    const bool has_next = next_item >= 0;
    if (has_next) {
      item_of(next_item, nb, nkvh, np);
      if constexpr (SPLIT) {
        nlen = len_of(nb);
        npid = page_ids(nb, np, ppp_of(clamp_len(nlen)), 0);
      } else {
        npid = page_ids(nb, np, a.ppp, 0);
        nlen = len_of(nb);
      }
    }

    float acc[G][NACC];
    float m_ref[G], m_true[G], lsum[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m_ref[g] = kNegInf;
      m_true[g] = kNegInf;  // lane-local running max here; reduced over the wave at the merge
      lsum[g] = 0.f;
#pragma unroll
      for (int i = 0; i < NACC; ++i) acc[g][i] = 0.f;
    }
    const uint32_t* q_cur = &sm.q_lds[slot][0][0];
    // per score of the lane: exponent reference (uniform over the lanes of its head), running
    // max, running sum (over the lane's own tokens) and ALiBi slope in base-2 units
    float rs_ref[NLV], rs_max[NLV], rs_sum[NLV], rs_slope[NLV];
#pragma unroll
    for (int k = 0; k < NLV; ++k) {
      rs_ref[k] = kNegInf;
      rs_max[k] = kNegInf;
      rs_sum[k] = 0.f;
      rs_slope[k] = ALIBI ? a.alibi[kvh * G + lv_head(k)] * kLog2e : 0.f;
    }
    // max / sum over the lanes of one head (token halves and rows; duplicates of a value in
    // lanes kc ^ 2, kc ^ 4 are not added twice)
    auto head_max = [&](float v) {
      v = fmaxf(v, dpp<kDppQuadXor1>(v));
      v = fmaxf(v, dpp<kDppRor8>(v));
      v = fmaxf(v, xor_lanes(v, 16));
      return fmaxf(v, xor_lanes(v, 32));
    };
    auto head_sum = [&](float v) {
      v += dpp<kDppQuadXor1>(v);
      v += dpp<kDppRor8>(v);
      v += xor_lanes(v, 16);
      return v + xor_lanes(v, 32);
    };
    auto lane_xor4 = [&](float v) { return dpp<kDppQuadRev>(dpp<kDppHalfMirror>(v)); };

    // one page; `nt` is the cache policy of the loads it issues for page nx
    auto page = [&](auto nt, int i) {
      const int pg = pg_begin + w + W * i;
      const int ntok = min(BS, len - pg * BS);
      // refill target: the next page, or the last page again past the end (see issue_k)
      const int nx = i + 1 < n_my ? i + 1 : i;
      ensure_ids(nx);
      // ---- scores (reduce-scatter layout, see above)
      asm volatile("" ::: "memory");  // q is re-read from LDS every page (registers are scarce)
      // partial dot products of head g's q row with the lane's two K tokens
      auto qk2 = [&](int g, float& s0, float& s1) {
        uint4 qv[KCPL];
#pragma unroll
        for (int k = 0; k < KCPL; ++k) qv[k] = *reinterpret_cast<const uint4*>(q_cur + g * (D / 2) + (kc + 8 * k) * 4);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float d0 = 0.f, d1 = 0.f;
#pragma unroll
          for (int k = 0; k < KCPL; ++k) {
            const uint4 kk = as_bf16x8(kr[j][k]);
            d0 = dot2_bf16(qv[k].x, kk.x, d0);
            d1 = dot2_bf16(qv[k].y, kk.y, d1);
            d0 = dot2_bf16(qv[k].z, kk.z, d0);
            d1 = dot2_bf16(qv[k].w, kk.w, d1);
          }
          (j == 0 ? s0 : s1) = d0 + d1;
        }
      };
      float xs[NLV];
#pragma unroll
      for (int bk = 0; bk < NB8; ++bk) {  // 4 heads: partners kc ^ 7, kc ^ 2, kc ^ 1
        float x8[8];
#pragma unroll
        for (int rh = 0; rh < 4; ++rh) qk2(4 * bk + (rh ^ (kc >> 1)), x8[2 * rh], x8[2 * rh + 1]);
        float y4[4], z2[2];
#pragma unroll
        for (int r = 0; r < 4; ++r) y4[r] = x8[r] + dpp<kDppHalfMirror>(x8[r ^ 6]);
#pragma unroll
        for (int r = 0; r < 2; ++r) z2[r] = y4[r] + dpp<kDppQuadXor2>(y4[r ^ 2]);
        xs[bk] = (odd ? z2[1] : z2[0]) + dpp<kDppQuadXor1>(odd ? z2[0] : z2[1]);
      }
      if constexpr (HAS4) {  // 2 heads: partners kc ^ 2, kc ^ 1, then the copy in kc ^ 4
        float x4[4];
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) qk2(H4 + (rh ^ ((kc >> 1) & 1)), x4[2 * rh], x4[2 * rh + 1]);
        float z2[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) z2[r] = x4[r] + dpp<kDppQuadXor2>(x4[r ^ 2]);
        const float z = (odd ? z2[1] : z2[0]) + dpp<kDppQuadXor1>(odd ? z2[0] : z2[1]);
        xs[NB8] = z + lane_xor4(z);
      }
      if constexpr (HAS2) {  // 1 head: partner kc ^ 1, then the copies in kc ^ 2, kc ^ 4
        float x2[2];
        qk2(H2, x2[0], x2[1]);
        float z = (odd ? x2[1] : x2[0]) + dpp<kDppQuadXor1>(odd ? x2[0] : x2[1]);
        z += dpp<kDppQuadXor2>(z);
        xs[NLV - 1] = z + lane_xor4(z);
      }
      issue_k(nt, nx);

      // ---- softmax: lane-local running max; the exponent reference of a head (uniform over
      // its lanes) moves, and the head's accumulators are rescaled, only when some score
      // exceeds it by more than the headroom
      bool over = false;
#pragma unroll
      for (int k = 0; k < NLV; ++k) {
        float x = xs[k] * a.scale_log2;
        if constexpr (ALIBI) x = fmaf(rs_slope[k], (float)(pg * BS + rs_t - t_last), x);
        if (ntok < BS) x = rs_t < ntok ? x : kNegInf;  // tail page (uniform branch)
        xs[k] = x;
        rs_max[k] = fmaxf(rs_max[k], x);
        over |= x > rs_ref[k] + kRebaseBf16;
      }
      if (__builtin_amdgcn_ballot_w64(over) != 0) {  // the first page, and rarely later
        float alpha[NLV];
#pragma unroll
        for (int k = 0; k < NLV; ++k) {
          const float hm = head_max(rs_max[k]);
          const float nref = hm > rs_ref[k] + kRebaseBf16 ? hm : rs_ref[k];  // uniform per head
          alpha[k] = fast_exp2(rs_ref[k] - nref);  // 0 on the first page
          rs_ref[k] = nref;
          rs_sum[k] *= alpha[k];
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float ag = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[lv_of_head(g)]), lv_src_lane(g)));
#pragma unroll
          for (int q = 0; q < NACC; ++q) acc[g][q] *= ag;
        }
      }
      // ---- P to the wave's LDS row (bf16), in the order the V lanes read it
#pragma unroll
      for (int k = 0; k < NLV; ++k) {
        const float pv = fast_exp2(xs[k] - rs_ref[k]);
        rs_sum[k] += pv;
        if (lv_owner(k)) sm.p_lds[w][lv_head(k)][p_slot<LV, XP>(rs_t)] = (uint16_t)(pack_bf16x2(pv, 0.f) & 0xffffu);
      }
      wave_lds_fence();

      // V as bf16 pairs (a conversion under FP8, a plain copy otherwise)
      uint4 vr[NVREG];
#pragma unroll
      for (int q = 0; q < NVREG; ++q) vr[q] = as_bf16x8(vraw[q]);
      // ---- tail page: zero V of invalid tokens (their slots may hold anything, even NaN)
      if (ntok < BS) {
        if constexpr (XP) {
          const int u = lane & 1;
#pragma unroll
          for (int q = 0; q < NVC; ++q) {
            uint32_t x[4] = {vr[q].x, vr[q].y, vr[q].z, vr[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int t = 8 * u + 2 * e;
              x[e] = (t >= ntok) ? 0u : (t + 1 >= ntok ? (x[e] & 0xffffu) : x[e]);
            }
            vr[q] = make_uint4(x[0], x[1], x[2], x[3]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < VT; ++j)
            if (vt + (64 / LV) * j >= ntok)
#pragma unroll
              for (int k = 0; k < VCPL; ++k) vr[j * VCPL + k] = make_uint4(0, 0, 0, 0);
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
            float t0 = dot2_bf16(pp.x, vr[q].x, acc[g][q]);
            float t1 = dot2_bf16(pp.y, vr[q].y, 0.f);
            t0 = dot2_bf16(pp.z, vr[q].z, t0);
            t1 = dot2_bf16(pp.w, vr[q].w, t1);
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
            const uint4 va = vr[j * VCPL + k], vb = vr[(j + 1) * VCPL + k];
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
      issue_v(nt, nx);
    };
    int i = 0;
    for (; i + 2 < n_my; ++i) page(Streaming{}, i);   // refills pages 1 .. n_my-2
    for (; i < n_my; ++i) page(Cached{}, i); // refills the last page, then re-reads it
    // the next item's q goes to the other LDS buffer while the waves meet (an LDS DMA in
    // flight during the page loop would make every LDS read there wait for all loads)
    if (has_next) fetch_q(nb, nkvh, slot ^ 1);

    // ---- merge: l over the q.K token groups; acc over the P.V token groups; then waves
    {
      float ls[NLV], mt[NLV];
#pragma unroll
      for (int k = 0; k < NLV; ++k) {
        ls[k] = head_sum(rs_sum[k]);
        mt[k] = head_max(rs_max[k]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int k = lv_of_head(g), src = lv_src_lane(g);
        lsum[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls[k]), src));
        m_true[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mt[k]), src));
        m_ref[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rs_ref[k]), src));
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
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
    if (has_next) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // q landed; published by the barrier below

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
        const float f = fast_exp2(sm.red_mref[v][g] - M);
        o = fmaf(f, sm.red_acc[v][g][d], o);
        L = fmaf(f, sm.red_l[v][g], L);
      }
      if constexpr (FP8) o *= a.v_scale;
      if constexpr (ALIBI) M += alibi_shift2(a, kvh * G + g, len, t_last);  // after the weights
      store_item_value<D, true, FINAL>(a, bh0 + g, p, d, o, M, L, single);
    }
    __syncthreads();
    if constexpr (FINAL)
      if (nparts > 1) finish_item_fused<D, true, W>(a, b, kvh, G, nparts);
    if (!has_next) break;
    slot ^= 1;
  }
}

// Waves per SIMD the register allocator must leave room for: 4 where the kernel fits in
// 128 VGPRs without spilling, else no constraint.
constexpr int bf16_min_waves(int D, int G) { return (D == 64 && G <= 5) || (D == 128 && G <= 4) ? 4 : 1; }

template <int D, int G, bool XP, int W, bool DENSE, bool SPLIT, bool FINAL, bool ALIBI, bool FP8>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(bf16_min_waves(D, G), 8))) void decode_partial_bf16_kernel(DecodePartialArgs a, int grid_parts) {
  __shared__ Bf16Smem<W, G, D> sm;
  if constexpr (DENSE) {
    extern __shared__ int s_worklist[];
    __shared__ int s_wave[2 * W];
    const DenseItems wl = build_worklist<64 * W>(a.lens, a.S, a.len_cap, a.ps, SPLIT ? a.nsplit : 0, a.KVH,
                                                 s_worklist, s_wave);
    write_sentinels(wl, a.H, grid_parts, a.P, a.m, a.l);
    if constexpr (FINAL) write_empty_outputs<D, true>(wl, a);
    const int first = wg_item(wl, blockIdx.x, gridDim.x, 0);
    if (first >= 0) bf16_items<D, G, XP, W, true, SPLIT, FINAL, ALIBI, FP8>(a, wl, first, sm);
  } else {
    bf16_items<D, G, XP, W, false, SPLIT, FINAL, ALIBI, FP8>(a, DenseItems{}, blockIdx.x, sm);
  }
}


// Waves per work item. With 3 at head_dim 128 a CU holds 5 workgroups (15 waves) instead
// of 4, so a batch like llama_gqa4 (1,272 items) starts every item at once instead of
// running a second, partial round on a quarter of the slots: measured 58.2-58.6 us
// against 59.2 us per phase-1 launch there. At head_dim 256 the fourth wave pays off
// (wide_gqa6: 220 us with 4, 234 us with 3).
#ifndef PKV_BF16_WAVES
#define PKV_BF16_WAVES 0
#endif
constexpr int bf16_waves(int D) { return PKV_BF16_WAVES > 0 ? PKV_BF16_WAVES : (D == 128 ? 3 : 4); }
template <bool XP, int D, int G, bool SPLIT, bool FINAL, bool ALIBI, bool FP8 = false>
hipError_t launch_bf16_one(const DecodePartialArgs& a, int grid_parts, hipStream_t s) {
  constexpr int W = bf16_waves(D);
  const long upper = (long)a.S * a.KVH * grid_parts;
  // The dense work list costs one extra memory round trip per workgroup (the lengths before
  // the first page ids) but keeps every workgroup busy and balanced. The plain (partition,
  // sequence, kv head) grid needs no such trip: its empty partitions exit at once and free
  // their slots, so when the whole grid is resident within about two rounds it is the
  // faster of the two (llama_gqa4, 2,048 workgroups on 1,280 slots: 58.2 against 59.2 us).
  // Larger grids keep the list.
  bool plain = !use_dense_worklist(a.S, a.KVH, grid_parts);
  if constexpr (!SPLIT) {
    if (!plain) {
      const int pcap = resident_grid(
          reinterpret_cast<const void*>(&decode_partial_bf16_kernel<D, G, XP, W, false, false, FINAL, ALIBI, FP8>), 64 * W,
          0);
      plain = upper <= 2L * pcap;
    }
  }
  if (!plain) {
    // one workgroup per resident slot (every workgroup starts at once and walks its items
    // with the next one prefetched) unless there are many items per slot, where the
    // hardware's own refill of finished slots balances uneven items better
    const size_t lds = worklist_lds_words(a.S) * sizeof(int);
#ifndef PKV_RESIDENT_RATIO
#define PKV_RESIDENT_RATIO 4
#endif
    int cap = resident_grid(
        reinterpret_cast<const void*>(&decode_partial_bf16_kernel<D, G, XP, W, true, SPLIT, FINAL, ALIBI, FP8>), 64 * W,
        lds);
    if (upper > (long)PKV_RESIDENT_RATIO * cap) cap = dense_grid_cap();
    const int grid = (int)(upper < cap ? upper : cap);
    hipLaunchKernelGGL((decode_partial_bf16_kernel<D, G, XP, W, true, SPLIT, FINAL, ALIBI, FP8>), dim3(grid),
                       dim3(64 * W), lds, s, a, grid_parts);
  } else {
    // the plain grid: one workgroup per (partition, sequence, kv head), partition-major
    if (upper > INT32_MAX) return hipErrorNotSupported;
    hipLaunchKernelGGL((decode_partial_bf16_kernel<D, G, XP, W, false, SPLIT, FINAL, ALIBI, FP8>), dim3((unsigned)upper),
                       dim3(64 * W), 0, s, a, grid_parts);
  }
  return hipGetLastError();
}

// One mode (SPLIT: NUM_SPLITS partitions; FINAL: the one-launch decode) for every head
// dim, group size, ALiBi and float8 combination; each mode of each layout is compiled in a
// translation unit of its own (decode_valu_bf16_<layout>_<mode>.hip) so that the build runs
// them in parallel.
template <bool XP, int D, int G, bool SPLIT, bool FINAL>
hipError_t launch_bf16_gm(const DecodePartialArgs& a, int grid_parts, hipStream_t s) {
  if (a.kv_fp8)
    return a.alibi != nullptr ? launch_bf16_one<XP, D, G, SPLIT, FINAL, true, true>(a, grid_parts, s)
                              : launch_bf16_one<XP, D, G, SPLIT, FINAL, false, true>(a, grid_parts, s);
  return a.alibi != nullptr ? launch_bf16_one<XP, D, G, SPLIT, FINAL, true, false>(a, grid_parts, s)
                            : launch_bf16_one<XP, D, G, SPLIT, FINAL, false, false>(a, grid_parts, s);
}

template <bool XP, int D, bool SPLIT, bool FINAL>
hipError_t launch_bf16_dm(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  switch (G) {
    case 1: return launch_bf16_gm<XP, D, 1, SPLIT, FINAL>(a, grid_parts, s);
    case 2: return launch_bf16_gm<XP, D, 2, SPLIT, FINAL>(a, grid_parts, s);
    case 3: return launch_bf16_gm<XP, D, 3, SPLIT, FINAL>(a, grid_parts, s);
    case 4: return launch_bf16_gm<XP, D, 4, SPLIT, FINAL>(a, grid_parts, s);
    case 5: return launch_bf16_gm<XP, D, 5, SPLIT, FINAL>(a, grid_parts, s);
    case 6: return launch_bf16_gm<XP, D, 6, SPLIT, FINAL>(a, grid_parts, s);
    case 7: return launch_bf16_gm<XP, D, 7, SPLIT, FINAL>(a, grid_parts, s);
    case 8: return launch_bf16_gm<XP, D, 8, SPLIT, FINAL>(a, grid_parts, s);
    default: return hipErrorNotSupported;
  }
}

template <bool XP, bool SPLIT, bool FINAL>
hipError_t launch_bf16_mode(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_bf16_dm<XP, 64, SPLIT, FINAL>(a, G, grid_parts, s);
    case 128: return launch_bf16_dm<XP, 128, SPLIT, FINAL>(a, G, grid_parts, s);
    case 256: return launch_bf16_dm<XP, 256, SPLIT, FINAL>(a, G, grid_parts, s);
    default: return hipErrorNotSupported;
  }
}

// The per-mode launchers of one layout (defined in the per-mode translation units).
#define PKV_BF16_MODE_LAUNCHERS(L)                                                                          \
  hipError_t launch_bf16_##L##_plain(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s);       \
  hipError_t launch_bf16_##L##_split(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s);       \
  hipError_t launch_bf16_##L##_final(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s);       \
  hipError_t launch_bf16_##L##_split_final(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s);
PKV_BF16_MODE_LAUNCHERS(tm)
PKV_BF16_MODE_LAUNCHERS(xp)
#undef PKV_BF16_MODE_LAUNCHERS

}  // namespace pkv
