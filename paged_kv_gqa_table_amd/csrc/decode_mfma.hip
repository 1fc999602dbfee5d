// Split-K paged decode, phase 1, on the matrix cores (query-head groups 8 <= G <= 16, bf16).
//
// Computes the same partials as the vector-ALU kernel (decode_valu.h): for one (sequence,
// kv head, partition) and each of its G query heads, m = max score, l = sum exp(s - m) and
// acc = sum exp(s - m) V (PagedAttention V2 Triton page, _partition_attn_kernel; unnormalized
// accumulator as in the flash-decode post's _flash_decode_partial_kernel, whose Q group
// tile times the page's K is the dense contraction used here).
//
// gfx950 design:
//  * Same dense work list, workgroup shape (4 waves, pages round-robin) and LDS merge as
//    the vector-ALU kernel; a wave handles one page (16 tokens) at a time.
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = the page's K (lane: token l%16, 8 dims),
//    B = Q^T of the group padded to 16 heads (registers, loaded once per item).
//  * P^T comes straight from the S^T accumulator layout (lane: head l%16, tokens 4*(l/16)+i)
//    and is the B operand of O^T = V^T P^T on v_mfma_f32_16x16x16_bf16 (k = 16 tokens).
//    x-packed V ([D][16] per page) gives each lane its 4 tokens of one dim as one 8-byte
//    load. Token-major V gives a lane 8 dims of one token per 16-byte load; byte permutes
//    turn the 4 tokens' chunks into 8 A operands (tile n of a 128-dim block holds dims
//    8 * row + n), so no LDS transpose is needed.
//  * Lane-local running max; the 4 lanes of a head share a base-2 exponent reference that
//    is re-based (behind a wave-uniform branch) only when some score passes it by more than
//    the headroom; the exact max, reduced over the head's lanes once per item, is stored in
//    natural-log units.
#include <type_traits>

#include "common.h"
#include "decode_args.h"
#include "decode_epilogue.h"
#include "worklist.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr float kMfmaRebase = 8.f;

PKV_DEVICE f32x4_t mfma_k32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}
PKV_DEVICE f32x4_t mfma_k16(uint2 a, uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                   c, 0, 0, 0);
}

// Element e (0..7) of chunks x and y as a bf16 pair (x[e], y[e]).
PKV_DEVICE uint32_t pick_pair(const uint4& x, const uint4& y, int e) {
  const uint32_t xa = e < 2 ? x.x : e < 4 ? x.y : e < 6 ? x.z : x.w;
  const uint32_t ya = e < 2 ? y.x : e < 4 ? y.y : e < 6 ? y.z : y.w;
  return (e & 1) ? pair_hi(xa, ya) : pair_lo(xa, ya);
}

template <int W, int D>
struct MfmaSmem {
  // rows padded by one float: a merge store writes one column of the 16 heads' rows, which
  // at a row stride of D floats (a multiple of the 64 banks) all land in one bank
  float red_acc[W][16][D + 1];
  float red_m[W][16];
  float red_mref[W][16];
  float red_l[W][16];
};

// FP8: the K/V pools hold float8 e4m3 values (one byte each, same element order; x-packed
// keys in 16-element chunks), loaded 8 bytes where bf16 loads 16 and converted exactly to
// bf16 right before the matrix-core instructions; k_scale is folded into scale_log2 and
// v_scale multiplies the merged accumulator. ALIBI: scores carry the ALiBi bias
// (alibi_shift2 in decode_epilogue.h).
template <int D, bool XP, int W, bool FINAL, bool ALIBI, bool FP8>
__device__ __forceinline__ void mfma_partition(const DecodePartialArgs& a, const int G, const int b, const int kvh,
                                               const int p, const int len, MfmaSmem<W, D>& sm) {
  constexpr int BS = 16;
  constexpr int ROWB = D * 2;                   // bytes of a bf16 query row
  constexpr int KVROWB = FP8 ? D : ROWB;        // bytes of a K/V token row
  constexpr int PAGEB = BS * KVROWB;
  constexpr int KS = D / 32;   // k-steps of S^T
  constexpr int NT = D / 16;   // O^T tiles
  constexpr int NB = D / 128;  // 128-dim blocks (token-major V)
  static_assert(D % 128 == 0 || XP, "token-major V needs whole 128-dim blocks");

  const int lane = threadIdx.x & 63;
  const int w = uniform((int)(threadIdx.x >> 6));
  const int g = lane >> 4;
  const int hl = lane & 15;
  const int H = a.H;

  const int npages_seq = (len + BS - 1) / BS;
  const int ppp = uniform(part_tokens(len, a.ps, a.nsplit, BS) / BS);
  const int pg_begin = p * ppp;
  const int pg_end = min(pg_begin + ppp, npages_seq);
  const int n_my = pg_end - pg_begin - w > 0 ? (pg_end - pg_begin - w + W - 1) / W : 0;
  const int t_last = min(pg_end * BS, len) - 1;  // the partition's last token (ALiBi reference)
  const int32_t* bt_row = a.bt + (size_t)b * a.mb;
  int pid_cache = 0;
  auto load_ids = [&](int i0) {
    const int i = i0 + lane;
    int id = (i < n_my) ? bt_row[pg_begin + w + W * i] : 0;
    id = id < 0 ? 0 : id;
    pid_cache = id >= a.NB ? a.NB - 1 : id;
  };
  load_ids(0);

  // Q^T (B of S^T): lane = (head hl, dims 32 s + 8 g .. +8); heads past G are zero
  uint4 qb[KS];
  {
    const char* qrow = reinterpret_cast<const char*>(a.q) + ((size_t)b * H + (size_t)kvh * G + hl) * ROWB;
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[s] = hl < G ? ld16(qrow + (s * 32 + g * 8) * 2) : make_uint4(0, 0, 0, 0);
  }

  // ALiBi slope of this lane's head in base-2 units (heads past G: 0)
  const float slope2 = (ALIBI && hl < G) ? a.alibi[kvh * G + hl] * kLog2e : 0.f;
  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf, m_true = kNegInf, lsum = 0.f;  // head hl

  const size_t block_stride = (size_t)a.KVH * PAGEB;
  const char* kbase = reinterpret_cast<const char*>(a.kc) + (size_t)kvh * PAGEB;
  const char* vbase = reinterpret_cast<const char*>(a.vc) + (size_t)kvh * PAGEB;
  auto page_ptr = [&](const char* base, int i) -> const char* {
    const int id = __builtin_amdgcn_readlane(pid_cache, i & 63);
    return base + (size_t)id * block_stride;
  };

  // K/V registers as loaded: 8 elements (16 bytes bf16, 8 bytes float8), or for x-packed V
  // 4 tokens of one dim (8 bytes bf16, 4 bytes float8); converted to bf16 at use
  using KV8 = typename std::conditional<FP8, uint2, uint4>::type;
  using V4 = typename std::conditional<FP8, uint32_t, uint2>::type;
  KV8 kr[KS];
  KV8 vt[XP ? 1 : 4][XP ? 1 : NB];  // token-major: tokens 4g+i, chunk 16*blk + hl
  V4 vx[XP ? NT : 1];               // x-packed: dim 16 t + hl, tokens 4g .. 4g+3
  // Pages are loaded non-temporally, except each wave's last page: the loop refills the
  // registers past the end by re-reading that page (so the loads stay unconditional and
  // need no merge copies), which must then be an L2 hit, not HBM.
  auto ldkv = [&](auto nt, const char* p) -> KV8 {
    if constexpr (FP8) {
      if constexpr (decltype(nt)::value) return ld8_nt(p);
      else return ld8(p);
    } else {
      if constexpr (decltype(nt)::value) return ld16_kv(p);
      else return ld16(p);
    }
  };
  // byte offset of the 8 key elements of dims 8c .. 8c + 7 of token t within a page
  auto k_off = [&](int t, int c) -> int {
    if constexpr (XP && FP8) return ((c >> 1) * BS + t) * 16 + (c & 1) * 8;
    else if constexpr (XP) return (c * BS + t) * 16;
    else return t * KVROWB + c * (FP8 ? 8 : 16);
  };
  auto issue_k = [&](auto nt, int i) {
    const char* kp = page_ptr(kbase, i);
#pragma unroll
    for (int s = 0; s < KS; ++s) kr[s] = ldkv(nt, kp + k_off(hl, 4 * s + g));  // dims 32s+8g.., token hl
  };
  auto issue_v = [&](auto nt, int i) {
    const char* vp = page_ptr(vbase, i);
    if constexpr (XP) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        vx[t] = *reinterpret_cast<const V4*>(vp + ((16 * t + hl) * BS + 4 * g) * (FP8 ? 1 : 2));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < NB; ++k) vt[j][k] = ldkv(nt, vp + (4 * g + j) * KVROWB + (16 * k + hl) * (FP8 ? 8 : 16));
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
    const int ntok = min(BS, len - pg * BS);
    const bool more = i + 1 < n_my;
    if (more && ((i + 1) & 63) == 0) load_ids(i + 1);

    f32x4_t st = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) st = mfma_k32(as_bf16x8(kr[s]), qb[s], st);
    issue_k(nt, more ? i + 1 : i);

    float x[4];
    float tmax = kNegInf;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float xv = st[j] * a.scale_log2;
      if constexpr (ALIBI) xv = fmaf(slope2, (float)(pg * BS + 4 * g + j - t_last), xv);
      x[j] = (4 * g + j < ntok) ? xv : kNegInf;
      tmax = fmaxf(tmax, x[j]);
    }
    // lane-local running max (this lane's tokens); the head's four lanes share the exponent
    // reference m_ref, which moves only when some score passes it by more than the headroom
    m_true = fmaxf(m_true, tmax);
    if (__builtin_amdgcn_ballot_w64(tmax > m_ref + kMfmaRebase) != 0) {  // the first page, and rarely later
      float hm = fmaxf(m_true, xor_lanes(m_true, 16));
      hm = fmaxf(hm, xor_lanes(hm, 32));  // the head's max so far, in all four of its lanes
      const bool rebase = hm > m_ref + kMfmaRebase;
      const float nref = rebase ? hm : m_ref;
      const float alpha = fast_exp2(m_ref - nref);
      m_ref = nref;
      lsum *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] *= alpha;
    }
    float pr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pr[j] = fast_exp2(x[j] - m_ref);
      lsum += pr[j];
    }
    const uint2 pb = make_uint2(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]));

    // V as bf16 (a conversion under FP8, a plain copy otherwise)
    uint2 vxb[XP ? NT : 1];
    uint4 vtb[XP ? 1 : 4][XP ? 1 : NB];
    if constexpr (XP) {
#pragma unroll
      for (int t = 0; t < NT; ++t) vxb[t] = as_bf16x4(vx[t]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < NB; ++k) vtb[j][k] = as_bf16x8(vt[j][k]);
    }
    if (ntok < BS) {  // tail page: zero V of invalid tokens (their slots may hold NaN)
      if constexpr (XP) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int t0 = 4 * g;
          uint32_t lo = vxb[t].x, hi = vxb[t].y;
          lo = (t0 >= ntok) ? 0u : (t0 + 1 >= ntok ? (lo & 0xffffu) : lo);
          hi = (t0 + 2 >= ntok) ? 0u : (t0 + 3 >= ntok ? (hi & 0xffffu) : hi);
          vxb[t] = make_uint2(lo, hi);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * g + j >= ntok)
#pragma unroll
            for (int k = 0; k < NB; ++k) vtb[j][k] = make_uint4(0, 0, 0, 0);
      }
    }

    if constexpr (XP) {
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = mfma_k16(vxb[t], pb, acc[t]);
    } else {
#pragma unroll
      for (int k = 0; k < NB; ++k)
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const uint2 av = make_uint2(pick_pair(vtb[0][k], vtb[1][k], n), pick_pair(vtb[2][k], vtb[3][k], n));
          acc[k * 8 + n] = mfma_k16(av, pb, acc[k * 8 + n]);
        }
    }
    issue_v(nt, more ? i + 1 : i);
  };
  int i = 0;
  for (; i + 2 < n_my; ++i) page(Streaming{}, i);    // refills pages 1 .. n_my-2
  for (; i < n_my; ++i) page(Cached{}, i);  // refills the last page, then re-reads it

  // ---- merge: l and the max over the 4 lanes of a head, then waves through LDS
  lsum += xor_lanes(lsum, 16);
  lsum += xor_lanes(lsum, 32);
  m_true = fmaxf(m_true, xor_lanes(m_true, 16));
  m_true = fmaxf(m_true, xor_lanes(m_true, 32));
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int d;
      if constexpr (XP) d = 16 * t + 4 * g + j;
      else d = (t / 8) * 128 + 8 * (4 * g + j) + (t % 8);
      sm.red_acc[w][hl][d] = acc[t][j];
    }
  if (g == 0) {
    sm.red_m[w][hl] = m_true;
    sm.red_mref[w][hl] = m_ref;
    sm.red_l[w][hl] = lsum;
  }
  __syncthreads();
  const int nparts = FINAL ? item_parts(a, len) : 0;
  const bool single = FINAL && nparts == 1;  // final output straight from the merge
  const size_t bh0 = (size_t)b * H + (size_t)kvh * G;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * W) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = sm.red_m[0][h];
#pragma unroll
    for (int v = 1; v < W; ++v) M = fmaxf(M, sm.red_m[v][h]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const float f = fast_exp2(sm.red_mref[v][h] - M);
      o = fmaf(f, sm.red_acc[v][h][d], o);
      L = fmaf(f, sm.red_l[v][h], L);
    }
    if constexpr (FP8) o *= a.v_scale;
    if constexpr (ALIBI) M += alibi_shift2(a, kvh * G + h, len, t_last);  // after the weights
    store_item_value<D, true, FINAL>(a, bh0 + h, p, d, o, M, L, single);
  }
  __syncthreads();
  if constexpr (FINAL)
    if (nparts > 1) finish_item_fused<D, true, W>(a, b, kvh, G, nparts);
}

// Waves per SIMD the register allocation must allow. Left alone, the compiler parks the
// output accumulators in AGPRs and lands at 148-168 registers (three waves per SIMD); held
// to 128, the partial kernels at D <= 128 fit without spills and four 4-wave workgroups
// share a CU. The one-launch (FINAL) kernels would spill at 128, and D = 256 cannot fit.
template <int D, bool FINAL>
constexpr int mfma_min_waves() { return (D <= 128 && !FINAL) ? 4 : 1; }

template <int D, bool XP, int W, bool DENSE, bool FINAL, bool ALIBI, bool FP8>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(mfma_min_waves<D, FINAL>())))
void decode_partial_mfma_kernel(DecodePartialArgs a, int G, int grid_parts) {
  __shared__ MfmaSmem<W, D> sm;
  if constexpr (DENSE) {
    extern __shared__ int s_worklist[];
    __shared__ int s_wave[2 * W];
    const DenseItems it = build_worklist<64 * W>(a.lens, a.S, a.len_cap, a.ps, a.nsplit, a.KVH, s_worklist, s_wave);
    write_sentinels(it, a.H, grid_parts, a.P, a.m, a.l);
    if constexpr (FINAL) write_empty_outputs<D, true>(it, a);
    for (int item = blockIdx.x; item < it.n_items; item += gridDim.x) {
      int b, kvh, p;
      decode_item(it, item, b, kvh, p);
      b = uniform(b);
      kvh = uniform(kvh);
      p = uniform(p);
      int len = a.lens[b];
      len = len > a.len_cap ? a.len_cap : len;
      mfma_partition<D, XP, W, FINAL, ALIBI, FP8>(a, G, b, kvh, p, uniform(len), sm);
    }
  } else {  // partition-major: empty partitions sit at high indices and are dispatched last
    const int sk = a.S * a.KVH;
    const int p = (int)(blockIdx.x / sk);
    const int r = (int)(blockIdx.x - p * sk);
    const int b = r / a.KVH, kvh = r - b * a.KVH;
    int len = a.lens[b];
    len = len < 0 ? 0 : (len > a.len_cap ? a.len_cap : len);
    if (p * part_tokens(len, a.ps, a.nsplit, 16) >= len) {
      if ((int)threadIdx.x < G && a.m != nullptr) {
        const size_t si = ((size_t)b * a.H + (size_t)kvh * G + threadIdx.x) * a.P + p;
        a.m[si] = kNegInf;
        a.l[si] = 0.f;
      }
      if constexpr (FINAL)
        if (p == 0) write_empty_rows<D, true>(a, b, kvh, G);
      return;
    }
    mfma_partition<D, XP, W, FINAL, ALIBI, FP8>(a, G, b, kvh, p, len, sm);
  }
}

template <int D, bool XP, bool FINAL, bool ALIBI, bool FP8>
hipError_t launch_mfma_f(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  constexpr int W = 4;
  if (use_dense_worklist(a.S, a.KVH, grid_parts)) {
    const long upper = (long)a.S * a.KVH * grid_parts;
    const int grid = (int)(upper < dense_grid_cap() ? upper : dense_grid_cap());
    hipLaunchKernelGGL((decode_partial_mfma_kernel<D, XP, W, true, FINAL, ALIBI, FP8>), dim3(grid), dim3(64 * W),
                       worklist_lds_words(a.S) * sizeof(int), s, a, G, grid_parts);
  } else {
    const long upper = (long)a.S * a.KVH * grid_parts;
    if (upper > INT32_MAX) return hipErrorNotSupported;
    hipLaunchKernelGGL((decode_partial_mfma_kernel<D, XP, W, false, FINAL, ALIBI, FP8>), dim3((unsigned)upper),
                       dim3(64 * W), 0, s, a, G, grid_parts);
  }
  return hipGetLastError();
}

template <int D, bool XP, bool FINAL>
hipError_t launch_mfma_fin(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  if (a.kv_fp8)
    return a.alibi != nullptr ? launch_mfma_f<D, XP, FINAL, true, true>(a, G, grid_parts, s)
                              : launch_mfma_f<D, XP, FINAL, false, true>(a, G, grid_parts, s);
  return a.alibi != nullptr ? launch_mfma_f<D, XP, FINAL, true, false>(a, G, grid_parts, s)
                            : launch_mfma_f<D, XP, FINAL, false, false>(a, G, grid_parts, s);
}

template <int D, bool XP>
hipError_t launch_mfma_d(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  return a.out != nullptr ? launch_mfma_fin<D, XP, true>(a, G, grid_parts, s)
                          : launch_mfma_fin<D, XP, false>(a, G, grid_parts, s);
}

template <bool XP>
hipError_t launch_mfma(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  if (G < 8 || G > 16) return hipErrorNotSupported;
  switch (a.D) {
    case 64:
      if constexpr (XP) return launch_mfma_d<64, XP>(a, G, grid_parts, s);
      else return hipErrorNotSupported;
    case 128: return launch_mfma_d<128, XP>(a, G, grid_parts, s);
    case 256: return launch_mfma_d<256, XP>(a, G, grid_parts, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_decode_mfma_bf16_tm(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  // D = 64 token-major rows are 128 bytes: no whole 128-dim V block; the vector-ALU kernel
  // covers G <= 8 there and the generic kernel larger groups.
  if (a.D == 64) return G <= 8 ? launch_decode_valu_bf16_tm(a, G, grid_parts, s)
                               : launch_decode_generic(a, G, grid_parts, false, false, s);
  return launch_mfma<false>(a, G, grid_parts, s);
}
hipError_t launch_decode_mfma_bf16_xp(const DecodePartialArgs& a, int G, int grid_parts, hipStream_t s) {
  return launch_mfma<true>(a, G, grid_parts, s);
}

}  // namespace pkv
