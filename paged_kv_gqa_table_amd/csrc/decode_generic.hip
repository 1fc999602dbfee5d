// Split-K paged decode, phase 1 (and the one-launch final mode), for page pools whose
// block size is not 16 tokens. The tuned kernels (decode_valu_bf16.h, decode_mfma.hip,
// decode_valu.h) build their lane layouts around 16-token pages; this one takes any block
// size, head dim 64/128/256, groups of up to 16 query heads, float32 or bf16 queries, bf16
// or float8 e4m3 pools, both layouts, ALiBi, and every partition policy the others take.
//
// What it computes is what they compute (PagedAttention V2 page, _partition_attn_kernel;
// flash-decode post, _flash_decode_partial_kernel): per (sequence b, kv head, partition p)
// and query head of the group, m = max score, l = sum exp(score - m), acc = sum exp(score -
// m) V, over the partition's tokens; token t sits in block block_tables[b, t / bs], slot
// t % bs.
//
// Design (plain, not tuned): one workgroup of four waves per item on the partition-major
// plain grid (empty partitions write their sentinels and leave). The waves take 64-token
// chunks of the partition in turn. For the scores a lane owns one token: it reads its K
// row in 8-element pieces (one 16-byte load for bf16, two for float32, one 8-byte load for
// float8; the x-packed layout's pieces follow its [D / x][bs][x] order) and dots them with
// the group's query rows, which sit in LDS as float32 (broadcast reads). The chunk's
// maximum and sum per head are wave reductions; the running softmax is re-based every
// chunk (exact, no headroom). For P V a lane owns D / 64 output dims: the chunk's P and
// each token's block and slot go through LDS, and the lane reads its dims of each token's
// V row. The four waves merge through LDS as in the tuned kernels, then the shared
// epilogue stores partials or, in the final mode, the output.
#include "decode_epilogue.h"

namespace pkv {
namespace {

constexpr int kGenW = 4;     // waves per item
constexpr int kGenG = 16;    // most query heads per kv head

template <int D>
struct GenSmem {
  union {
    struct {
      float q[kGenG][D];          // the item's query rows, float32
      float p[kGenW][kGenG][64];  // a wave's P of its current chunk
      int blk[kGenW][64];         // each chunk token's block id (clamped into the pool)
      int slot[kGenW][64];        // ... and its slot in the block
    } run;
    float red_acc[kGenW][kGenG][D];  // each wave's accumulator, for the merge (after the chunks)
  } u;
  float red_m[kGenW][kGenG];       // each wave's running max (base 2), -inf without tokens
  float red_l[kGenW][kGenG];
};

PKV_DEVICE float wave_max64(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
PKV_DEVICE float wave_sum64(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Element kinds of the pools: KV = 0 the query's type (bf16 or float32), 1 float8 e4m3.
template <bool QF32, int KV>
struct GenElem {
  static constexpr int bytes = KV == 1 ? 1 : (QF32 ? 4 : 2);
  static constexpr int x = 16 / bytes;  // x of the x-packed key layout
};

// Eight consecutive elements (8-aligned) of a row, as float32.
template <bool QF32, int KV>
PKV_DEVICE void load8(const char* p, float (&f)[8]) {
  if constexpr (KV == 1) {
    const uint2 v = ld8(p);
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, true);
    f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
    f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
  } else if constexpr (QF32) {
    const uint4 u = ld16(p), v = ld16(p + 16);
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y); f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
    f[4] = __uint_as_float(v.x); f[5] = __uint_as_float(v.y); f[6] = __uint_as_float(v.z); f[7] = __uint_as_float(v.w);
  } else {
    const uint4 u = ld16(p);
    f[0] = bf16lo(u.x); f[1] = bf16hi(u.x); f[2] = bf16lo(u.y); f[3] = bf16hi(u.y);
    f[4] = bf16lo(u.z); f[5] = bf16hi(u.z); f[6] = bf16lo(u.w); f[7] = bf16hi(u.w);
  }
}

// One element as float32.
template <bool QF32, int KV>
PKV_DEVICE float load1(const char* p) {
  if constexpr (KV == 1) {
    const uint32_t b = *reinterpret_cast<const uint8_t*>(p);
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)b, false)[0];
  } else if constexpr (QF32) {
    return *reinterpret_cast<const float*>(p);
  } else {
    return bf16lo(*reinterpret_cast<const uint16_t*>(p));
  }
}

template <int D, bool QF32, int KV, bool XP, bool FINAL, bool ALIBI>
__global__ __launch_bounds__(64 * kGenW) void decode_generic_kernel(DecodePartialArgs a) {
  __shared__ GenSmem<D> sm;
  using E = GenElem<QF32, KV>;
  constexpr int EB = E::bytes;
  constexpr int DPL = D / 64;  // output dims per lane
  const int lane = threadIdx.x & 63;
  const int w = uniform((int)(threadIdx.x >> 6));
  const int G = a.H / a.KVH;
  const int sk = a.S * a.KVH;
  const int p = (int)(blockIdx.x / sk);
  const int r = (int)(blockIdx.x - p * sk);
  const int b = r / a.KVH, kvh = r - b * a.KVH;
  int len = a.lens[b];
  len = uniform(len < 0 ? 0 : (len > a.len_cap ? a.len_cap : len));
  const int bs = a.bs;
  const int pt = part_tokens(len, a.ps, a.nsplit, bs);
  const int t0 = p * pt;
  if (t0 >= len) {  // empty partition (PagedAttention V2 page, unused-partition branch)
    if ((int)threadIdx.x < G && a.m != nullptr) {
      const size_t si = ((size_t)b * a.H + (size_t)kvh * G + threadIdx.x) * a.P + p;
      a.m[si] = kNegInf;
      a.l[si] = 0.f;
    }
    if constexpr (FINAL)
      if (p == 0) write_empty_rows<D, !QF32>(a, b, kvh, G);
    return;
  }
  const int t1 = min(t0 + pt, len);
  const int t_last = t1 - 1;  // ALiBi reference (the bias is kept partition-relative)

  // ---- the group's query rows to LDS as float32
  const size_t qrow0 = (size_t)b * a.H + (size_t)kvh * G;
  for (int i = threadIdx.x; i < G * D; i += 64 * kGenW) {
    const int g = i / D, d = i - g * D;
    float v;
    if constexpr (QF32) v = reinterpret_cast<const float*>(a.q)[(qrow0 + g) * D + d];
    else v = bf16lo(reinterpret_cast<const uint16_t*>(a.q)[(qrow0 + g) * D + d]);
    sm.u.run.q[g][d] = v;
  }
  __syncthreads();

  const char* kc = reinterpret_cast<const char*>(a.kc);
  const char* vc = reinterpret_cast<const char*>(a.vc);
  const int32_t* bt_row = a.bt + (size_t)b * a.mb;
  float slope2[kGenG];  // ALiBi slopes in base-2 units
#pragma unroll
  for (int g = 0; g < kGenG; ++g) slope2[g] = (ALIBI && g < G) ? a.alibi[kvh * G + g] * kLog2e : 0.f;

  float acc[kGenG][DPL];
  float m_run[kGenG], l_run[kGenG];
#pragma unroll
  for (int g = 0; g < kGenG; ++g) {
    m_run[g] = kNegInf;
    l_run[g] = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[g][i] = 0.f;
  }

  for (int c0 = t0 + 64 * w; c0 < t1; c0 += 64 * kGenW) {
    const int t = c0 + lane;
    const bool valid = t < t1;
    const int tt = valid ? t : t1 - 1;  // invalid lanes read the partition's last token (masked)
    int id = bt_row[tt / bs];
    id = id < 0 ? 0 : (id >= a.NB ? a.NB - 1 : id);
    const int sl = tt - (tt / bs) * bs;
    const size_t hb = (size_t)id * a.KVH + kvh;  // (block, kv head) index
    // ---- scores of this lane's token for the G heads
    float s[kGenG];
#pragma unroll
    for (int g = 0; g < kGenG; ++g) s[g] = 0.f;
    for (int d = 0; d < D; d += 8) {
      const char* kp;
      if constexpr (!XP) {
        kp = kc + ((hb * bs + sl) * D + d) * EB;
      } else if constexpr (E::x >= 8) {  // one x-chunk holds the 8 elements
        kp = kc + (((hb * (D / E::x) + d / E::x) * bs + sl) * E::x + d % E::x) * EB;
      } else {  // float32, x = 4: the 8 elements span two chunks of the token
        kp = nullptr;
      }
      float k8[8];
      if constexpr (XP && E::x < 8) {
        const char* p0 = kc + (((hb * (D / 4) + d / 4) * bs + sl) * 4) * EB;
        const char* p1 = kc + (((hb * (D / 4) + d / 4 + 1) * bs + sl) * 4) * EB;
        const uint4 u = ld16(p0), v = ld16(p1);
        k8[0] = __uint_as_float(u.x); k8[1] = __uint_as_float(u.y); k8[2] = __uint_as_float(u.z);
        k8[3] = __uint_as_float(u.w); k8[4] = __uint_as_float(v.x); k8[5] = __uint_as_float(v.y);
        k8[6] = __uint_as_float(v.z); k8[7] = __uint_as_float(v.w);
      } else {
        load8<QF32, KV>(kp, k8);
      }
#pragma unroll
      for (int g = 0; g < kGenG; ++g) {
        if (g < G) {
          const float4 qa = *reinterpret_cast<const float4*>(&sm.u.run.q[g][d]);
          const float4 qb = *reinterpret_cast<const float4*>(&sm.u.run.q[g][d + 4]);
          float x = s[g];
          x = fmaf(qa.x, k8[0], x); x = fmaf(qa.y, k8[1], x); x = fmaf(qa.z, k8[2], x); x = fmaf(qa.w, k8[3], x);
          x = fmaf(qb.x, k8[4], x); x = fmaf(qb.y, k8[5], x); x = fmaf(qb.z, k8[6], x); x = fmaf(qb.w, k8[7], x);
          s[g] = x;
        }
      }
    }
    // ---- online softmax per head over the chunk (re-based every chunk)
#pragma unroll
    for (int g = 0; g < kGenG; ++g) {
      if (g < G) {
        float x = s[g] * a.scale_log2;
        if constexpr (ALIBI) x = fmaf(slope2[g], (float)(t - t_last), x);
        x = valid ? x : kNegInf;
        const float m_new = fmaxf(m_run[g], wave_max64(x));  // finite: the chunk's first token is valid
        const float alpha = fast_exp2(m_run[g] - m_new);     // 0 on the wave's first chunk
        const float pe = fast_exp2(x - m_new);               // 0 for masked tokens
        l_run[g] = l_run[g] * alpha + wave_sum64(pe);
        m_run[g] = m_new;
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[g][i] *= alpha;
        sm.u.run.p[w][g][lane] = pe;
      }
    }
    sm.u.run.blk[w][lane] = id;
    sm.u.run.slot[w][lane] = sl;
    wave_lds_fence();
    // ---- P V: this lane's D / 64 dims of each token of the chunk, eight tokens' V loads
    // in flight at a time (tokens past the partition read the last one with P = 0)
    constexpr int U = 8;
    const int nt = min(64, t1 - c0);
    for (int j0 = 0; j0 < nt; j0 += U) {
      float v[U][DPL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = min(j0 + u, nt - 1);
        const size_t hbj = (size_t)sm.u.run.blk[w][j] * a.KVH + kvh;
        const int slj = sm.u.run.slot[w][j];
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          const int d = lane * DPL + i;
          const size_t e = XP ? (hbj * D + d) * bs + slj : (hbj * bs + slj) * D + d;
          v[u][i] = load1<QF32, KV>(vc + e * EB);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (j0 + u < nt) {
#pragma unroll
          for (int g = 0; g < kGenG; ++g) {
            if (g < G) {
              const float pj = sm.u.run.p[w][g][j0 + u];
#pragma unroll
              for (int i = 0; i < DPL; ++i) acc[g][i] = fmaf(pj, v[u][i], acc[g][i]);
            }
          }
        }
      }
    }
    wave_lds_fence();  // the chunk's P and rows are read before the next chunk overwrites them
  }

  // ---- merge the waves through LDS (the accumulators take the chunk buffers' space)
  __syncthreads();
#pragma unroll
  for (int g = 0; g < kGenG; ++g) {
    if (g < G) {
#pragma unroll
      for (int i = 0; i < DPL; ++i) sm.u.red_acc[w][g][lane * DPL + i] = acc[g][i];
      if (lane == 0) {
        sm.red_m[w][g] = m_run[g];
        sm.red_l[w][g] = l_run[g];
      }
    }
  }
  __syncthreads();
  const int nparts = FINAL ? item_parts(a, len) : 0;
  const bool single = FINAL && nparts == 1;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * kGenW) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = sm.red_m[0][g];
#pragma unroll
    for (int v = 1; v < kGenW; ++v) M = fmaxf(M, sm.red_m[v][g]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < kGenW; ++v) {
      const float f = fast_exp2(sm.red_m[v][g] - M);  // waves without tokens carry -inf: f = 0
      o = fmaf(f, sm.u.red_acc[v][g][d], o);
      L = fmaf(f, sm.red_l[v][g], L);
    }
    if (a.kv_fp8) o *= a.v_scale;
    if constexpr (ALIBI) M += alibi_shift2(a, kvh * G + g, len, t_last);  // after the weights
    store_item_value<D, !QF32, FINAL>(a, qrow0 + g, p, d, o, M, L, single);
  }
  __syncthreads();
  if constexpr (FINAL)
    if (nparts > 1) finish_item_fused<D, !QF32, kGenW>(a, b, kvh, G, nparts);
}

template <int D, bool QF32, int KV, bool XP>
hipError_t launch_gen_d(const DecodePartialArgs& a, int grid_parts, hipStream_t s) {
  const long grid = (long)a.S * a.KVH * grid_parts;
  if (grid <= 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorNotSupported;
  const bool fin = a.out != nullptr, alibi = a.alibi != nullptr;
#define PKV_GEN_LAUNCH(F, A)                                                                                 \
  hipLaunchKernelGGL((decode_generic_kernel<D, QF32, KV, XP, F, A>), dim3((unsigned)grid), dim3(64 * kGenW), 0, s, a)
  if (fin) {
    if (alibi) PKV_GEN_LAUNCH(true, true); else PKV_GEN_LAUNCH(true, false);
  } else {
    if (alibi) PKV_GEN_LAUNCH(false, true); else PKV_GEN_LAUNCH(false, false);
  }
#undef PKV_GEN_LAUNCH
  return hipGetLastError();
}

template <bool QF32, int KV, bool XP>
hipError_t launch_gen_t(const DecodePartialArgs& a, int grid_parts, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_gen_d<64, QF32, KV, XP>(a, grid_parts, s);
    case 128: return launch_gen_d<128, QF32, KV, XP>(a, grid_parts, s);
    case 256: return launch_gen_d<256, QF32, KV, XP>(a, grid_parts, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_decode_generic(const DecodePartialArgs& a, int G, int grid_parts, bool xp, bool q_f32,
                                 hipStream_t s) {
  if (G < 1 || G > kGenG || a.bs < 1) return hipErrorNotSupported;
  if (q_f32) {
    if (a.kv_fp8) return hipErrorNotSupported;  // float8 caches are read with a bf16 query
    return xp ? launch_gen_t<true, 0, true>(a, grid_parts, s) : launch_gen_t<true, 0, false>(a, grid_parts, s);
  }
  if (a.kv_fp8)
    return xp ? launch_gen_t<false, 1, true>(a, grid_parts, s) : launch_gen_t<false, 1, false>(a, grid_parts, s);
  return xp ? launch_gen_t<false, 0, true>(a, grid_parts, s) : launch_gen_t<false, 0, false>(a, grid_parts, s);
}

}  // namespace pkv
