// MLA decode: one new token per sequence against its latent KV cache, split-K on the
// matrix cores, then the cross-split combine.
//
// What is computed is the MLA paged-prefill kernel's result (kernelindex gemini-2.5-pro
// Triton page, _mla_paged_prefill_causal_h16_ckv512_kpe64_ps1_kernel) for q_len = 1: the
// query of batch b sees all kv_len keys tok_j = kv_indices[kv_indptr[b] + j] (one token
// per page), x_j = sm_scale (q_nope . ckv_j + q_pe . kpe_j), O = softmax(x) . ckv and
// lse = log2 sum_j exp(x_j) (base 2). Split-K as on the decode pages: per split of `split`
// keys the partials m (natural log), l and the unnormalized accumulator, then the
// log-sum-exp-weighted combine (the decode reduce's one-wave row combine, 512 wide).
//
// gfx950 design (the operand layouts of the matrix-core GQA decode kernel, the 16 heads
// being one MFMA tile):
//  * One workgroup of 4 waves per (split, batch) item, the non-empty items on the lowest
//    workgroup ids (mla_item); a wave takes groups of
//    16 keys round-robin. Token ids are loaded two groups ahead, one per lane (lane l holds
//    the id of key l % 16 of the group).
//  * S^T = K Q^T: 18 k-steps of v_mfma_f32_16x16x32_bf16 (16 over ckv, 2 over kpe). A is
//    the 16 gathered key rows (lane: key l % 16, 8 dims per step), B is Q^T (lane: head
//    l % 16), loaded once per item.
//  * O^T = V^T P^T on v_mfma_f32_16x16x16_bf16 with V = the same keys' ckv rows (re-read,
//    an L2 hit; read with non-temporal loads as their last use): each lane loads 16-byte
//    chunks of 4 keys and byte permutes make the A operands; P^T comes straight from the
//    S^T accumulator, rounded to bf16.
//  * The 512-wide accumulator is 32 tiles x 4 floats per lane (one wave per SIMD); the
//    four waves merge through LDS in four 128-dim passes.
#include "common.h"
#include "decode_epilogue.h"
#include "mla_args.h"

namespace pkv {
namespace {

typedef __bf16 mla_bf16x8_t __attribute__((ext_vector_type(8)));
typedef short mla_s16x4_t __attribute__((ext_vector_type(4)));
typedef float mla_f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMdH = 16;     // heads (one MFMA tile)
constexpr int kMdDc = 512;   // ckv dims (= V dims)
constexpr int kMdDp = 64;    // kpe dims
constexpr int kMdKS = 18;    // 32-dim k-steps of the logits: 16 over ckv, 2 over kpe
constexpr int kMdNB = 4;     // 128-dim blocks of the output
constexpr int kMdNT = 32;    // 16-dim output tiles
constexpr int kMdW = 4;      // waves per item
constexpr float kMdRebase = 8.f;

PKV_DEVICE mla_f32x4_t md_mfma_k32(uint4 a, uint4 b, mla_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mla_bf16x8_t, a),
                                                 __builtin_bit_cast(mla_bf16x8_t, b), c, 0, 0, 0);
}
PKV_DEVICE mla_f32x4_t md_mfma_k16(uint2 a, uint2 b, mla_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mla_s16x4_t, a),
                                                   __builtin_bit_cast(mla_s16x4_t, b), c, 0, 0, 0);
}
// Element e (0..7) of chunks x and y as a bf16 pair (x[e], y[e]).
PKV_DEVICE uint32_t md_pick_pair(const uint4& x, const uint4& y, int e) {
  const uint32_t xa = e < 2 ? x.x : e < 4 ? x.y : e < 6 ? x.z : x.w;
  const uint32_t ya = e < 2 ? y.x : e < 4 ? y.y : e < 6 ? y.z : y.w;
  return (e & 1) ? pair_hi(xa, ya) : pair_lo(xa, ya);
}

struct MlaDecSmem {
  float red_acc[kMdW][kMdH][128];  // one 128-dim block of every wave's accumulator
  float red_m[kMdW][kMdH];
  float red_mref[kMdW][kMdH];
  float red_l[kMdW][kMdH];
};

// First key index and length of batch b's keys, clamped into kv_indices and to len_cap.
PKV_DEVICE void mla_batch_range(const MlaDecodeArgs& a, int b, int& kv0, int& len) {
  int k0 = a.kv_indptr[b], k1 = a.kv_indptr[b + 1];
  k0 = k0 < 0 ? 0 : (k0 > a.num_kv_indices ? a.num_kv_indices : k0);
  k1 = k1 < k0 ? k0 : (k1 > a.num_kv_indices ? a.num_kv_indices : k1);
  len = k1 - k0;
  len = len > a.len_cap ? a.len_cap : len;
  kv0 = uniform(k0);
  len = uniform(len);
}

constexpr int kMdDenseMaxB = 64 * kMdW;  // batches the in-workgroup item scan covers (one per thread)

// (batch, split) of this workgroup. The grid has one workgroup per pair (batch x gp, gp =
// ceil(max_kv_len / split) splits, so gridDim.x / batch = gp). With
// at most 256 batches the non-empty pairs come first, batch-major (workgroup i < N takes
// the i-th non-empty item), then the empty ones in the same order: the items take the
// lowest workgroup ids, which the dispatcher deals round-robin over the XCDs, so no XCD
// gets more items than its share. (Split-major, an XCD gets every split of the batches
// b = x mod 8, and a batch with more splits than the others pushes some XCD into a
// second round.) Larger batches: split-major.
PKV_DEVICE void mla_item(const MlaDecodeArgs& a, int& b, int& p) {
  const int bid = (int)blockIdx.x;
  if (a.batch > kMdDenseMaxB) {
    p = bid / a.batch;
    b = bid - p * a.batch;
    return;
  }
  __shared__ int s_pre[kMdDenseMaxB];  // inclusive prefix sum of the batches' non-empty splits
  __shared__ int s_hit[2];
  const int t = threadIdx.x;
  const int gp = (int)(gridDim.x / (unsigned)a.batch);
  int n = 0;  // non-empty splits of batch t in the grid: min(ceil(len / split), gp), len as in mla_batch_range
  if (t < a.batch) {
    int k0 = a.kv_indptr[t], k1 = a.kv_indptr[t + 1];
    k0 = k0 < 0 ? 0 : (k0 > a.num_kv_indices ? a.num_kv_indices : k0);
    k1 = k1 < k0 ? k0 : (k1 > a.num_kv_indices ? a.num_kv_indices : k1);
    int len = k1 - k0;
    len = len > a.len_cap ? a.len_cap : len;
    n = (len + a.split - 1) / a.split;
    n = n > gp ? gp : n;
  }
  s_pre[t] = n;
  if (t == 0) s_hit[0] = -1;
  __syncthreads();
  for (int off = 1; off < kMdDenseMaxB; off <<= 1) {
    const int v = t >= off ? s_pre[t - off] : 0;
    __syncthreads();
    s_pre[t] += v;
    __syncthreads();
  }
  const int incl = s_pre[t], excl = incl - n;
  const int total = s_pre[kMdDenseMaxB - 1];
  if (t < a.batch) {
    if (bid < total) {
      if (excl <= bid && bid < incl) {
        s_hit[0] = t;
        s_hit[1] = bid - excl;
      }
    } else {
      const int j = bid - total;            // j-th empty pair
      const int e0 = t * gp - excl;        // empty pairs of the batches before t
      if (e0 <= j && j < e0 + (gp - n)) {  // batch t's splits n .. gp-1
        s_hit[0] = t;
        s_hit[1] = n + (j - e0);
      }
    }
  }
  __syncthreads();
  b = s_hit[0];
  p = s_hit[1];
}

__global__ __launch_bounds__(64 * kMdW) void mla_decode_partial_kernel(MlaDecodeArgs a) {
  __shared__ MlaDecSmem sm;
  int b, p;
  mla_item(a, b, p);
  if (b < 0) return;  // uniform; not reached when the grid is batch x P pairs
  b = uniform(b);
  p = uniform(p);
  const int lane = threadIdx.x & 63;
  const int w = uniform((int)(threadIdx.x >> 6));
  const int g = lane >> 4;
  const int hl = lane & 15;
  int kv0, len;
  mla_batch_range(a, b, kv0, len);
  const int t_begin = p * a.split;
  if (t_begin >= len) {  // empty split: sentinel (PagedAttention V2 page, unused-partition branch)
    if ((int)threadIdx.x < kMdH) {
      const size_t si = ((size_t)b * kMdH + threadIdx.x) * a.P + p;
      a.m[si] = kNegInf;
      a.l[si] = 0.f;
    }
    return;  // uniform across the workgroup
  }
  const int t_end = min(t_begin + a.split, len);
  const int n_groups = (t_end - t_begin + 15) >> 4;
  const int n_my = n_groups - w > 0 ? (n_groups - w + kMdW - 1) / kMdW : 0;

  // B of S^T: Q^T, lane = head hl, dims 32 s + 8 g .. +8
  uint4 qb[kMdKS];
  {
    const char* qn = reinterpret_cast<const char*>(a.q_nope) + ((size_t)b * kMdH + hl) * (kMdDc * 2);
    const char* qp = reinterpret_cast<const char*>(a.q_pe) + ((size_t)b * kMdH + hl) * (kMdDp * 2);
#pragma unroll
    for (int s = 0; s < 16; ++s) qb[s] = ld16(qn + (s * 32 + g * 8) * 2);
#pragma unroll
    for (int s = 16; s < kMdKS; ++s) qb[s] = ld16(qp + ((s - 16) * 32 + g * 8) * 2);
  }

  // id of key t of this batch (t < len; past-the-end keys of a group read the last key),
  // clamped into the pool
  auto tok_id = [&](int t) -> int {
    t = t < len ? t : len - 1;
    const int id = a.kv_indices[kv0 + t];
    return id < 0 ? 0 : (id >= a.num_pages ? a.num_pages - 1 : id);
  };
  auto group_t0 = [&](int i) { return t_begin + 16 * (w + kMdW * i); };

  uint4 kr[kMdKS];
  uint4 vt[4][kMdNB];  // keys 4g + j, chunk 16 k + hl of the ckv row
  auto issue_k = [&](int id) {  // this lane's key (hl) of the group
    const char* crow = reinterpret_cast<const char*>(a.ckv) + (size_t)id * (kMdDc * 2);
    const char* prow = reinterpret_cast<const char*>(a.kpe) + (size_t)id * (kMdDp * 2);
#pragma unroll
    for (int s = 0; s < 16; ++s) kr[s] = ld16(crow + (s * 32 + g * 8) * 2);
#pragma unroll
    for (int s = 16; s < kMdKS; ++s) kr[s] = ld16(prow + ((s - 16) * 32 + g * 8) * 2);
  };
  auto issue_v = [&](int id) {  // keys 4g + j: their ids sit in lanes 4g + j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idj = __shfl(id, 4 * g + j, 64);
      const char* vrow = reinterpret_cast<const char*>(a.ckv) + (size_t)idj * (kMdDc * 2);
#pragma unroll
      for (int k = 0; k < kMdNB; ++k) vt[j][k] = ld16_nt(vrow + (16 * k + hl) * 16);
    }
  };

  mla_f32x4_t acc[kMdNT];
#pragma unroll
  for (int t = 0; t < kMdNT; ++t) acc[t] = mla_f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf, m_true = kNegInf, lsum = 0.f;  // head hl

  int id_cur = n_my > 0 ? tok_id(group_t0(0) + hl) : 0;
  int id_nxt = n_my > 1 ? tok_id(group_t0(1) + hl) : id_cur;
  if (n_my > 0) {
    issue_k(id_cur);
    issue_v(id_cur);
  }
  for (int i = 0; i < n_my; ++i) {
    const int id_nn = i + 2 < n_my ? tok_id(group_t0(i + 2) + hl) : id_nxt;
    const int ntok = min(16, t_end - group_t0(i));
    const bool more = i + 1 < n_my;

    mla_f32x4_t st = mla_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kMdKS; ++s) st = md_mfma_k32(kr[s], qb[s], st);
    if (more) issue_k(id_nxt);

    // S^T lane layout: head hl, keys 4g .. 4g+3 of the group
    float x[4];
    float tmax = kNegInf;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = (4 * g + j < ntok) ? st[j] * a.sm_scale_log2 : kNegInf;
      tmax = fmaxf(tmax, x[j]);
    }
    tmax = fmaxf(tmax, xor_lanes(tmax, 16));
    tmax = fmaxf(tmax, xor_lanes(tmax, 32));
    m_true = fmaxf(m_true, tmax);
    const bool rebase = m_true > m_ref + kMdRebase;  // true on the first group (m_ref = -inf)
    if (__builtin_amdgcn_ballot_w64(rebase) != 0) {
      const float nref = rebase ? m_true : m_ref;
      const float alpha = fast_exp2(m_ref - nref);
      m_ref = nref;
      lsum *= alpha;
#pragma unroll
      for (int t = 0; t < kMdNT; ++t) acc[t] *= alpha;
    }
    float pr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pr[j] = fast_exp2(x[j] - m_ref);
      lsum += pr[j];
    }
    const uint2 pb = make_uint2(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]));
#pragma unroll
    for (int k = 0; k < kMdNB; ++k)
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const uint2 av = make_uint2(md_pick_pair(vt[0][k], vt[1][k], n), md_pick_pair(vt[2][k], vt[3][k], n));
        acc[k * 8 + n] = md_mfma_k16(av, pb, acc[k * 8 + n]);
      }
    if (more) issue_v(id_nxt);
    id_cur = id_nxt;
    id_nxt = id_nn;
  }

  // ---- merge: l over the 4 lanes of a head, then the waves through LDS, 128 dims a pass
  lsum += xor_lanes(lsum, 16);
  lsum += xor_lanes(lsum, 32);
  if (g == 0) {
    sm.red_m[w][hl] = m_true;
    sm.red_mref[w][hl] = m_ref;
    sm.red_l[w][hl] = lsum;
  }
  const size_t row0 = (size_t)b * kMdH;
#pragma unroll
  for (int k = 0; k < kMdNB; ++k) {
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.red_acc[w][hl][8 * (4 * g + j) + n] = acc[k * 8 + n][j];
    __syncthreads();
    for (int idx = threadIdx.x; idx < kMdH * 128; idx += 64 * kMdW) {
      const int h = idx >> 7;
      const int dl = idx & 127;
      float M = sm.red_m[0][h];
#pragma unroll
      for (int v = 1; v < kMdW; ++v) M = fmaxf(M, sm.red_m[v][h]);
      float o = 0.f, L = 0.f;
#pragma unroll
      for (int v = 0; v < kMdW; ++v) {
        const float f = fast_exp2(sm.red_mref[v][h] - M);  // waves without keys carry -inf: f = 0
        o = fmaf(f, sm.red_acc[v][h][dl], o);
        L = fmaf(f, sm.red_l[v][h], L);
      }
      const size_t si = (row0 + h) * a.P + p;
      a.acc[si * kMdDc + k * 128 + dl] = o;
      if (k == 0 && dl == 0) {
        a.m[si] = M * kLn2;
        a.l[si] = L;
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void mla_decode_reduce_kernel(MlaDecodeArgs a) {
  const int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6);  // b * 16 + h
  if (row >= a.batch * kMdH) return;
  int kv0, len;
  mla_batch_range(a, row / kMdH, kv0, len);
  const int np = (len + a.split - 1) / a.split;
  reduce_row_wave<kMdDc, true>(a.acc, a.m, a.l, a.P, np, false, (size_t)row, a.out, a.lse, 1.f / kLn2);
}

}  // namespace

hipError_t launch_mla_decode(const MlaDecodeArgs& a, int grid_parts, hipStream_t s) {
  const long items = (long)a.batch * grid_parts;
  if (items > 0) {
    hipLaunchKernelGGL(mla_decode_partial_kernel, dim3((unsigned)items), dim3(64 * kMdW), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int rows = a.batch * kMdH;
  hipLaunchKernelGGL(mla_decode_reduce_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
