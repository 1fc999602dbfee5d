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
// gfx950 design:
//  * One workgroup of 4 waves per (split, batch) item, the non-empty items on the lowest
//    workgroup ids (mla_item). The item's keys go through LDS in tiles of 32: each wave
//    moves 8 keys' ckv rows (one 1 KiB transfer each) and their kpe rows (one transfer)
//    from global memory straight into LDS (global_load_lds, no registers), with the
//    layout, swizzles and operand reads of the prefill kernel (mla_tile.h). Four tile
//    buffers: while one tile is computed the next three are in flight, so the memory
//    system always holds about 100 KiB of this CU's keys.
//  * Every wave computes the whole S^T = K Q^T of a tile (36 v_mfma_f32_16x16x32_bf16:
//    two 16-key halves x 18 k-steps, Q^T in registers for the whole item) and the same
//    online softmax, so the four waves hold identical maxima and sums without exchanging
//    them; wave w then adds P V for output dims [128 w, 128 w + 128) only (8 MFMAs with
//    V^T from the transposing LDS read). The duplicated logits cost matrix-core time the
//    memory-bound loop has to spare, and keep the accumulator at 32 registers per lane.
//  * Every key is read from HBM once (V is the ckv row already in LDS), and the partial
//    rows are written straight from each wave's accumulator.
//  * With a counters array the combine runs in the same launch: the last workgroup to
//    finish a batch combines its splits (see the end of the kernel); without, a second
//    launch combines every batch.
#include "common.h"
#include "decode_epilogue.h"
#include "mla_args.h"
#include "mla_tile.h"

namespace pkv {
namespace {

using namespace mla;

constexpr int kMdH = 16;       // heads (one MFMA tile)
constexpr int kMdDc = 512;     // ckv dims (= V dims)
constexpr int kMdKSW = 9;      // 32-dim k-steps of the logits per wave: 8 over ckv, 1 over kpe
constexpr int kMdW = 4;        // waves per item
constexpr int kMdKT = 32;      // keys per tile
constexpr int kMdKPW = kMdKT / kMdW;      // keys of a tile each wave moves
constexpr int kMdDT = kMdDc / 16 / kMdW;  // 16-dim output tiles per wave
#ifndef PKV_MLA_DECODE_BUFFERS
#define PKV_MLA_DECODE_BUFFERS 4
#endif
constexpr int kMdNBUF = PKV_MLA_DECODE_BUFFERS;  // tile buffers
constexpr float kMdRebase = 8.f;
static_assert(kMdNBUF >= 3 && kMdNBUF <= 4, "tile buffers");

typedef int md_ids_t __attribute__((ext_vector_type(kMdKPW), aligned(4)));  // a wave's key ids

struct MlaDecSmem {
  uint4 ckv[kMdNBUF][kMdKT * kCkvStride];
  uint4 kpe[kMdNBUF][kMdKT * kKpeChunks];
  f32x4_t xs[2][kMdW / 2][64];  // logit shares of the current tile: [key half][dim half][lane]
};

// s_waitcnt vmcnt(n) for the counts the key loop needs (n transfers may stay in flight)
PKV_DEVICE void md_wait_transfers(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
    case 27: asm volatile("s_waitcnt vmcnt(27)" ::: "memory"); break;
    case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    case 48: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

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
// Also returns the batch's key range (kv0, len) as mla_batch_range gives it.
PKV_DEVICE void mla_item(const MlaDecodeArgs& a, int& b, int& p, int& kv0, int& len) {
  const int bid = (int)blockIdx.x;
  if (a.batch > kMdDenseMaxB) {
    p = bid / a.batch;
    b = bid - p * a.batch;
    mla_batch_range(a, b, kv0, len);
    return;
  }
  __shared__ int s_wtot[kMdW];  // non-empty splits of each wave's batches
  __shared__ int s_hit[4];
  const int t = threadIdx.x;
  const int gp = (int)(gridDim.x / (unsigned)a.batch);
  int n = 0;  // non-empty splits of batch t in the grid: min(ceil(len / split), gp), len as in mla_batch_range
  int k0 = 0, lt = 0;
  if (t < a.batch) {
    k0 = a.kv_indptr[t];
    int k1 = a.kv_indptr[t + 1];
    k0 = k0 < 0 ? 0 : (k0 > a.num_kv_indices ? a.num_kv_indices : k0);
    k1 = k1 < k0 ? k0 : (k1 > a.num_kv_indices ? a.num_kv_indices : k1);
    lt = k1 - k0;
    lt = lt > a.len_cap ? a.len_cap : lt;
    n = (lt + a.split - 1) / a.split;
    n = n > gp ? gp : n;
  }
  // inclusive scan of n over the workgroup: inside each wave by lane shifts, then the
  // totals of the waves before it
  const int lane = t & 63, wv = t >> 6;
  int incl = n;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wtot[wv] = incl;
  if (t == 0) s_hit[0] = -1;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int v = 0; v < kMdW; ++v) {
    incl += v < wv ? s_wtot[v] : 0;
    total += s_wtot[v];
  }
  const int excl = incl - n;
  if (t < a.batch) {
    if (bid < total) {
      if (excl <= bid && bid < incl) {
        s_hit[0] = t;
        s_hit[1] = bid - excl;
        s_hit[2] = k0;
        s_hit[3] = lt;
      }
    } else {
      const int j = bid - total;            // j-th empty pair
      const int e0 = t * gp - excl;        // empty pairs of the batches before t
      if (e0 <= j && j < e0 + (gp - n)) {  // batch t's splits n .. gp-1
        s_hit[0] = t;
        s_hit[1] = n + (j - e0);
        s_hit[2] = k0;
        s_hit[3] = lt;
      }
    }
  }
  __syncthreads();
  b = s_hit[0];
  p = s_hit[1];
  kv0 = uniform(s_hit[2]);
  len = uniform(s_hit[3]);
}

// One workgroup per CU (the tile buffers take most of the LDS): one wave per SIMD.
__global__ __launch_bounds__(64 * kMdW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_partial_kernel(MlaDecodeArgs a) {
  __shared__ __attribute__((aligned(16))) MlaDecSmem sm;
  int b, p, kv0, len;
  mla_item(a, b, p, kv0, len);
  if (b < 0) return;  // uniform; not reached when the grid is batch x P pairs
  b = uniform(b);
  p = uniform(p);
  const int lane = threadIdx.x & 63;
  const int w = uniform((int)(threadIdx.x >> 6));
  const int g = lane >> 4;
  const int hq = lane & 15;
  const int kh = w & 1;   // key half of the tile whose logits this wave sums
  const int dh = w >> 1;  // half of the 576 logit dims it sums them over
  const int t_begin = p * a.split;
  if (t_begin >= len) {  // empty split: sentinel (PagedAttention V2 page, unused-partition branch)
    if ((int)threadIdx.x < kMdH) {
      const size_t si = ((size_t)b * kMdH + threadIdx.x) * a.P + p;
      a.m[si] = kNegInf;
      a.l[si] = 0.f;
    }
    if (a.counters != nullptr && len == 0 && p == 0) {  // one launch: an empty batch's out = 0, lse = -inf
      uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + (size_t)b * kMdH * kMdDc;
      for (int i = threadIdx.x; i < kMdH * kMdDc; i += 64 * kMdW) orow[i] = 0;
      if ((int)threadIdx.x < kMdH) a.lse[(size_t)b * kMdH + threadIdx.x] = kNegInf;
    }
    return;  // uniform across the workgroup
  }
  const int n_keys = uniform(min(a.split, len - t_begin));
  const int n_kt = (n_keys + kMdKT - 1) / kMdKT;

  // ids of this wave's keys kMdKPW w .. of tile kt, through the scalar cache (keys past the
  // item's last one re-read that key; they are masked)
  const __attribute__((address_space(4))) int32_t* ids =
      (const __attribute__((address_space(4))) int32_t*)(a.kv_indices + kv0 + t_begin);
  auto load_ids = [&](int kt, int (&t)[kMdKPW]) {
    const int first = kt * kMdKT + kMdKPW * w;
    if (first + kMdKPW <= n_keys) {  // uniform: all ids exist, one scalar load
      const md_ids_t v = *reinterpret_cast<const __attribute__((address_space(4))) md_ids_t*>(ids + first);
#pragma unroll
      for (int k = 0; k < kMdKPW; ++k) t[k] = v[k];
    } else {
#pragma unroll
      for (int k = 0; k < kMdKPW; ++k) t[k] = ids[min(first + k, n_keys - 1)];
    }
  };
  // the first tiles' ids go out together, ahead of Q
  int tok_pre[kMdNBUF][kMdKPW];
#pragma unroll
  for (int j = 0; j < kMdNBUF; ++j)
    if (j < n_kt) load_ids(j, tok_pre[j]);

  // B of the logits: this wave's 9 k-steps of Q^T (lane = head hq): ckv dims
  // 32 (8 dh + j) + 8 g .. +8 for j < 8, then kpe dims 32 dh + 8 g .. +8
  uint4 qb[kMdKSW];
  {
    const char* qn = reinterpret_cast<const char*>(a.q_nope) + ((size_t)b * kMdH + hq) * (kMdDc * 2);
    const char* qp = reinterpret_cast<const char*>(a.q_pe) + ((size_t)b * kMdH + hq) * (64 * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) qb[j] = ld16(qn + ((8 * dh + j) * 32 + g * 8) * 2);
    qb[8] = ld16(qp + (dh * 32 + g * 8) * 2);
  }
  // Q must be in registers before the key loop: the compiler cannot see the tile
  // transfers, so a wait it placed for Q inside the loop would also wait for them.
#pragma unroll
  for (int j = 0; j < kMdKSW; ++j) asm volatile("" ::"v"(qb[j].x), "v"(qb[j].y), "v"(qb[j].z), "v"(qb[j].w));

  // one transfer per kpe row block when page * 128 fits in 32 bits, else one per key
  const bool kpe_block = a.num_pages <= (1 << 25);
  const int per_tile = kpe_block ? kMdKPW + 1 : 2 * kMdKPW;  // transfers per wave and tile
  auto issue_tile = [&](const int (&tok_in)[kMdKPW], int buf) {
    int tok[kMdKPW];
#pragma unroll
    for (int k = 0; k < kMdKPW; ++k) tok[k] = tok_in[k] < 0 ? 0 : (tok_in[k] >= a.num_pages ? a.num_pages - 1 : tok_in[k]);
#pragma unroll
    for (int k = 0; k < kMdKPW; ++k) {
      const int row_k = kMdKPW * w + k;
      const char* row = reinterpret_cast<const char*>(a.ckv) + (size_t)tok[k] * (kMdDc * 2);
      lds_dma16_s(row, (uint32_t)lane * 16, &sm.ckv[buf][row_k * kCkvStride]);
    }
    // kpe rows: lanes 8k .. 8k+7 move key k (lane i lands in position i of the wave's 8 rows
    // and loads global chunk (i & 7) ^ kpe_swz(row))
    const int kl = lane >> 3;
    const uint32_t chunk16 = (uint32_t)((lane & 7) ^ kpe_swz(kMdKPW * w + kl)) * 16;
    void* kpe_dst = &sm.kpe[buf][kMdKPW * w * kKpeChunks];
    if (kpe_block) {
      int tk = tok[0];
#pragma unroll
      for (int k = 1; k < kMdKPW; ++k) tk = kl == k ? tok[k] : tk;
      lds_dma16_s(a.kpe, (uint32_t)tk * (64 * 2) + chunk16, kpe_dst);
    } else {
#pragma unroll
      for (int k = 0; k < kMdKPW; ++k)
        if (kl == k) lds_dma16_s(reinterpret_cast<const char*>(a.kpe) + (size_t)tok[k] * (64 * 2), chunk16, kpe_dst);
    }
  };
  // every buffer is filled before the loop; tile kt's buffer takes tile kt + kMdNBUF at
  // the end of iteration kt
#pragma unroll
  for (int j = 0; j < kMdNBUF - 1; ++j)
    if (j < n_kt) issue_tile(tok_pre[j], j);
  int tok_next[kMdKPW];  // ids of the next tile to issue
#pragma unroll
  for (int k = 0; k < kMdKPW; ++k) tok_next[k] = tok_pre[kMdNBUF - 1][k];

  // this wave's share of a tile's logits: key rows 16 kh + hq (A), its 9 k-steps
  auto logits_partial = [&](int buf) {
    const uint4* crow = sm.ckv[buf] + (16 * kh + hq) * kCkvStride + g;
    const uint4* prow = sm.kpe[buf] + (16 * kh + hq) * kKpeChunks;
    uint4 ka[kMdKSW];
#pragma unroll
    for (int j = 0; j < 8; ++j) ka[j] = crow[(8 * dh + j) * 4];
    ka[8] = prow[(dh * 4 + g) ^ kpe_swz(hq)];
    f32x4_t st = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMdKSW; ++j) st = mfma16x16x32(ka[j], qb[j], st);
    sm.xs[kh][dh][lane] = st;
  };

  // O^T accumulators of this wave's dims: tile n holds rows j -> dim 16 (kMdDT w + n) + j, cols = heads
  f32x4_t acc[kMdDT];
#pragma unroll
  for (int n = 0; n < kMdDT; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf, m_true = kNegInf, lsum = 0.f;  // head hq (the same in every wave)
  // V^T reads: this lane is source lane 4k + q of its group (see the prefill kernel)
  const int vr = 4 * g + (hq >> 2);
  const int vcol = (int)(((uint32_t)hq >> 1) & 1) * 16 + (hq & 1) * 8;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt % kMdNBUF;
    md_wait_transfers(min(n_kt - 1 - kt, kMdNBUF - 2) * per_tile);  // this wave's transfers of tile kt
    __syncthreads();  // tile kt landed; every wave is done with tile kt - 1
    if (kt + kMdNBUF - 1 < n_kt) issue_tile(tok_next, (kt + kMdNBUF - 1) % kMdNBUF);
    logits_partial(buf);
    __syncthreads();  // the four shares of tile kt's logits are written
    f32x4_t st[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) st[hf] = sm.xs[hf][0][lane] + sm.xs[hf][1][lane];
    const int key0 = kt * kMdKT;
    float x[8];
    float tmax = kNegInf;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = (key0 + hf * 16 + 4 * g + i < n_keys) ? st[hf][i] * a.sm_scale_log2 : kNegInf;
        x[hf * 4 + i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, xor_lanes(tmax, 16));
    tmax = fmaxf(tmax, xor_lanes(tmax, 32));
    m_true = fmaxf(m_true, tmax);
    const bool rebase = m_true > m_ref + kMdRebase;
    if (__builtin_amdgcn_ballot_w64(rebase) != 0) {
      const float nref = rebase ? m_true : m_ref;
      const float alpha = fast_exp2(m_ref - nref);
      m_ref = nref;
      lsum *= alpha;
#pragma unroll
      for (int n = 0; n < kMdDT; ++n) acc[n] *= alpha;
    }
    float pr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr[e] = fast_exp2(x[e] - m_ref);
      lsum += pr[e];
    }
    const uint4 pb = make_uint4(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                                pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7]));
    const uint4* ckv = sm.ckv[buf];
    const char* vrow_lo = reinterpret_cast<const char*>(ckv + vr * kCkvStride) + vcol;
    const char* vrow_hi = reinterpret_cast<const char*>(ckv + (16 + vr) * kCkvStride) + vcol;
#pragma unroll
    for (int n = 0; n < kMdDT; ++n) {
      const int nn = kMdDT * w + n;
      const uint2 lo = lds_read_tr16(vrow_lo + nn * 32);
      const uint2 hi = lds_read_tr16(vrow_hi + nn * 32);
      acc[n] = mfma16x16x32(make_uint4(lo.x, lo.y, hi.x, hi.y), pb, acc[n]);
    }
    asm volatile("" ::: "memory");
    if (kt + kMdNBUF < n_kt) load_ids(kt + kMdNBUF, tok_next);
  }

  // ---- the partial rows, relative to the exact maximum m_true: l over the 4 lanes of a head
  lsum += xor_lanes(lsum, 16);
  lsum += xor_lanes(lsum, 32);
  const float f = fast_exp2(m_ref - m_true);  // <= 1; the first tile set m_ref, so both are finite
  const size_t si = ((size_t)b * kMdH + hq) * a.P + p;
  float* arow = a.acc + si * kMdDc;
  const bool fused = a.counters != nullptr;
#pragma unroll
  for (int n = 0; n < kMdDT; ++n) {
    const int d = 16 * (kMdDT * w + n) + 4 * g;  // lane: head hq, rows 4 g .. 4 g + 3 of the tile
    const float4 v = make_float4(acc[n][0] * f, acc[n][1] * f, acc[n][2] * f, acc[n][3] * f);
    if (fused) {  // rows another workgroup of this launch combines: stores every XCD sees
      const uint64_t* src = reinterpret_cast<const uint64_t*>(&v);
      uint64_t* dst = reinterpret_cast<uint64_t*>(arow + d);
      __hip_atomic_store(dst, src[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(dst + 1, src[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      *reinterpret_cast<float4*>(arow + d) = v;
    }
  }
  if (w == 0 && g == 0) {
    st_f32<true>(a.m + si, m_true * kLn2);
    st_f32<true>(a.l + si, lsum * f);
  }
  if (fused) {
    // one launch: the workgroup that completes batch b's count combines its 16 rows (four
    // heads per wave) and resets the count; the ordering is the GQA one-launch decode's
    // (coherent partial stores, each wave's own stores complete, a barrier, one
    // device-scope count, coherent loads by the last workgroup)
    const int gp = (int)(gridDim.x / (unsigned)a.batch);
    int np = (len + a.split - 1) / a.split;
    np = np > gp ? gp : np;
    __shared__ int s_last;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    int* ctr = a.counters + b;
    if (threadIdx.x == 0)
      s_last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == np - 1;
    __syncthreads();
    if (s_last) {
      for (int h = w; h < kMdH; h += kMdW)
        reduce_row_wave<kMdDc, true, true>(a.acc, a.m, a.l, a.P, np, false, (size_t)b * kMdH + h, a.out, a.lse,
                                            1.f / kLn2);
      if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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
  if (a.counters != nullptr) {
    if (items > 0) return hipSuccess;  // the partial kernel combined every batch
    // no key anywhere (max_kv_len = 0): the reduce writes every batch's zeros and -inf
  }
  const int rows = a.batch * kMdH;
  hipLaunchKernelGGL(mla_decode_reduce_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
