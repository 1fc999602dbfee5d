// MLA causal paged prefill (page_size 1) on gfx950 matrix cores.
//
// What it computes is the kernel of the kernelindex gemini-2.5-pro Triton page
// (_mla_paged_prefill_causal_h16_ckv512_kpe64_ps1_kernel): for query row r of batch b
// (row i of that batch) and head h, over the keys j <= kv_len - q_len + i of the batch,
//   x_j = sm_scale * (q_nope . ckv_j + q_pe . kpe_j),   O = sum_j softmax(x)_j ckv_j,
//   lse = log2 sum_j exp(x_j),
// with O = 0 and lse = -inf for a row that sees no key.
//
// gfx950 design (not the page's: it recomputes the 576-wide logits once per 512-dim
// output slice and runs two passes; here it is one pass with an online softmax):
//  * A workgroup is kQT = 8 waves = 8 consecutive query tokens of one batch; a wave owns
//    the 16 heads of its token (16 MFMA rows). Tiles are handed out longest first (batches
//    by KV length, last tile of a batch first, in chunks of kMaxBatch batches). One workgroup fills a CU (two
//    waves per SIMD, 256 registers each: 128 hold the wave's O).
//  * Keys come in tiles of 32: the 32 [ckv | kpe] rows (1152 B each) are gathered through
//    kv_indices straight into LDS with global_load_lds_dwordx4 (no staging registers),
//    double-buffered. Each wave moves 4 keys: one transfer per key for its 1 KiB ckv row
//    (scalar address, page ids from one scalar load) and one 32-lane transfer for the
//    four keys' kpe rows (scalar base, per-lane offsets), so the gather costs almost no
//    vector instructions.
//  * The gather rate a CU sustains bounds the kernel (measured: more tiles in flight did
//    not help, fewer bytes per token did), so as many tokens as the register file allows
//    share each gathered tile. The transfers are issued as inline assembly, invisible to the
//    compiler's wait insertion, so tile kt+1 lands while tile kt is computed; the kernel
//    waits for them itself before the barrier that publishes a buffer.
//  * S^T = K . Q^T with v_mfma_f32_16x16x32_bf16: A = a K row slice read from LDS, B = the
//    wave's Q^T kept in registers for the whole key loop (18 k-steps over 576 dims).
//  * The S^T accumulator layout (lane = head, 4 keys per lane) is exactly the B operand
//    of O^T = V^T . P^T, so P never moves. V^T operands (16 consecutive dims x 8 keys per
//    16-lane group) come straight from the row-major ckv tile through gfx950's transposing
//    LDS read (ds_read_b64_tr_b16): inside a 16-lane group, source lane 4k + q points at 4
//    dims (4q .. 4q+3) of key k, and lane j receives dim j of keys 0..3. Two such reads
//    give a lane its 8 keys, with no permutes in registers.
//  * Softmax in base 2 (sm_scale * log2 e folded into one multiply), so lse comes out in
//    base 2 directly. The per-head max is reduced across the 4 lanes of a head with
//    lane permutes; l and O are re-based lazily (only when the max outgrows the
//    reference by 2^8), with a wave-uniform branch.
#include "common.h"
#include "mla_args.h"
#include "mla_tile.h"

namespace pkv {

namespace {

using namespace mla;

constexpr int kH = 16;          // heads (MFMA rows / cols)
constexpr int kDc = 512;        // ckv dims (also V dims)
constexpr int kDp = 64;         // kpe dims
constexpr int kQT = 8;          // query tokens per workgroup (one per wave)
constexpr int kNT = kQT * 64;   // threads per workgroup
constexpr int kKT = 32;         // keys per tile
constexpr int kKeysPerWave = kKT / kQT;      // keys of a tile gathered by each wave
static_assert(kKeysPerWave * kQT == kKT, "tile shape");
constexpr int kMaxBatch = kMlaMaxBatch;  // batches per chunk of the tile list
constexpr float kMlaRebase = 8.f;

typedef int idsv_t __attribute__((ext_vector_type(kKeysPerWave), aligned(4)));  // a wave's page ids

}  // namespace

// CHUNKED: more than kMaxBatch batches (the tile list is built chunk by chunk); the
// single-chunk instance keeps the chunk bookkeeping out of the key loop's scalar registers.
template <bool CHUNKED>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(2, 2)))  // 2 waves per SIMD
void mla_prefill_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(16))) uint4 s_ckv[2][kKT * kCkvStride];  // double-buffered key tiles
  __shared__ __attribute__((aligned(16))) uint4 s_kpe[2][kKT * kKpeChunks];
  __shared__ int s_tiles[kMaxBatch + 1];  // exclusive prefix of query tiles, by sorted position
  __shared__ int s_border[kMaxBatch];     // batch at each sorted position
  __shared__ int s_kvl[kMaxBatch];        // clamped kv_len per batch
  __shared__ int s_wave[kQT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform((int)(tid >> 6));
  const int B = a.batch;

  // ---- tile list: tiles of kQT query tokens, built for kMaxBatch batches at a time (the
  // list is held in LDS). Inside such a chunk, batches go longest KV first (ties by index)
  // and, inside a batch, the last (longest) tile first, so the longest tiles start in the
  // first wave of workgroups and the short ones fill in behind them. The chunks' lists are
  // concatenated: workgroup s takes tiles s, s + R, s + 2R, ... of the whole list (R
  // workgroups), so a workgroup that finishes a chunk early starts the next one at once
  // and no workgroup waits for another.
  const int R = gridDim.x;
  int carry = 0;  // tiles of the earlier chunks, mod R
  for (int c0 = 0; c0 < (CHUNKED ? B : 1); c0 += kMaxBatch) {
    const int CB = CHUNKED ? min(kMaxBatch, B - c0) : B;
    {
      const int per = (CB + kNT - 1) / kNT;
      const int i0 = tid * per;
      for (int i = i0; i < i0 + per && i < CB; ++i) {
        const int kl = a.kv_indptr[c0 + i + 1] - a.kv_indptr[c0 + i];
        s_kvl[i] = kl < 0 ? 0 : kl;
      }
      __syncthreads();
      for (int i = i0; i < i0 + per && i < CB; ++i) {
        const int ki = s_kvl[i];
        int rank = 0;
        for (int j = 0; j < CB; ++j) rank += (s_kvl[j] > ki) || (s_kvl[j] == ki && j < i);
        s_border[rank] = c0 + i;
      }
      __syncthreads();
      // exclusive prefix of tile counts over the sorted positions
      int local = 0;
      for (int k = i0; k < i0 + per && k < CB; ++k) {
        const int i = s_border[k];
        const int ql = a.qo_indptr[i + 1] - a.qo_indptr[i];
        local += ql > 0 ? (ql + kQT - 1) / kQT : 0;
      }
      int x = local;
  #pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      if (lane == 63) s_wave[w] = x;
      __syncthreads();
      int base = 0;
      for (int v = 0; v < w; ++v) base += s_wave[v];
      int run = base + x - local;
      for (int k = i0; k < i0 + per && k < CB; ++k) {
        s_tiles[k] = run;
        const int i = s_border[k];
        const int ql = a.qo_indptr[i + 1] - a.qo_indptr[i];
        run += ql > 0 ? (ql + kQT - 1) / kQT : 0;
      }
      if (tid == 0) {
        int total = 0;
        for (int v = 0; v < kQT; ++v) total += s_wave[v];
        s_tiles[CB] = total;
      }
      __syncthreads();
    }
    const int n_tiles = uniform(s_tiles[CB]);
    const int first = !CHUNKED ? (int)blockIdx.x : (blockIdx.x >= carry ? blockIdx.x - carry : blockIdx.x + R - carry);

    for (int tile = first; tile < n_tiles; tile += R) {
      // sorted position (then batch) of this tile
      int lo = 0, hi = CB;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_tiles[mid] <= tile) lo = mid; else hi = mid;
      }
      const int pos = uniform(lo);
      const int b = uniform(s_border[pos]);
      const int q0 = a.qo_indptr[b], q1 = a.qo_indptr[b + 1];
      const int k0 = a.kv_indptr[b];
      const int q_len = q1 - q0;
      int kv_len = a.kv_indptr[b + 1] - k0;
      kv_len = kv_len < 0 ? 0 : kv_len;
      const int nt_b = s_tiles[pos + 1] - s_tiles[pos];
      const int t_in_b = uniform(nt_b - 1 - (tile - s_tiles[pos]));  // last tile of the batch first
      const int i_tok = t_in_b * kQT + w;                             // this wave's query token
      const bool has_row = i_tok < q_len;
      const int r = q0 + i_tok;
      const int prefix = kv_len - q_len;
      // keys visible to this wave's row: [0, vis)
      int vis = has_row ? prefix + i_tok + 1 : 0;
      vis = vis < 0 ? 0 : (vis > kv_len ? kv_len : vis);
      // keys the workgroup needs: up to its last valid row
      const int i_last = min(t_in_b * kQT + kQT - 1, q_len - 1);
      int n_keys = prefix + i_last + 1;
      n_keys = n_keys < 0 ? 0 : (n_keys > kv_len ? kv_len : n_keys);
      n_keys = uniform(n_keys);
      const int n_kt = (n_keys + kKT - 1) / kKT;

      // ---- Q^T operands (B of S^T = K Q^T): lane = (head l%16, dims (l/16)*8 .. +8 of each k-step)
      const int hq = lane & 15;
      const int g = lane >> 4;
      uint4 qb[18];
      if (has_row) {
        const char* qn = reinterpret_cast<const char*>(a.q_nope) + ((size_t)r * kH + hq) * kDc * 2;
        const char* qp = reinterpret_cast<const char*>(a.q_pe) + ((size_t)r * kH + hq) * kDp * 2;
  #pragma unroll
        for (int s = 0; s < 16; ++s) qb[s] = ld16(qn + (s * 32 + g * 8) * 2);
  #pragma unroll
        for (int s = 0; s < 2; ++s) qb[16 + s] = ld16(qp + (s * 32 + g * 8) * 2);
      } else {
  #pragma unroll
        for (int s = 0; s < 18; ++s) qb[s] = make_uint4(0, 0, 0, 0);
      }
      // Q must be in registers before the key loop: the compiler cannot see the tile
      // transfers, so a wait it placed for Q inside the loop would also wait for them.
  #pragma unroll
      for (int s = 0; s < 18; ++s) asm volatile("" ::"v"(qb[s].x), "v"(qb[s].y), "v"(qb[s].z), "v"(qb[s].w));

      // ---- gather of one key tile into LDS buffer `buf`: wave w moves keys kKeysPerWave w ..
      // kKeysPerWave (w + 1) - 1 of the tile (keys past the workgroup's last one re-read its
      // last key; they are masked). The page ids of tile kt+2 are read through the scalar
      // cache during tile kt.
      const __attribute__((address_space(4))) int32_t* ids =
          (const __attribute__((address_space(4))) int32_t*)(a.kv_indices + k0);
      int tok_next[kKeysPerWave];
      auto load_ids = [&](int kt) {
        const int first = kt * kKT + kKeysPerWave * w;
        int t[kKeysPerWave];
        if (first + kKeysPerWave <= n_keys) {  // uniform: all ids exist, one scalar load
          const idsv_t v = *reinterpret_cast<const __attribute__((address_space(4))) idsv_t*>(ids + first);
  #pragma unroll
          for (int k = 0; k < kKeysPerWave; ++k) t[k] = v[k];
        } else {  // the workgroup's last tile: keys past its last one re-read that key
          const int last = n_keys > 0 ? n_keys - 1 : 0;
  #pragma unroll
          for (int k = 0; k < kKeysPerWave; ++k) t[k] = ids[min(first + k, last)];
        }
  #pragma unroll
        for (int k = 0; k < kKeysPerWave; ++k) tok_next[k] = t[k];  // clamped when used
      };
      // LDS position i of a ckv row holds global chunk i
      auto issue_tile = [&](int buf) {
        int tok[kKeysPerWave];
  #pragma unroll
        for (int k = 0; k < kKeysPerWave; ++k)
          tok[k] = tok_next[k] < 0 ? 0 : (tok_next[k] >= a.num_pages ? a.num_pages - 1 : tok_next[k]);
  #pragma unroll
        for (int k = 0; k < kKeysPerWave; ++k) {
          const int row_k = kKeysPerWave * w + k;
          const char* row = reinterpret_cast<const char*>(a.ckv) + (size_t)tok[k] * (kDc * 2);
          lds_dma16_s(row, (uint32_t)lane * 16, &s_ckv[buf][row_k * kCkvStride]);
        }
        // kpe rows of the wave's keys: lanes 8k .. 8k+7 move key k (lane i lands in slot i,
        // i.e. position i & 7 of row kKeysPerWave w + k, and loads global chunk
        // (i & 7) ^ kpe_swz(row)). One transfer from the kpe array with a per-lane 32-bit
        // offset while page * 128 fits in 32 bits; else one transfer per key.
        const int kl = lane >> 3;
        const uint32_t chunk16 = (uint32_t)((lane & 7) ^ kpe_swz(kKeysPerWave * w + kl)) * 16;
        void* kpe_dst = &s_kpe[buf][kKeysPerWave * w * kKpeChunks];
        if (a.num_pages <= (1 << 25)) {  // uniform
          int tk = tok[0];
  #pragma unroll
          for (int k = 1; k < kKeysPerWave; ++k) tk = kl == k ? tok[k] : tk;
          if (kl < kKeysPerWave) lds_dma16_s(a.kpe, (uint32_t)tk * (kDp * 2) + chunk16, kpe_dst);
        } else {
  #pragma unroll
          for (int k = 0; k < kKeysPerWave; ++k)
            if (kl == k)
              lds_dma16_s(reinterpret_cast<const char*>(a.kpe) + (size_t)tok[k] * (kDp * 2), chunk16, kpe_dst);
        }
      };

      // O^T accumulators: tile n holds rows j -> dim 16 n + j, cols = heads
      f32x4_t acc[32];
  #pragma unroll
      for (int i = 0; i < 32; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      float m_ref = kNegInf, m_true = kNegInf, lsum = 0.f;  // per head (lane's column)

      // tile kt + 1 is issued at the top of tile kt, into the buffer tile kt - 1 released
      if (n_kt > 0) {
        load_ids(0);
        issue_tile(0);
        if (n_kt > 1) load_ids(1);
      }
      for (int kt = 0; kt < n_kt; ++kt) {
        const int buf = kt & 1;
        vmcnt0();          // this wave's transfers of tile kt
        __syncthreads();   // every wave's transfers of tile kt landed; everyone is done with tile kt-1
        if (kt + 1 < n_kt) issue_tile(buf ^ 1);
        const int key0 = kt * kKT;
        if (key0 < vis) {  // uniform: else this wave's row sees none of these keys
          // ---- S^T for two 16-key halves
          f32x4_t st[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
          const uint4* ckv = s_ckv[buf];
          const uint4* kpe = s_kpe[buf];
          // A: key row (l%16) of each half, dims (l/16)*8.. of each k-step; the two halves'
          // chains interleave so each LDS read has the other chain's MFMA to hide behind
          const uint4* crow = ckv + hq * kCkvStride + g;
          const uint4* prow = kpe + hq * kKpeChunks;
  #pragma unroll
          for (int s = 0; s < 16; ++s) {
            const uint4 a0 = crow[s * 4];
            const uint4 a1 = crow[16 * kCkvStride + s * 4];
            st[0] = mfma16x16x32(a0, qb[s], st[0]);
            st[1] = mfma16x16x32(a1, qb[s], st[1]);
          }
  #pragma unroll
          for (int s = 0; s < 2; ++s) {
            const uint4 a0 = prow[(s * 4 + g) ^ kpe_swz(hq)];
            const uint4 a1 = prow[16 * kKpeChunks + ((s * 4 + g) ^ kpe_swz(hq))];
            st[0] = mfma16x16x32(a0, qb[16 + s], st[0]);
            st[1] = mfma16x16x32(a1, qb[16 + s], st[1]);
          }
          // next ids: the scalar load completes under the softmax (any later LDS wait would
          // also wait for it)
          if (kt + 2 < n_kt) load_ids(kt + 2);
          // lane holds keys key0 + hf*16 + 4g + i for head hq
          float x[8];
          float tmax = kNegInf;
  #pragma unroll
          for (int hf = 0; hf < 2; ++hf)
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int kj = key0 + hf * 16 + 4 * g + i;
              const float v = (kj < vis) ? st[hf][i] * a.sm_scale_log2 : kNegInf;
              x[hf * 4 + i] = v;
              tmax = fmaxf(tmax, v);
            }
          tmax = fmaxf(tmax, xor_lanes(tmax, 16));
          tmax = fmaxf(tmax, xor_lanes(tmax, 32));
          m_true = fmaxf(m_true, tmax);
          const bool rebase = m_true > m_ref + kMlaRebase;  // also true on the first tile (m_ref = -inf)
          if (__builtin_amdgcn_ballot_w64(rebase) != 0) {   // wave-uniform branch
            const float nref = rebase ? m_true : m_ref;
            const float alpha = fast_exp2(m_ref - nref);
            m_ref = nref;
            lsum *= alpha;
  #pragma unroll
            for (int i = 0; i < 32; ++i) acc[i] *= alpha;
          }
          float p[8];
  #pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = fast_exp2(x[e] - m_ref);
            lsum += p[e];
          }
          // P^T as the B operand: k-slot e <-> key (e < 4 ? 4g + e : 16 + 4g + e - 4)
          const uint4 pb = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                      pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));

          // ---- O^T += V^T P^T over 32 blocks of 16 dims. This lane is source lane 4k + q of
          // its group: it points at dims 16 n + 4 q .. +3 of keys 4g + k (k-slots 0..3 of the
          // group) and 16 + 4g + k (k-slots 4..7), the key order of P^T.
          // (chunk 2n + ((hq >> 1) & 1) of a row, at byte (hq & 1) * 8 in it)
          const int vr = 4 * g + (hq >> 2);
          const int vcol = (int)(((uint32_t)hq >> 1) & 1) * 16 + (hq & 1) * 8;
          const char* vrow_lo = reinterpret_cast<const char*>(ckv + vr * kCkvStride) + vcol;
          const char* vrow_hi = reinterpret_cast<const char*>(ckv + (16 + vr) * kCkvStride) + vcol;
  #pragma unroll
          for (int n = 0; n < 32; ++n) {
            const uint2 lo = lds_read_tr16(vrow_lo + n * 32);
            const uint2 hi = lds_read_tr16(vrow_hi + n * 32);
            acc[n] = mfma16x16x32(make_uint4(lo.x, lo.y, hi.x, hi.y), pb, acc[n]);
          }
        } else if (kt + 2 < n_kt) {
          load_ids(kt + 2);
        }
      }

      // ---- finish: total l per head over the 4 lanes of the column, normalize, store
      lsum += xor_lanes(lsum, 16);
      lsum += xor_lanes(lsum, 32);
      if (has_row) {
        const bool any = lsum > 0.f;
        const float inv = any ? 1.f / lsum : 0.f;
        // lane: head hq, rows 4g .. 4g+3 of tile n -> dims 16 n + 4 g .. +3
        uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + ((size_t)r * kH + hq) * kDc;
  #pragma unroll
        for (int n = 0; n < 32; ++n) {
          uint2 o;
          o.x = pack_bf16x2(acc[n][0] * inv, acc[n][1] * inv);
          o.y = pack_bf16x2(acc[n][2] * inv, acc[n][3] * inv);
          *reinterpret_cast<uint2*>(orow + 16 * n + 4 * g) = o;
        }
        if (g == 0) a.lse[(size_t)r * kH + hq] = any ? m_ref + __log2f(lsum) : kNegInf;
      }
      __syncthreads();  // LDS buffers are reused by the next tile of work
    }
    if constexpr (CHUNKED) {
      carry = (int)(((long)carry + n_tiles) % R);
      __syncthreads();  // every wave has read this chunk's list before the next one is built
    }
  }
}

hipError_t launch_mla_prefill(const MlaArgs& a, hipStream_t s) {
  // upper bound of query tiles: total_q / kQT + one partial tile per batch
  const long bound = (long)a.total_q / kQT + a.batch;
  const int cap = dense_grid_cap();
  const int grid = (int)(bound < cap ? bound : cap);
  if (grid <= 0) return hipSuccess;
  if (a.batch > kMaxBatch)
    hipLaunchKernelGGL(mla_prefill_kernel<true>, dim3(grid), dim3(kNT), 0, s, a);
  else
    hipLaunchKernelGGL(mla_prefill_kernel<false>, dim3(grid), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
