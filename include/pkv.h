/*
 * pkv.h -- C ABI of the paged-KV attention library for AMD Instinct MI355X (gfx950).
 *
 * Operations:
 *   paged_decode_partial  split-K single-token decode over a paged KV cache with
 *                         grouped-query heads: per-partition online-softmax partials
 *   paged_decode_reduce   log-sum-exp weighted combine of those partials
 *   paged_decode_split_partial, paged_decode_split_reduce
 *                         the same two phases with [FD]'s NUM_SPLITS page-aligned splits
 *   paged_decode          the whole decode in one launch (single pass when every
 *                         sequence fits one partition)
 *   paged_decode_partial_ex, paged_decode_ex
 *                         phase 1 / the one-launch decode with cache options: float8
 *                         e4m3 K/V caches with k_scale / v_scale, and ALiBi slopes
 *   paged_attention_v2    [PAv2]'s launcher: x-packed cache, 512-token partitions,
 *                         normalized partials (tmp_output, exp_sums, max_logits)
 *   mla_paged_prefill     MLA causal paged prefill (page_size 1), base-2 LSE
 *   mla_paged_prefill_pages  the same over pages of several tokens
 *   mla_paged_decode      MLA decode (one new token per sequence), split-K
 *   paged_decode_static   paged_decode for callers that cannot allocate: the partials
 *                         live in a static device array the library holds
 * and a measurement helper, pkv_read_bandwidth (a plain streaming read of a buffer),
 * that no part of the attention path uses.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer (HIP global memory) owned by the
 *     caller; every scalar is a host value. The library allocates nothing, keeps no
 *     pointer after returning, and launches asynchronously on `stream` (a hipStream_t
 *     passed as void*; NULL means the default stream). Results are ready when that
 *     stream has drained up to the launch.
 *   - Tensors are dense and row-major (C order) in the shapes given below.
 *   - The return value is a pkv_status. On any status other than PKV_OK nothing was
 *     launched (argument errors are found on the host before any HIP call), except
 *     PKV_EHIP, which reports a launch failure from the HIP runtime. pkv_last_error()
 *     returns a message for the calling thread's last non-OK status.
 *   - The library is stateless and reentrant; calls on different streams may overlap.
 *   - Values that live in device memory (lengths, page ids, index pointers) cannot be
 *     checked on the host. Kernels clamp every such value into the range that keeps
 *     their memory accesses inside the buffers described here, so a caller that breaks
 *     the stated contract gets unspecified numbers, never an out-of-bounds access.
 *
 * Sources for what is computed (pages named by title; no code taken from them):
 *   [PAv2]  "paged_attention_v2_triton.py -- CCCL-derived Triton PagedAttention V2"
 *           (dev.modelhub.org.cn, project_6): the two-kernel split design, the
 *           x-packed key layout, the empty-partition sentinel, the launcher arguments.
 *   [FD]    koas-w.github.io flash-decode post (2026-05-25): the token-major K/V
 *           layout, the unnormalized split partials and the combine formula.
 *   [MLA]   kernelindex.com, gemini-2.5-pro Triton MLA paged prefill
 *           (_mla_paged_prefill_causal_h16_ckv512_kpe64_ps1_kernel and _forward).
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,        /* an argument breaks the documented contract              */
  PKV_EUNSUPPORTED = 2,  /* a well-formed combination with no compiled kernel       */
  PKV_EHIP = 3           /* the HIP runtime reported an error for the launch        */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 /* K/V caches only, with a bf16 query */ } pkv_dtype;

typedef enum {
  /* K and V: [num_blocks, num_kv_heads, block_size, head_dim]            ([FD] kernel arguments) */
  PKV_KV_TOKEN_MAJOR = 0,
  /* K: [num_blocks, num_kv_heads, head_dim / x, block_size, x], x = 16 / sizeof(elem);
     V: [num_blocks, num_kv_heads, head_dim, block_size]                 ([PAv2] kernel arguments) */
  PKV_KV_XPACKED = 1
} pkv_kv_layout;

/*
 * paged_decode_partial -- phase 1 of split-K decode ([PAv2] _partition_attn_kernel,
 * [FD] _flash_decode_partial_kernel).
 *
 * For sequence b (length len_b = seq_lens[b]), query head h and partition p covering
 * tokens [p*ps, min((p+1)*ps, len_b)), with s_t = scale * <query[b,h,:], K_t> and kv
 * head h / G (G = num_heads / num_kv_heads):
 *   partial_m[b,h,p]     = max_t s_t                       (natural-log units)
 *   partial_l[b,h,p]     = sum_t exp(s_t - m)
 *   partial_acc[b,h,p,:] = sum_t exp(s_t - m) * V_t        (NOT divided by l)
 * Token t of sequence b is slot t % block_size of physical block
 * block_tables[b, t / block_size]. Each K/V page is read once for all G query heads.
 * A partition with p*ps >= len_b gets partial_m = -inf and partial_l = 0; its
 * partial_acc row is not written. Partitions p >= ceil(max_seq_len / ps) are not
 * touched at all.
 *
 *   query         [num_seqs, num_heads, head_dim], element type `dtype`
 *   key_cache,
 *   value_cache   page pools in `layout`, element type `dtype`, num_blocks blocks
 *   block_tables  [num_seqs, max_blocks_per_seq] int32; entries past
 *                 ceil(len_b / block_size) may hold anything (e.g. -1): they can be
 *                 loaded (within the row) but never select a page that is read
 *   seq_lens      [num_seqs] int32, 0 <= len_b <= max_seq_len
 *   partial_acc   [num_seqs, num_heads, max_num_partitions, head_dim] float32
 *   partial_m,
 *   partial_l     [num_seqs, num_heads, max_num_partitions] float32
 * PKV_EINVAL: a NULL pointer (NULL is allowed only when num_seqs == 0), a negative
 *   size, num_heads % num_kv_heads != 0, partition_size not a positive multiple of
 *   block_size, max_num_partitions < ceil(max_seq_len / partition_size),
 *   max_seq_len > max_blocks_per_seq * block_size.
 * PKV_EUNSUPPORTED: head_dim not in {64, 128, 256}; G > 16;
 *   num_seqs * num_kv_heads * ceil(max_seq_len / partition_size) above 2^31 - 1 (one
 *   workgroup each), or num_seqs * num_heads above 2^30 - 1.
 * bf16 groups of G < 8 (and G = 8 at head_dim 64 token-major) and every float32 group run
 *   on the vector ALUs; bf16 groups of 8 <= G <= 16 run on the matrix cores, padded to 16
 *   heads. Those kernels take 16-token blocks; any other block_size >= 1, and bf16 groups
 *   of 9-16 heads at head_dim 64 token-major, run on a generic kernel (not tuned).
 * num_seqs == 0 or max_seq_len == 0 launches nothing except the sentinel writes that
 *   the length rule above asks for.
 * A length above max_seq_len (a broken contract) is cut to max_num_partitions partitions,
 *   so no write lands outside the partial arrays.
 */
int paged_decode_partial(const void* query, int dtype,
                         const void* key_cache, const void* value_cache, int layout,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* seq_lens,
                         int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                         int block_size, int num_blocks,
                         float scale, int partition_size, int max_num_partitions,
                         int max_seq_len,
                         float* partial_acc, float* partial_m, float* partial_l,
                         void* stream);

/*
 * paged_decode_reduce -- phase 2 of split-K decode ([FD] _flash_decode_combine_kernel;
 * partition count per sequence as in [PAv2] _reduce_partitions_kernel).
 *
 * For each (b, h) over the P_b = ceil(len_b / partition_size) partitions of sequence b
 * (capped at max_num_partitions; partitions past P_b are never read):
 *   M = max_p m_p,  w_p = exp(m_p - M)
 *   out[b,h,:] = sum_p w_p * acc_p / sum_p w_p * l_p     rounded to out_dtype (RNE)
 *   lse[b,h]   = M + ln(sum_p w_p * l_p)                 natural log (if lse != NULL)
 * len_b == 0 gives out = 0 and lse = -inf.
 *
 *   partial_*  as written by paged_decode_partial
 *   out        [num_seqs, num_heads, head_dim], element type `out_dtype`
 *   lse        [num_seqs, num_heads] float32, or NULL
 * PKV_EINVAL: NULL pointers (other than lse), negative sizes, partition_size <= 0,
 *   max_num_partitions <= 0 with num_seqs > 0.
 * PKV_EUNSUPPORTED: head_dim not in {64, 128, 256}.
 */
int paged_decode_reduce(const float* partial_acc, const float* partial_m,
                        const float* partial_l, const int32_t* seq_lens,
                        int num_seqs, int num_heads, int head_dim,
                        int partition_size, int max_num_partitions,
                        void* out, int out_dtype, float* lse, void* stream);

/*
 * paged_decode_split_partial / paged_decode_split_reduce -- the two phases with [FD]'s
 * split policy (_flash_decode_partial_kernel: NUM_SPLITS splits per sequence, each a run
 * of whole pages).
 *
 * Sequence b's nb = ceil(len_b / block_size) pages are cut into runs of
 * bps = ceil(nb / num_splits) pages; split s covers tokens
 * [s*bps*block_size, min((s+1)*bps*block_size, len_b)). Splits starting at or past page nb
 * are empty (m = -inf, l = 0, acc row not written). Everything else is as in
 * paged_decode_partial / paged_decode_reduce, with num_splits in place of
 * max_num_partitions: partial_acc is [num_seqs, num_heads, num_splits, head_dim] and
 * partial_m, partial_l are [num_seqs, num_heads, num_splits]. The reduce reads the
 * ceil(nb / bps) non-empty splits of each sequence.
 * PKV_EINVAL: num_splits <= 0, and the conditions of the fixed-partition entry points.
 * PKV_EUNSUPPORTED: as paged_decode_partial.
 */
int paged_decode_split_partial(const void* query, int dtype,
                               const void* key_cache, const void* value_cache, int layout,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* seq_lens,
                               int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                               int block_size, int num_blocks, float scale, int num_splits,
                               int max_seq_len,
                               float* partial_acc, float* partial_m, float* partial_l,
                               void* stream);
int paged_decode_split_reduce(const float* partial_acc, const float* partial_m,
                              const float* partial_l, const int32_t* seq_lens,
                              int num_seqs, int num_heads, int head_dim,
                              int block_size, int num_splits,
                              void* out, int out_dtype, float* lse, void* stream);

/*
 * paged_decode -- the whole decode step in ONE launch ([FD] Decode_Paged_GQAAttention_Kernel
 * when a sequence has one partition; otherwise its split-K kernels with the combine run by
 * the last workgroup to finish a (sequence, kv head)).
 *
 * Computes what paged_decode_partial followed by paged_decode_reduce computes (or the
 * _split_ pair when num_splits > 0; partition_size is then ignored), writing
 *   out[b,h,:] (element type `dtype`, RNE) and lse[b,h] (natural log; lse may be NULL).
 * A sequence with a single partition is written straight from its workgroup. For longer
 * ones the partial arrays are scratch space owned by the caller (same shapes as for
 * paged_decode_partial, max_num_partitions >= num_splits under the split policy), and
 *   counters   [num_seqs * num_kv_heads] int32 of device memory, all ZERO on entry; the
 *              launch leaves them zero again, so one zeroed buffer serves every later
 *              call on the same stream. Calls that overlap in time need separate counters
 *              and partial arrays.
 * max_num_partitions == 1 is the single-pass form: every sequence is one partition whatever
 * its length (partition_size and num_splits are then ignored) and partial_acc, partial_m,
 * partial_l and counters may be NULL.
 * len_b == 0 gives out = 0 and lse = -inf.
 * PKV_EINVAL: as paged_decode_partial; NULL out; NULL partial arrays or counters when
 *   max_num_partitions > 1.
 * PKV_EUNSUPPORTED: as paged_decode_partial.
 */
int paged_decode(const void* query, int dtype,
                 const void* key_cache, const void* value_cache, int layout,
                 const int32_t* block_tables, int max_blocks_per_seq,
                 const int32_t* seq_lens,
                 int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                 int block_size, int num_blocks, float scale,
                 int partition_size, int num_splits, int max_num_partitions, int max_seq_len,
                 float* partial_acc, float* partial_m, float* partial_l, int32_t* counters,
                 void* out, float* lse, void* stream);

/*
 * paged_decode_partial_ex -- paged_decode_partial (num_splits == 0) or
 * paged_decode_split_partial (num_splits > 0, partition_size ignored) with cache options
 * ([PAv2]'s launcher names alibi_slopes, kv_cache_dtype, k_scale and v_scale without using
 * them; the readings here are those of paged_attention_v2 below):
 *   kv_dtype      `dtype` (the cache holds the query's type; k_scale = v_scale = 1), or
 *                 PKV_FP8_E4M3: key_cache / value_cache hold float8 e4m3 (OCP) values, one
 *                 byte each, in `layout` (x-packed with x = 16); the keys and values used are
 *                 k_scale and v_scale times the stored values. Needs a bf16 query.
 *   alibi_slopes  [num_heads] float32 device array, or NULL: the score of key t of sequence
 *                 b for head h becomes scale * <q, k_t> - alibi_slopes[h] * (len_b - 1 - t)
 *                 (Press, Smith and Lewis, ICLR 2022; the decoded token is the last position).
 * The partials are those of the plain entry points, with partial_m of each partition
 * including the bias; combine them with paged_decode_reduce / paged_decode_split_reduce.
 * Every other argument, status and bound is that of paged_decode_partial (max_num_partitions
 * >= num_splits under the split policy).
 * PKV_EINVAL additionally: kv_dtype neither `dtype` nor PKV_FP8_E4M3, scales not finite,
 *   scales other than 1 without a float8 cache. PKV_EUNSUPPORTED: a float8 cache with a
 *   query other than bf16.
 */
int paged_decode_partial_ex(const void* query, int dtype,
                            const void* key_cache, const void* value_cache, int layout,
                            int kv_dtype, float k_scale, float v_scale, const float* alibi_slopes,
                            const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* seq_lens,
                            int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                            int block_size, int num_blocks, float scale,
                            int partition_size, int num_splits, int max_num_partitions,
                            int max_seq_len,
                            float* partial_acc, float* partial_m, float* partial_l,
                            void* stream);

/*
 * paged_decode_ex -- paged_decode with the cache options of paged_decode_partial_ex
 * (kv_dtype, k_scale, v_scale, alibi_slopes; same meaning, checks and statuses). Everything
 * else, including the counters contract, is that of paged_decode.
 */
int paged_decode_ex(const void* query, int dtype,
                    const void* key_cache, const void* value_cache, int layout,
                    int kv_dtype, float k_scale, float v_scale, const float* alibi_slopes,
                    const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* seq_lens,
                    int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                    int block_size, int num_blocks, float scale,
                    int partition_size, int num_splits, int max_num_partitions, int max_seq_len,
                    float* partial_acc, float* partial_m, float* partial_l, int32_t* counters,
                    void* out, float* lse, void* stream);

/*
 * paged_attention_v2 -- [PAv2]'s paged_attention_v2_triton launcher as a C call: both
 * phases on `stream` with its fixed 512-token partitions and its x-packed cache layout
 * (PKV_KV_XPACKED), keeping its normalized partial form:
 *   max_logits[b,h,p]   = max_t s_t                      (natural-log units)
 *   exp_sums[b,h,p]     = sum_t exp(s_t - max_logits)
 *   tmp_output[b,h,p,:] = sum_t exp(s_t - max_logits) V_t / exp_sums   (float32)
 *   out[b,h,:] = sum_p exp(m_p - M) exp_sums_p tmp_output_p / sum_p exp(m_p - M) exp_sums_p
 * over the ceil(len_b / 512) partitions of sequence b (M = max_p m_p); `dtype` is the type
 * of query, caches and out. Empty partitions get max_logits = -inf, exp_sums = 0.
 *   out         [num_seqs, num_heads, head_size]
 *   exp_sums, max_logits  [num_seqs, num_heads, max_num_partitions] float32
 *   tmp_output  [num_seqs, num_heads, max_num_partitions, head_size] float32
 *   query [num_seqs, num_heads, head_size]; key_cache [num_blocks, num_kv_heads,
 *   head_size / x, block_size, x]; value_cache [num_blocks, num_kv_heads, head_size, block_size]
 * alibi_slopes  [num_heads] float32 device array, or NULL. [PAv2]'s launcher accepts the
 *   argument without defining or using it; here it is the published ALiBi bias (Press,
 *   Smith and Lewis, ICLR 2022): the score of key t of sequence b for head h becomes
 *   scale * <q, k_t> - alibi_slopes[h] * (len_b - 1 - t), the decoded token being the
 *   sequence's last position.
 * kv_cache_dtype  `dtype` (the cache holds the query's type; k_scale = v_scale = 1 required),
 *   or PKV_FP8_E4M3: key_cache / value_cache hold float8 e4m3 (OCP) values, x-packed with
 *   x = 16; the keys and values used are k_scale and v_scale times the stored values
 *   ([PAv2]'s launcher takes these three arguments without using them; this is the plainest
 *   reading, a per-tensor dequantization factor). Needs a bf16 query.
 * PKV_EINVAL / PKV_EUNSUPPORTED: as paged_decode_partial with partition_size = 512.
 */
int paged_attention_v2(void* out, float* exp_sums, float* max_logits, float* tmp_output,
                       const void* query, int dtype,
                       const void* key_cache, const void* value_cache,
                       int num_kv_heads, float scale,
                       const int32_t* block_tables, int max_blocks_per_seq,
                       const int32_t* seq_lens,
                       int num_seqs, int num_heads, int head_size, int block_size,
                       int num_blocks, int max_seq_len, int max_num_partitions,
                       const float* alibi_slopes, int kv_cache_dtype, float k_scale,
                       float v_scale, void* stream);

/*
 * mla_paged_prefill -- MLA causal paged prefill, page_size 1 ([MLA]).
 *
 * Batch b owns query rows r in [qo_indptr[b], qo_indptr[b+1]) and key tokens
 * kv_indices[kv_indptr[b] + j], j in [0, kv_len), kv_len = kv_indptr[b+1]-kv_indptr[b].
 * Row r = qo_indptr[b] + i sees keys j <= kv_len - q_len + i (bottom-right causal).
 *   x_j  = sm_scale * (q_nope[r,h,:] . ckv[tok_j,0,:] + q_pe[r,h,:] . kpe[tok_j,0,:])
 *   out[r,h,:] = sum_j softmax(x)_j * ckv[tok_j,0,:]         bfloat16 (RNE)
 *   lse[r,h]   = log2(sum_j exp(x_j))                         float32, base 2
 * A row that sees no key (kv_len == 0) gets out = 0 and lse = -inf.
 *
 *   q_nope     [total_q, num_heads, ckv_dim] bf16       q_pe  [total_q, num_heads, kpe_dim] bf16
 *   ckv_cache  [num_pages, page_size, ckv_dim] bf16     kpe_cache [num_pages, page_size, kpe_dim] bf16
 *   qo_indptr, kv_indptr  [batch + 1] int32, non-decreasing, qo_indptr[0] = kv_indptr[0] = 0,
 *              qo_indptr[batch] = total_q, kv_len >= q_len per batch, q_len <= max_q_len
 *   kv_indices [kv_indptr[batch]] int32 in [0, num_pages)
 *   out        [total_q, num_heads, ckv_dim] bf16        lse [total_q, num_heads] float32
 * PKV_EINVAL: NULL pointers with total_q > 0, negative sizes, sm_scale not finite.
 * PKV_EUNSUPPORTED: anything but num_heads = 16, ckv_dim = 512, kpe_dim = 64, page_size = 1
 *   (the shapes [MLA]'s _forward asserts). Any batch count: the kernel orders its tiles
 *   512 batches at a time.
 */
int mla_paged_prefill(const void* q_nope, const void* q_pe,
                      const void* ckv_cache, const void* kpe_cache,
                      const int32_t* qo_indptr, const int32_t* kv_indptr,
                      const int32_t* kv_indices,
                      int batch, int total_q, int max_q_len, int num_pages,
                      int num_heads, int ckv_dim, int kpe_dim, int page_size,
                      float sm_scale, void* out, float* lse, void* stream);

/*
 * mla_paged_prefill_pages -- mla_paged_prefill over pages of page_size >= 1 tokens.
 *
 * [MLA]'s kernel takes a PAGE_SIZE but its host wrapper asserts 1; this is the plainest
 * reading of its page-counting kv_indptr: batch b owns pages
 * kv_indices[kv_indptr[b] .. kv_indptr[b+1]-1] in order, every page holds page_size tokens
 * except the last, which holds kv_last_page_len[b] (page_size when kv_last_page_len is
 * NULL), so kv_len = (pages - 1) * page_size + last; key token j is slot j % page_size of
 * page kv_indices[kv_indptr[b] + j / page_size]. Everything else (causal alignment, logits,
 * output, base-2 LSE, empty rows) is as in mla_paged_prefill.
 *   ckv_cache [num_pages, page_size, 512] bf16    kpe_cache [num_pages, page_size, 64] bf16
 *   kv_indptr [batch + 1] int32 in pages, kv_indptr[batch] = num_kv_indices
 *   kv_indices [num_kv_indices] int32 page ids in [0, num_pages)
 *   kv_last_page_len [batch] int32 in [1, page_size], or NULL
 *   token_indptr [batch + 1] int32, token_rows [num_kv_indices * page_size] int32: device
 *              scratch owned by the caller; a first small kernel writes the token offsets
 *              and the pool row (page * page_size + slot) of every token there, then the
 *              page_size-1 prefill kernel runs on the pool viewed as
 *              [num_pages * page_size, 1, dim]. Their contents after the call are unspecified.
 * PKV_EINVAL / PKV_EUNSUPPORTED: as mla_paged_prefill (any page_size >= 1 is accepted), NULL
 *   scratch, num_pages * page_size or num_kv_indices * page_size of 2^31 or more.
 */
int mla_paged_prefill_pages(const void* q_nope, const void* q_pe,
                            const void* ckv_cache, const void* kpe_cache,
                            const int32_t* qo_indptr, const int32_t* kv_indptr,
                            const int32_t* kv_indices, const int32_t* kv_last_page_len,
                            int batch, int total_q, int max_q_len, int num_pages,
                            int num_kv_indices, int num_heads, int ckv_dim, int kpe_dim,
                            int page_size, float sm_scale,
                            int32_t* token_indptr, int32_t* token_rows,
                            void* out, float* lse, void* stream);

/*
 * mla_paged_decode -- MLA decode: one new token per sequence ([MLA]'s computation with
 * q_len = 1, so the token sees all kv_len keys), split-K over the latent cache on the
 * matrix cores, then the combine; one launch on `stream` with `counters`, else two.
 *
 * Batch b's keys are tok_j = kv_indices[kv_indptr[b] + j], j < kv_len_b (page_size 1).
 * Split s covers keys [s * split_tokens, min((s+1) * split_tokens, kv_len_b)); its partials
 * are m = max_j x_j (natural log), l = sum_j exp(x_j - m), acc = sum_j exp(x_j - m) ckv_j,
 * with x_j = sm_scale (q_nope[b,h] . ckv_j + q_pe[b,h] . kpe_j); splits past the last get
 * m = -inf, l = 0. The combine writes
 *   out[b,h,:] = sum_j softmax(x)_j ckv_j   bf16 (RNE);  lse[b,h] = log2 sum_j exp(x_j)
 * and kv_len_b = 0 gives out = 0, lse = -inf.
 *   q_nope [batch, 16, 512] bf16, q_pe [batch, 16, 64] bf16
 *   ckv_cache [num_pages, 1, 512] bf16, kpe_cache [num_pages, 1, 64] bf16
 *   kv_indptr [batch + 1] int32 (kv_indptr[batch] = num_kv_indices), kv_indices int32 in [0, num_pages)
 *   partial_acc [batch, 16, max_num_splits, 512], partial_m / partial_l [batch, 16, max_num_splits]
 *              float32: caller-owned scratch
 *   counters   [batch] int32 of device memory, all ZERO on entry and left zero: the combine
 *              then runs in the same launch (the last workgroup to finish a batch combines
 *              its splits); NULL: a second launch combines every batch. Calls that overlap
 *              in time need separate counters and partial arrays.
 *   out [batch, 16, 512] bf16, lse [batch, 16] float32 (base 2)
 * max_kv_len bounds every kv_len_b (a longer batch is cut to max_num_splits splits).
 * PKV_EINVAL: NULL pointers with batch > 0, non-positive split_tokens or max_num_splits,
 *   max_num_splits < ceil(max_kv_len / split_tokens), num_pages = 0 with batch > 0.
 * PKV_EUNSUPPORTED: anything but num_heads 16, ckv_dim 512, kpe_dim 64, page_size 1.
 */
int mla_paged_decode(const void* q_nope, const void* q_pe,
                     const void* ckv_cache, const void* kpe_cache,
                     const int32_t* kv_indptr, const int32_t* kv_indices,
                     int batch, int num_pages, int num_kv_indices, int max_kv_len,
                     int num_heads, int ckv_dim, int kpe_dim, int page_size, float sm_scale,
                     int split_tokens, int max_num_splits,
                     float* partial_acc, float* partial_m, float* partial_l, int32_t* counters,
                     void* out, float* lse, void* stream);

/*
 * paged_decode_static -- paged_decode without any allocation, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Not a computation of its own: the same two phases as
 * paged_decode_partial + paged_decode_reduce (or their _split_ forms when num_splits > 0),
 * with the partials kept in a scratch array that the library holds in device memory.
 *
 * Arguments are those of paged_decode without the partial arrays and counters:
 * out[b,h,:] (element type `dtype`, RNE) and lse[b,h] (natural log; lse may be NULL).
 * The partitions are ceil(max_seq_len / partition_size) fixed ones, or num_splits splits
 * under the NUM_SPLITS policy; with a single fixed partition the single-pass kernel runs
 * and no scratch is touched.
 *
 * Scratch: one static array of PKV_STATIC_SCRATCH_BYTES per GPU, held until the process
 * ends. The partials need num_seqs * num_heads * partitions * (head_dim + 2) floats (each
 * of the three arrays rounded up to 256 bytes); larger calls are refused with
 * PKV_EUNSUPPORTED before anything is launched. Every call on one GPU uses that GPU's
 * array: calls that overlap in time on the same GPU (other streams, other host threads)
 * race on it and must be serialised by the caller. Phase 1 writes every partial row or
 * sentinel phase 2 reads, so no call depends on what an earlier one left there.
 * The function calls no allocating routine. The first call on each device looks up the
 * array's device address (hipGetSymbolAddress) and keeps it.
 * PKV_EINVAL / PKV_EUNSUPPORTED: as paged_decode_partial; NULL out; scratch too small.
 */
#define PKV_STATIC_SCRATCH_BYTES (64u * 1024u * 1024u)
int paged_decode_static(const void* query, int dtype,
                        const void* key_cache, const void* value_cache, int layout,
                        const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* seq_lens,
                        int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                        int block_size, int num_blocks, float scale,
                        int partition_size, int num_splits, int max_seq_len,
                        void* out, float* lse, void* stream);

/* Measurement helper, not part of the attention path: reads `bytes` bytes of device memory
 * at `buf` once, as a plain streaming read (16-byte loads, grid-stride over the buffer), on
 * `stream`. Timing it gives the read bandwidth the GPU sustains for the simplest access
 * pattern, the reference point the decode kernels' paged gathers are compared with.
 *   buf   device memory, 16-byte aligned; bytes a multiple of 16 (0: nothing to do)
 *   sink  one uint32 of device memory, written only in a case that never arises in
 *         practice (it keeps the loads from being optimised away); its value is unspecified
 * PKV_EINVAL: NULL buf or sink with bytes > 0, misaligned buf, bytes not a multiple of 16.
 * PKV_EHIP: the launch failed. */
int pkv_read_bandwidth(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Message for the calling thread's last non-OK status ("" if none). Never NULL. */
const char* pkv_last_error(void);

/* Library version string, e.g. "pkv 0.1.0 gfx950". */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
