// C ABI of the library (include/pkv.h): argument validation on the host, dispatch to a
// compiled kernel instance, launch on the caller's stream. Nothing here allocates.
#include "../../include/pkv.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <algorithm>
#include <cstdio>
#include <mutex>
#include <string>

#include "decode_args.h"
#include "mla_args.h"
#include "probe_args.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

}  // namespace

namespace pkv {
// Records the calling thread's message for pkv_last_error() and returns `code`; shared with
// the entry points defined in other translation units.
int set_last_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}
}  // namespace pkv

namespace {

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  if (e == hipErrorNotSupported) return fail(PKV_EUNSUPPORTED, "%s: no compiled kernel for these arguments", what);
  return fail(PKV_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

constexpr int kPagedAttentionV2Partition = 512;  // the PagedAttention V2 launcher's fixed PARTITION_SIZE

}  // namespace

namespace pkv {
// Workgroup cap of the dense decode launches: 16 per compute unit of the current device
// (queried once per device). Grids up to this size are dispatched whole and balanced by
// the hardware; larger work lists are strided over the capped grid.
int dense_grid_cap() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 4096;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
#ifndef PKV_GRID_PER_CU
#define PKV_GRID_PER_CU 16
#endif
    cached[dev] = cus * PKV_GRID_PER_CU;
  }
  return cached[dev];
}

int resident_grid(const void* kernel, int block_threads, size_t dyn_lds) {
  struct Entry {
    const void* kernel;
    int dev, threads;
    size_t lds;
    int grid;
  };
  static Entry cache[256];
  static int n_cache = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return dense_grid_cap();
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n_cache; ++i)
      if (cache[i].kernel == kernel && cache[i].dev == dev && cache[i].threads == block_threads &&
          cache[i].lds == dyn_lds)
        return cache[i].grid;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, dyn_lds) != hipSuccess ||
      per_cu <= 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    return dense_grid_cap();
  }
  const int grid = per_cu * cus;
  std::lock_guard<std::mutex> lock(mu);
  if (n_cache < 256) cache[n_cache++] = Entry{kernel, dev, block_threads, dyn_lds, grid};
  return grid;
}
}  // namespace pkv

namespace {

// Partition map and outputs of one phase-1 launch (see DecodePartialArgs).
struct Phase1Mode {
  int partition_size;   // tokens per partition (ignored when num_splits > 0)
  int num_splits;       // > 0: NUM_SPLITS page-aligned policy
  int normalize;        // store acc / l
  void* out;            // final mode when not null
  float* lse;
  int* counters;
  const float* alibi;   // [num_heads] ALiBi slopes or null
  int kv_fp8;           // K/V pools in float8 e4m3 (bf16 query)
  float k_scale, v_scale;
};

// Validation and dispatch shared by every decode entry point. `who` names the entry point
// in error messages.
int decode_phase1(const char* who, const void* query, int dtype, const void* key_cache, const void* value_cache,
                  int layout, const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens,
                  int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                  float scale, int max_num_partitions, int max_seq_len, float* partial_acc, float* partial_m,
                  float* partial_l, const Phase1Mode& mode, void* stream) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_EINVAL, "%s: unknown dtype %d", who, dtype);
  if (layout != PKV_KV_TOKEN_MAJOR && layout != PKV_KV_XPACKED)
    return fail(PKV_EINVAL, "%s: unknown layout %d", who, layout);
  if (num_seqs < 0) return fail(PKV_EINVAL, "%s: num_seqs < 0", who);
  if (num_seqs == 0) return PKV_OK;
  const bool final_mode = mode.out != nullptr;
  // a one-launch decode with one partition per sequence keeps no partials
  const bool keeps_partials = !final_mode || max_num_partitions > 1;
  if (!query || !key_cache || !value_cache || !block_tables || !seq_lens ||
      (keeps_partials && (!partial_acc || !partial_m || !partial_l)))
    return fail(PKV_EINVAL, "%s: NULL pointer argument", who);
  if (final_mode && max_num_partitions > 1 && !mode.counters)
    return fail(PKV_EINVAL, "%s: counters must not be NULL when max_num_partitions > 1", who);
  if (num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_num_partitions <= 0 || max_seq_len < 0)
    return fail(PKV_EINVAL, "%s: sizes must be positive (max_seq_len >= 0)", who);
  if (num_heads % num_kv_heads != 0)
    return fail(PKV_EINVAL, "%s: num_heads %d is not a multiple of num_kv_heads %d", who, num_heads, num_kv_heads);
  if (mode.num_splits < 0) return fail(PKV_EINVAL, "%s: num_splits < 0", who);
  if (mode.num_splits == 0 && keeps_partials && (mode.partition_size <= 0 || mode.partition_size % block_size != 0))
    return fail(PKV_EINVAL, "%s: partition_size %d is not a positive multiple of block_size %d", who,
                mode.partition_size, block_size);
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_EINVAL, "%s: max_seq_len %d exceeds max_blocks_per_seq * block_size", who, max_seq_len);
  int grid_parts;
  if (final_mode && !keeps_partials) {
    grid_parts = 1;  // single pass: one partition per sequence, the partition map is not used
  } else if (mode.num_splits > 0) {
    grid_parts = mode.num_splits;
    if (max_num_partitions < mode.num_splits)
      return fail(PKV_EINVAL, "%s: max_num_partitions %d < num_splits %d", who, max_num_partitions,
                  mode.num_splits);
  } else {
    grid_parts = (int)(((int64_t)max_seq_len + mode.partition_size - 1) / mode.partition_size);
    if (grid_parts > max_num_partitions)
      return fail(PKV_EINVAL, "%s: max_num_partitions %d < ceil(max_seq_len / partition_size) = %d", who,
                  max_num_partitions, grid_parts);
  }
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "%s: scale is not finite", who);
  const bool bf16 = dtype == PKV_BF16;
  if (!(head_dim == 64 || head_dim == 128 || head_dim == 256))
    return fail(PKV_EUNSUPPORTED, "%s: head_dim %d", who, head_dim);
  const int G = num_heads / num_kv_heads;
  if (G > 16) return fail(PKV_EUNSUPPORTED, "%s: %d query heads per kv head", who, G);
  if ((int64_t)num_seqs * num_kv_heads * std::max(grid_parts, 1) > INT32_MAX ||
      (int64_t)num_seqs * num_heads > INT32_MAX / 2)
    return fail(PKV_EUNSUPPORTED, "%s: grid too large (sequences x kv heads x partitions > 2^31 - 1)", who);
  if (grid_parts == 0 && !final_mode) return PKV_OK;  // every sequence is empty: nothing is touched
  if (grid_parts == 0) grid_parts = 1;  // final mode still writes the empty sequences' zeros

  pkv::DecodePartialArgs a;
  a.q = query; a.kc = key_cache; a.vc = value_cache;
  a.bt = block_tables; a.lens = seq_lens; a.mb = max_blocks_per_seq;
  a.S = num_seqs; a.H = num_heads; a.KVH = num_kv_heads; a.D = head_dim; a.NB = num_blocks;
  a.scale_log2 = scale * 1.4426950408889634f;
  const int64_t table_tokens = (int64_t)max_blocks_per_seq * block_size;
  if (final_mode && !keeps_partials) {
    // one partition per sequence whatever its length: the whole table row
    a.ps = (int)std::min<int64_t>(table_tokens, INT32_MAX / 2 / block_size * block_size);
    a.nsplit = 0;
    grid_parts = 1;
  } else {
    a.ps = mode.num_splits > 0 ? block_size : mode.partition_size;
    a.nsplit = mode.num_splits;
  }
  a.ppp = a.ps / block_size;
  a.bs = block_size;
  // lengths are cut to the partitions this launch covers (a length past max_seq_len breaks
  // the contract; it must still not push a partition index past the launched grid)
  a.len_cap = (int)std::min<int64_t>(table_tokens, a.nsplit > 0 ? table_tokens : (int64_t)grid_parts * a.ps);
  a.normalize = mode.normalize;
  a.alibi = mode.alibi;
  a.kv_fp8 = mode.kv_fp8;
  a.v_scale = mode.v_scale;
  if (mode.kv_fp8) a.scale_log2 *= mode.k_scale;
  a.P = max_num_partitions;
  a.acc = partial_acc; a.m = partial_m; a.l = partial_l;
  a.out = mode.out; a.lse = mode.lse; a.counters = mode.counters;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  hipError_t e;
  const bool xp = layout == PKV_KV_XPACKED;
  if (block_size != 16) {  // the tuned kernels take 16-token pages
    e = pkv::launch_decode_generic(a, G, grid_parts, xp, !bf16, s);
  } else if (bf16 && G >= 8) {
    e = xp ? pkv::launch_decode_mfma_bf16_xp(a, G, grid_parts, s)
           : pkv::launch_decode_mfma_bf16_tm(a, G, grid_parts, s);
  } else if (bf16) {
    e = xp ? pkv::launch_decode_valu_bf16_xp(a, G, grid_parts, s)
           : pkv::launch_decode_valu_bf16_tm(a, G, grid_parts, s);
  } else {
    e = xp ? pkv::launch_decode_valu_f32_xp(a, G, grid_parts, s)
           : pkv::launch_decode_valu_f32_tm(a, G, grid_parts, s);
  }
  std::string what = std::string(who) + " launch";
  return hip_status(e, what.c_str());
}

int decode_phase2(const char* who, const float* partial_acc, const float* partial_m, const float* partial_l,
                  const int32_t* seq_lens, int num_seqs, int num_heads, int head_dim, int partition_size,
                  int num_splits, int block_size, int normalized, int max_num_partitions, void* out, int out_dtype,
                  float* lse, void* stream) {
  if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) return fail(PKV_EINVAL, "%s: unknown out_dtype %d", who, out_dtype);
  if (num_seqs < 0 || num_heads < 0 || head_dim <= 0) return fail(PKV_EINVAL, "%s: bad sizes", who);
  if (num_seqs == 0 || num_heads == 0) return PKV_OK;
  if (!partial_acc || !partial_m || !partial_l || !seq_lens || !out)
    return fail(PKV_EINVAL, "%s: NULL pointer argument", who);
  if (num_splits < 0 || block_size <= 0 || max_num_partitions <= 0 || (num_splits == 0 && partition_size <= 0))
    return fail(PKV_EINVAL, "%s: partition_size (or num_splits), block_size and max_num_partitions must be positive",
                who);
  if (!(head_dim == 64 || head_dim == 128 || head_dim == 256))
    return fail(PKV_EUNSUPPORTED, "%s: head_dim %d", who, head_dim);
  if ((int64_t)num_seqs * num_heads > (int64_t)INT32_MAX / 2) return fail(PKV_EUNSUPPORTED, "%s: too many rows", who);
  pkv::DecodeReduceArgs a;
  a.acc = partial_acc; a.m = partial_m; a.l = partial_l; a.lens = seq_lens;
  a.S = num_seqs; a.H = num_heads; a.D = head_dim; a.P = max_num_partitions;
  a.ps = num_splits > 0 ? block_size : partition_size;
  a.nsplit = num_splits; a.bs = block_size; a.normalized = normalized;
  a.out = out; a.lse = lse;
  std::string what = std::string(who) + " launch";
  return hip_status(pkv::launch_decode_reduce(a, out_dtype == PKV_BF16, reinterpret_cast<hipStream_t>(stream)),
                    what.c_str());
}

// The cache options of the _ex entry points and the PagedAttention V2 launcher: the K/V
// element type (the query's, or float8 e4m3 with a bf16 query) and its dequantization scales.
int check_cache_options(const char* who, int dtype, int kv_dtype, float k_scale, float v_scale) {
  if (kv_dtype != dtype && kv_dtype != PKV_FP8_E4M3)
    return fail(PKV_EINVAL, "%s: kv_dtype %d is neither the query dtype nor PKV_FP8_E4M3", who, kv_dtype);
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PKV_EINVAL, "%s: k_scale / v_scale not finite", who);
  if (kv_dtype != PKV_FP8_E4M3 && (k_scale != 1.f || v_scale != 1.f))
    return fail(PKV_EINVAL, "%s: k_scale / v_scale apply to a float8 cache only", who);
  if (kv_dtype == PKV_FP8_E4M3 && dtype != PKV_BF16)
    return fail(PKV_EUNSUPPORTED, "%s: a float8 cache needs a bf16 query", who);
  return PKV_OK;
}

}  // namespace

extern "C" int paged_decode_partial(const void* query, int dtype, const void* key_cache,
                                    const void* value_cache, int layout,
                                    const int32_t* block_tables, int max_blocks_per_seq,
                                    const int32_t* seq_lens, int num_seqs, int num_heads,
                                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                    float scale, int partition_size, int max_num_partitions,
                                    int max_seq_len, float* partial_acc, float* partial_m,
                                    float* partial_l, void* stream) {
  const Phase1Mode mode{partition_size, 0, 0, nullptr, nullptr, nullptr, nullptr, 0, 1.f, 1.f};
  return decode_phase1("paged_decode_partial", query, dtype, key_cache, value_cache, layout, block_tables,
                       max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, max_num_partitions, max_seq_len, partial_acc, partial_m, partial_l, mode,
                       stream);
}

extern "C" int paged_decode_reduce(const float* partial_acc, const float* partial_m,
                                   const float* partial_l, const int32_t* seq_lens, int num_seqs,
                                   int num_heads, int head_dim, int partition_size,
                                   int max_num_partitions, void* out, int out_dtype, float* lse,
                                   void* stream) {
  return decode_phase2("paged_decode_reduce", partial_acc, partial_m, partial_l, seq_lens, num_seqs, num_heads,
                       head_dim, partition_size, 0, 16, 0, max_num_partitions, out, out_dtype, lse, stream);
}

extern "C" int paged_decode_split_partial(const void* query, int dtype, const void* key_cache,
                                          const void* value_cache, int layout, const int32_t* block_tables,
                                          int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs,
                                          int num_heads, int num_kv_heads, int head_dim, int block_size,
                                          int num_blocks, float scale, int num_splits, int max_seq_len,
                                          float* partial_acc, float* partial_m, float* partial_l, void* stream) {
  if (num_splits <= 0) return fail(PKV_EINVAL, "paged_decode_split_partial: num_splits must be positive");
  const Phase1Mode mode{0, num_splits, 0, nullptr, nullptr, nullptr, nullptr, 0, 1.f, 1.f};
  return decode_phase1("paged_decode_split_partial", query, dtype, key_cache, value_cache, layout, block_tables,
                       max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, num_splits, max_seq_len, partial_acc, partial_m, partial_l, mode, stream);
}

extern "C" int paged_decode_split_reduce(const float* partial_acc, const float* partial_m, const float* partial_l,
                                         const int32_t* seq_lens, int num_seqs, int num_heads, int head_dim,
                                         int block_size, int num_splits, void* out, int out_dtype, float* lse,
                                         void* stream) {
  if (num_splits <= 0) return fail(PKV_EINVAL, "paged_decode_split_reduce: num_splits must be positive");
  return decode_phase2("paged_decode_split_reduce", partial_acc, partial_m, partial_l, seq_lens, num_seqs,
                       num_heads, head_dim, 0, num_splits, block_size, 0, num_splits, out, out_dtype, lse, stream);
}

extern "C" int paged_decode(const void* query, int dtype, const void* key_cache, const void* value_cache,
                            int layout, const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* seq_lens, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                            int block_size, int num_blocks, float scale, int partition_size, int num_splits,
                            int max_num_partitions, int max_seq_len, float* partial_acc, float* partial_m,
                            float* partial_l, int32_t* counters, void* out, float* lse, void* stream) {
  if (!out) return fail(PKV_EINVAL, "paged_decode: NULL pointer argument (out)");
  const Phase1Mode mode{partition_size, num_splits, 0, out, lse, counters, nullptr, 0, 1.f, 1.f};
  return decode_phase1("paged_decode", query, dtype, key_cache, value_cache, layout, block_tables,
                       max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, max_num_partitions, max_seq_len, partial_acc, partial_m, partial_l, mode,
                       stream);
}

extern "C" int paged_decode_partial_ex(const void* query, int dtype, const void* key_cache, const void* value_cache,
                                       int layout, int kv_dtype, float k_scale, float v_scale,
                                       const float* alibi_slopes, const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* seq_lens, int num_seqs, int num_heads, int num_kv_heads,
                                       int head_dim, int block_size, int num_blocks, float scale, int partition_size,
                                       int num_splits, int max_num_partitions, int max_seq_len, float* partial_acc,
                                       float* partial_m, float* partial_l, void* stream) {
  const int cst = check_cache_options("paged_decode_partial_ex", dtype, kv_dtype, k_scale, v_scale);
  if (cst != PKV_OK) return cst;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3;
  const Phase1Mode mode{partition_size, num_splits, 0, nullptr, nullptr, nullptr, alibi_slopes, fp8 ? 1 : 0, k_scale,
                        v_scale};
  return decode_phase1("paged_decode_partial_ex", query, dtype, key_cache, value_cache, layout, block_tables,
                       max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, max_num_partitions, max_seq_len, partial_acc, partial_m, partial_l, mode,
                       stream);
}

extern "C" int paged_decode_ex(const void* query, int dtype, const void* key_cache, const void* value_cache,
                               int layout, int kv_dtype, float k_scale, float v_scale, const float* alibi_slopes,
                               const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens,
                               int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                               int num_blocks, float scale, int partition_size, int num_splits,
                               int max_num_partitions, int max_seq_len, float* partial_acc, float* partial_m,
                               float* partial_l, int32_t* counters, void* out, float* lse, void* stream) {
  if (!out) return fail(PKV_EINVAL, "paged_decode_ex: NULL pointer argument (out)");
  const int cst = check_cache_options("paged_decode_ex", dtype, kv_dtype, k_scale, v_scale);
  if (cst != PKV_OK) return cst;
  const bool fp8 = kv_dtype == PKV_FP8_E4M3;
  const Phase1Mode mode{partition_size, num_splits, 0, out, lse, counters, alibi_slopes, fp8 ? 1 : 0, k_scale,
                        v_scale};
  return decode_phase1("paged_decode_ex", query, dtype, key_cache, value_cache, layout, block_tables,
                       max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, max_num_partitions, max_seq_len, partial_acc, partial_m, partial_l, mode,
                       stream);
}

extern "C" int paged_attention_v2(void* out, float* exp_sums, float* max_logits, float* tmp_output,
                                  const void* query, int dtype, const void* key_cache, const void* value_cache,
                                  int num_kv_heads, float scale, const int32_t* block_tables,
                                  int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int num_heads,
                                  int head_size, int block_size, int num_blocks, int max_seq_len,
                                  int max_num_partitions, const float* alibi_slopes, int kv_cache_dtype,
                                  float k_scale, float v_scale, void* stream) {
  const int cst = check_cache_options("paged_attention_v2", dtype, kv_cache_dtype, k_scale, v_scale);
  if (cst != PKV_OK) return cst;
  const bool fp8 = kv_cache_dtype == PKV_FP8_E4M3;
  const Phase1Mode mode{kPagedAttentionV2Partition, 0, 1, nullptr, nullptr, nullptr, alibi_slopes, fp8 ? 1 : 0,
                        k_scale, v_scale};
  int st = decode_phase1("paged_attention_v2", query, dtype, key_cache, value_cache, PKV_KV_XPACKED, block_tables,
                         max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                         num_blocks, scale, max_num_partitions, max_seq_len, tmp_output, max_logits, exp_sums, mode,
                         stream);
  if (st != PKV_OK) return st;
  if (!out) return fail(PKV_EINVAL, "paged_attention_v2: NULL pointer argument (out)");
  return decode_phase2("paged_attention_v2", tmp_output, max_logits, exp_sums, seq_lens, num_seqs, num_heads,
                       head_size, kPagedAttentionV2Partition, 0, block_size, 1, max_num_partitions, out, dtype,
                       nullptr, stream);
}

extern "C" int mla_paged_prefill(const void* q_nope, const void* q_pe, const void* ckv_cache,
                                 const void* kpe_cache, const int32_t* qo_indptr,
                                 const int32_t* kv_indptr, const int32_t* kv_indices, int batch,
                                 int total_q, int max_q_len, int num_pages, int num_heads,
                                 int ckv_dim, int kpe_dim, int page_size, float sm_scale,
                                 void* out, float* lse, void* stream) {
  if (batch < 0 || total_q < 0 || max_q_len < 0 || num_pages < 0 || num_heads <= 0 || ckv_dim <= 0 ||
      kpe_dim <= 0 || page_size <= 0)
    return fail(PKV_EINVAL, "mla_paged_prefill: bad sizes");
  if (!std::isfinite(sm_scale)) return fail(PKV_EINVAL, "mla_paged_prefill: sm_scale is not finite");
  if (num_heads != 16 || ckv_dim != 512 || kpe_dim != 64 || page_size != 1)
    return fail(PKV_EUNSUPPORTED,
                "mla_paged_prefill: compiled for num_heads 16, ckv_dim 512, kpe_dim 64, page_size 1 "
                "(got %d, %d, %d, %d)", num_heads, ckv_dim, kpe_dim, page_size);
  if (total_q == 0 || batch == 0) return PKV_OK;
  if (!q_nope || !q_pe || !ckv_cache || !kpe_cache || !qo_indptr || !kv_indptr || !kv_indices || !out || !lse)
    return fail(PKV_EINVAL, "mla_paged_prefill: NULL pointer argument");
  if (max_q_len <= 0) return fail(PKV_EINVAL, "mla_paged_prefill: max_q_len must be positive when total_q > 0");
  if (num_pages <= 0) return fail(PKV_EINVAL, "mla_paged_prefill: num_pages must be positive when total_q > 0");
  pkv::MlaArgs a;
  a.q_nope = q_nope; a.q_pe = q_pe; a.ckv = ckv_cache; a.kpe = kpe_cache;
  a.qo_indptr = qo_indptr; a.kv_indptr = kv_indptr; a.kv_indices = kv_indices;
  a.batch = batch; a.total_q = total_q; a.max_q_len = max_q_len; a.num_pages = num_pages;
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  a.out = out; a.lse = lse;
  return hip_status(pkv::launch_mla_prefill(a, reinterpret_cast<hipStream_t>(stream)), "mla_paged_prefill launch");
}

extern "C" int mla_paged_prefill_pages(const void* q_nope, const void* q_pe, const void* ckv_cache,
                                       const void* kpe_cache, const int32_t* qo_indptr, const int32_t* kv_indptr,
                                       const int32_t* kv_indices, const int32_t* kv_last_page_len, int batch,
                                       int total_q, int max_q_len, int num_pages, int num_kv_indices,
                                       int num_heads, int ckv_dim, int kpe_dim, int page_size, float sm_scale,
                                       int32_t* token_indptr, int32_t* token_rows, void* out, float* lse,
                                       void* stream) {
  if (batch < 0 || total_q < 0 || max_q_len < 0 || num_pages < 0 || num_kv_indices < 0 || num_heads <= 0 ||
      ckv_dim <= 0 || kpe_dim <= 0 || page_size <= 0)
    return fail(PKV_EINVAL, "mla_paged_prefill_pages: bad sizes");
  if (!std::isfinite(sm_scale)) return fail(PKV_EINVAL, "mla_paged_prefill_pages: sm_scale is not finite");
  if (num_heads != 16 || ckv_dim != 512 || kpe_dim != 64)
    return fail(PKV_EUNSUPPORTED,
                "mla_paged_prefill_pages: compiled for num_heads 16, ckv_dim 512, kpe_dim 64 (got %d, %d, %d)",
                num_heads, ckv_dim, kpe_dim);
  if ((int64_t)num_pages * page_size >= INT32_MAX || (int64_t)num_kv_indices * page_size >= INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "mla_paged_prefill_pages: more than 2^31 tokens");
  if (total_q == 0 || batch == 0) return PKV_OK;
  if (!q_nope || !q_pe || !ckv_cache || !kpe_cache || !qo_indptr || !kv_indptr || !kv_indices || !out || !lse ||
      !token_indptr || !token_rows)
    return fail(PKV_EINVAL, "mla_paged_prefill_pages: NULL pointer argument");
  if (max_q_len <= 0) return fail(PKV_EINVAL, "mla_paged_prefill_pages: max_q_len must be positive when total_q > 0");
  if (num_pages <= 0) return fail(PKV_EINVAL, "mla_paged_prefill_pages: num_pages must be positive when total_q > 0");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  pkv::MlaPagesArgs e;
  e.kv_indptr = kv_indptr; e.kv_indices = kv_indices; e.last_len = kv_last_page_len;
  e.batch = batch; e.num_kv_indices = num_kv_indices; e.num_pages = num_pages; e.ps = page_size;
  e.tok_indptr = token_indptr; e.tok_rows = token_rows;
  int st = hip_status(pkv::launch_mla_expand_pages(e, s), "mla_paged_prefill_pages index launch");
  if (st != PKV_OK) return st;
  pkv::MlaArgs a;
  a.q_nope = q_nope; a.q_pe = q_pe; a.ckv = ckv_cache; a.kpe = kpe_cache;
  a.qo_indptr = qo_indptr; a.kv_indptr = token_indptr; a.kv_indices = token_rows;
  a.batch = batch; a.total_q = total_q; a.max_q_len = max_q_len; a.num_pages = num_pages * page_size;
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  a.out = out; a.lse = lse;
  return hip_status(pkv::launch_mla_prefill(a, s), "mla_paged_prefill_pages launch");
}

extern "C" int mla_paged_decode(const void* q_nope, const void* q_pe, const void* ckv_cache, const void* kpe_cache,
                                const int32_t* kv_indptr, const int32_t* kv_indices, int batch, int num_pages,
                                int num_kv_indices, int max_kv_len, int num_heads, int ckv_dim, int kpe_dim,
                                int page_size, float sm_scale, int split_tokens, int max_num_splits,
                                float* partial_acc, float* partial_m, float* partial_l, int32_t* counters,
                                void* out, float* lse, void* stream) {
  if (batch < 0 || num_pages < 0 || num_kv_indices < 0 || max_kv_len < 0 || num_heads <= 0 || ckv_dim <= 0 ||
      kpe_dim <= 0 || page_size <= 0 || split_tokens <= 0 || max_num_splits <= 0)
    return fail(PKV_EINVAL, "mla_paged_decode: bad sizes");
  if (!std::isfinite(sm_scale)) return fail(PKV_EINVAL, "mla_paged_decode: sm_scale is not finite");
  if (num_heads != 16 || ckv_dim != 512 || kpe_dim != 64 || page_size != 1)
    return fail(PKV_EUNSUPPORTED,
                "mla_paged_decode: compiled for num_heads 16, ckv_dim 512, kpe_dim 64, page_size 1 (got %d, %d, %d, %d)",
                num_heads, ckv_dim, kpe_dim, page_size);
  const int64_t grid_parts = ((int64_t)max_kv_len + split_tokens - 1) / split_tokens;
  if (grid_parts > max_num_splits)
    return fail(PKV_EINVAL, "mla_paged_decode: max_num_splits %d < ceil(max_kv_len / split_tokens) = %lld",
                max_num_splits, (long long)grid_parts);
  if ((int64_t)batch * (grid_parts > 0 ? grid_parts : 1) >= INT32_MAX || (int64_t)batch * 16 >= INT32_MAX / 2)
    return fail(PKV_EUNSUPPORTED, "mla_paged_decode: grid too large");
  if (batch == 0) return PKV_OK;
  if (!q_nope || !q_pe || !ckv_cache || !kpe_cache || !kv_indptr || !kv_indices || !partial_acc || !partial_m ||
      !partial_l || !out || !lse)
    return fail(PKV_EINVAL, "mla_paged_decode: NULL pointer argument");
  if (num_pages <= 0) return fail(PKV_EINVAL, "mla_paged_decode: num_pages must be positive");
  pkv::MlaDecodeArgs a;
  a.q_nope = q_nope; a.q_pe = q_pe; a.ckv = ckv_cache; a.kpe = kpe_cache;
  a.kv_indptr = kv_indptr; a.kv_indices = kv_indices;
  a.batch = batch; a.num_pages = num_pages; a.num_kv_indices = num_kv_indices;
  a.split = split_tokens; a.P = max_num_splits;
  // lengths are cut to the splits phase 1 launches, so the combine never reads a partial
  // row that phase 1 did not write, even when a kv_len breaks the max_kv_len contract
  a.len_cap = (int)std::min<int64_t>((int64_t)(grid_parts > 0 ? grid_parts : 1) * split_tokens, INT32_MAX);
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  a.acc = partial_acc; a.m = partial_m; a.l = partial_l; a.out = out; a.lse = lse;
  a.counters = counters;
  return hip_status(pkv::launch_mla_decode(a, (int)grid_parts, reinterpret_cast<hipStream_t>(stream)),
                    "mla_paged_decode launch");
}

extern "C" int pkv_read_bandwidth(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return PKV_OK;
  if (!buf || !sink) return fail(PKV_EINVAL, "pkv_read_bandwidth: NULL pointer argument");
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(PKV_EINVAL, "pkv_read_bandwidth: buffer must be 16-byte aligned and a multiple of 16 bytes");
  return hip_status(pkv::launch_read_probe(buf, bytes, sink, reinterpret_cast<hipStream_t>(stream)),
                    "pkv_read_bandwidth launch");
}

extern "C" const char* pkv_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* pkv_version(void) { return "pkv 0.1.0 gfx950"; }
