// C ABI of the library (include/pkv.h): argument validation on the host, dispatch to a
// compiled kernel instance, launch on the caller's stream. Nothing here allocates.
#include "../../include/pkv.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
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

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  if (e == hipErrorNotSupported) return fail(PKV_EUNSUPPORTED, "%s: no compiled kernel for these arguments", what);
  return fail(PKV_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

constexpr int kMaxGridYZ = 65535;

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

extern "C" int paged_decode_partial(const void* query, int dtype, const void* key_cache,
                                    const void* value_cache, int layout,
                                    const int32_t* block_tables, int max_blocks_per_seq,
                                    const int32_t* seq_lens, int num_seqs, int num_heads,
                                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                    float scale, int partition_size, int max_num_partitions,
                                    int max_seq_len, float* partial_acc, float* partial_m,
                                    float* partial_l, void* stream) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_EINVAL, "paged_decode_partial: unknown dtype %d", dtype);
  if (layout != PKV_KV_TOKEN_MAJOR && layout != PKV_KV_XPACKED)
    return fail(PKV_EINVAL, "paged_decode_partial: unknown layout %d", layout);
  if (num_seqs < 0) return fail(PKV_EINVAL, "paged_decode_partial: num_seqs < 0");
  if (num_seqs == 0) return PKV_OK;
  if (!query || !key_cache || !value_cache || !block_tables || !seq_lens || !partial_acc ||
      !partial_m || !partial_l)
    return fail(PKV_EINVAL, "paged_decode_partial: NULL pointer argument");
  if (num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_num_partitions <= 0 || max_seq_len < 0)
    return fail(PKV_EINVAL, "paged_decode_partial: sizes must be positive (max_seq_len >= 0)");
  if (num_heads % num_kv_heads != 0)
    return fail(PKV_EINVAL, "paged_decode_partial: num_heads %d is not a multiple of num_kv_heads %d",
                num_heads, num_kv_heads);
  if (partition_size <= 0 || partition_size % block_size != 0)
    return fail(PKV_EINVAL, "paged_decode_partial: partition_size %d is not a positive multiple of block_size %d",
                partition_size, block_size);
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_EINVAL, "paged_decode_partial: max_seq_len %d exceeds max_blocks_per_seq * block_size",
                max_seq_len);
  const int grid_parts = (int)(((int64_t)max_seq_len + partition_size - 1) / partition_size);
  if (grid_parts > max_num_partitions)
    return fail(PKV_EINVAL, "paged_decode_partial: max_num_partitions %d < ceil(max_seq_len / partition_size) = %d",
                max_num_partitions, grid_parts);
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "paged_decode_partial: scale is not finite");
  if (block_size != 16)
    return fail(PKV_EUNSUPPORTED, "paged_decode_partial: block_size %d (compiled for 16)", block_size);
  const bool bf16 = dtype == PKV_BF16;
  if (!(head_dim == 64 || head_dim == 128 || (bf16 && head_dim == 256)))
    return fail(PKV_EUNSUPPORTED, "paged_decode_partial: head_dim %d for %s", head_dim, bf16 ? "bf16" : "f32");
  const int G = num_heads / num_kv_heads;
  if (G > (bf16 ? 16 : 8))
    return fail(PKV_EUNSUPPORTED, "paged_decode_partial: %d query heads per kv head", G);
  if (num_kv_heads > kMaxGridYZ || num_seqs > kMaxGridYZ)
    return fail(PKV_EUNSUPPORTED, "paged_decode_partial: grid too large");
  if (grid_parts == 0) return PKV_OK;  // every sequence is empty: nothing is touched

  pkv::DecodePartialArgs a;
  a.q = query; a.kc = key_cache; a.vc = value_cache;
  a.bt = block_tables; a.lens = seq_lens; a.mb = max_blocks_per_seq;
  a.S = num_seqs; a.H = num_heads; a.KVH = num_kv_heads; a.D = head_dim; a.NB = num_blocks;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.ps = partition_size; a.ppp = partition_size / block_size; a.P = max_num_partitions;
  a.acc = partial_acc; a.m = partial_m; a.l = partial_l;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  hipError_t e;
  const bool xp = layout == PKV_KV_XPACKED;
  if (bf16 && G >= 8) {
    e = xp ? pkv::launch_decode_mfma_bf16_xp(a, G, grid_parts, s)
           : pkv::launch_decode_mfma_bf16_tm(a, G, grid_parts, s);
  } else if (bf16) {
    e = xp ? pkv::launch_decode_valu_bf16_xp(a, G, grid_parts, s)
           : pkv::launch_decode_valu_bf16_tm(a, G, grid_parts, s);
  } else {
    e = xp ? pkv::launch_decode_valu_f32_xp(a, G, grid_parts, s)
           : pkv::launch_decode_valu_f32_tm(a, G, grid_parts, s);
  }
  return hip_status(e, "paged_decode_partial launch");
}

extern "C" int paged_decode_reduce(const float* partial_acc, const float* partial_m,
                                   const float* partial_l, const int32_t* seq_lens, int num_seqs,
                                   int num_heads, int head_dim, int partition_size,
                                   int max_num_partitions, void* out, int out_dtype, float* lse,
                                   void* stream) {
  if (out_dtype != PKV_F32 && out_dtype != PKV_BF16)
    return fail(PKV_EINVAL, "paged_decode_reduce: unknown out_dtype %d", out_dtype);
  if (num_seqs < 0 || num_heads < 0 || head_dim <= 0)
    return fail(PKV_EINVAL, "paged_decode_reduce: bad sizes");
  if (num_seqs == 0 || num_heads == 0) return PKV_OK;
  if (!partial_acc || !partial_m || !partial_l || !seq_lens || !out)
    return fail(PKV_EINVAL, "paged_decode_reduce: NULL pointer argument");
  if (partition_size <= 0 || max_num_partitions <= 0)
    return fail(PKV_EINVAL, "paged_decode_reduce: partition_size and max_num_partitions must be positive");
  if (!(head_dim == 64 || head_dim == 128 || head_dim == 256))
    return fail(PKV_EUNSUPPORTED, "paged_decode_reduce: head_dim %d", head_dim);
  if ((int64_t)num_seqs * num_heads > (int64_t)INT32_MAX / 2)
    return fail(PKV_EUNSUPPORTED, "paged_decode_reduce: too many rows");
  pkv::DecodeReduceArgs a;
  a.acc = partial_acc; a.m = partial_m; a.l = partial_l; a.lens = seq_lens;
  a.S = num_seqs; a.H = num_heads; a.D = head_dim; a.ps = partition_size; a.P = max_num_partitions;
  a.out = out; a.lse = lse;
  return hip_status(pkv::launch_decode_reduce(a, out_dtype == PKV_BF16, reinterpret_cast<hipStream_t>(stream)),
                    "paged_decode_reduce launch");
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
  if (batch > pkv::kMlaMaxBatch)
    return fail(PKV_EUNSUPPORTED, "mla_paged_prefill: batch %d exceeds %d (the tile list is held in LDS)", batch,
                pkv::kMlaMaxBatch);
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
