// paged_decode_static: the whole split-K decode step with no allocation anywhere, for callers
// that cannot allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). The partials of phase 1 live in `scratch`, a file-scope
// device array of kStaticScratchBytes that every GPU the library runs on holds for the life
// of the process; phase 2 reads them back. The caller passes only inputs and outputs.
//
// The array's host-side name is not a device address: its address on each device is looked
// up once per device (hipGetSymbolAddress, with that device current) and kept; kernels only
// ever receive that looked-up pointer. Every call on one GPU shares that GPU's array, and
// the array keeps whatever the last call left in it: phase 1 writes every partial row or
// sentinel that phase 2 reads, so nothing needs clearing between calls, but calls that
// overlap in time on one GPU (different streams, or host threads) race on it.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/pkv.h"
#include "decode_args.h"

namespace {

constexpr size_t kStaticScratchBytes = PKV_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Device address of `scratch` on the current device, looked up on the first call per device.
int scratch_ptr(unsigned char** out) {
  static unsigned char* ptrs[kMaxDevices] = {};
  static std::mutex mu;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return pkv::set_last_error(PKV_EHIP, "paged_decode_static: hipGetDevice failed (%s)", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pkv::set_last_error(PKV_EUNSUPPORTED, "paged_decode_static: device index %d past %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return pkv::set_last_error(PKV_EHIP, "paged_decode_static: hipGetSymbolAddress of the scratch array failed (%s)",
                                 hipGetErrorString(e));
    ptrs[dev] = static_cast<unsigned char*>(p);
  }
  *out = ptrs[dev];
  return PKV_OK;
}

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

}  // namespace

extern "C" int paged_decode_static(const void* query, int dtype, const void* key_cache, const void* value_cache,
                                   int layout, const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* seq_lens, int num_seqs, int num_heads, int num_kv_heads,
                                   int head_dim, int block_size, int num_blocks, float scale, int partition_size,
                                   int num_splits, int max_seq_len, void* out, float* lse, void* stream) {
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || num_splits < 0 || max_seq_len < 0)
    return pkv::set_last_error(PKV_EINVAL, "paged_decode_static: bad sizes");
  if (num_seqs == 0) return PKV_OK;
  if (!out) return pkv::set_last_error(PKV_EINVAL, "paged_decode_static: NULL pointer argument (out)");
  if (num_splits == 0 && (partition_size <= 0 || block_size <= 0 || partition_size % block_size != 0))
    return pkv::set_last_error(PKV_EINVAL, "paged_decode_static: partition_size %d is not a positive multiple of "
                               "block_size %d", partition_size, block_size);
  const int64_t parts = num_splits > 0 ? num_splits : ((int64_t)max_seq_len + partition_size - 1) / partition_size;
  if (parts <= 1 && num_splits == 0) {
    // one partition holds every sequence: the single pass writes out directly, no scratch
    return paged_decode(query, dtype, key_cache, value_cache, layout, block_tables, max_blocks_per_seq, seq_lens,
                        num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, partition_size, 0,
                        1, max_seq_len, nullptr, nullptr, nullptr, nullptr, out, lse, stream);
  }
  if ((double)num_seqs * num_heads * (double)parts * (head_dim + 2) * sizeof(float) > (double)kStaticScratchBytes)
    return pkv::set_last_error(PKV_EUNSUPPORTED, "paged_decode_static: the partials need %.0f bytes; the static "
                               "scratch holds %zu (num_seqs * num_heads * partitions * (head_dim + 2) floats)",
                               (double)num_seqs * num_heads * (double)parts * (head_dim + 2) * sizeof(float),
                               kStaticScratchBytes);
  const int64_t rows = (int64_t)num_seqs * num_heads * parts;
  const size_t acc_bytes = round256((size_t)rows * head_dim * sizeof(float));
  const size_t ml_bytes = round256((size_t)rows * sizeof(float));
  const size_t need = acc_bytes + 2 * ml_bytes;
  if (need > kStaticScratchBytes)
    return pkv::set_last_error(PKV_EUNSUPPORTED, "paged_decode_static: the partials need %zu bytes; the static scratch "
                               "holds %zu (num_seqs * num_heads * partitions * (head_dim + 2) floats)", need,
                               kStaticScratchBytes);
  unsigned char* base = nullptr;
  int st = scratch_ptr(&base);
  if (st != PKV_OK) return st;
  float* acc = reinterpret_cast<float*>(base);
  float* m = reinterpret_cast<float*>(base + acc_bytes);
  float* l = reinterpret_cast<float*>(base + acc_bytes + ml_bytes);
  if (num_splits > 0) {
    st = paged_decode_split_partial(query, dtype, key_cache, value_cache, layout, block_tables, max_blocks_per_seq,
                                    seq_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                    scale, num_splits, max_seq_len, acc, m, l, stream);
    if (st != PKV_OK) return st;
    return paged_decode_split_reduce(acc, m, l, seq_lens, num_seqs, num_heads, head_dim, block_size, num_splits, out,
                                     dtype, lse, stream);
  }
  st = paged_decode_partial(query, dtype, key_cache, value_cache, layout, block_tables, max_blocks_per_seq, seq_lens,
                            num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                            partition_size, (int)parts, max_seq_len, acc, m, l, stream);
  if (st != PKV_OK) return st;
  return paged_decode_reduce(acc, m, l, seq_lens, num_seqs, num_heads, head_dim, partition_size, (int)parts, out, dtype,
                             lse, stream);
}
