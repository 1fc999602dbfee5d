// Key tiles of the MLA kernels in LDS: the layout of gathered [ckv | kpe] rows, their
// transfers from global memory straight into LDS, and the matrix-core operand reads.
#pragma once

#include "common.h"

namespace pkv {
namespace mla {

constexpr int kCkvChunks = 512 * 2 / 16;     // 64 16-byte chunks of a ckv row
constexpr int kKpeChunks = 64 * 2 / 16;      // 8 chunks of a kpe row
constexpr int kCkvStride = kCkvChunks + 2;   // padded LDS row (chunks): see the bank note below

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

PKV_DEVICE f32x4_t mfma16x16x32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// LDS bank spreading, as measured on gfx950 with a read probe (eight waves per CU, cycles
// per read instruction per CU): a ckv row sits at stride kCkvStride, 32 B past a multiple
// of 1 KiB, with its chunks in order. The logits read one 16-byte chunk from each of 16
// consecutive rows per 16-lane group, and at this stride those reads run at the rate of a
// contiguous read (4.4 cycles); rows at 1 KiB take 22 cycles, rows at 1 KiB + 16 or + 64 B,
// or this stride with chunk bit 0 flipped by row bits 2 ^ 3, 5.5. The transposing V reads
// (32 B from each of 16 rows) run at this stride at the rate of a contiguous transposing
// read (4.6 cycles per 512 B).
// kpe rows are packed (128 B) because one transfer fills 8 of them; chunk c of row r sits
// at position c ^ kpe_swz(r), which puts the 16 rows of a logits read on 16 distinct
// 16-byte positions of two 128-byte lines: 4.4 cycles, where the unswizzled packed rows
// take 11 and chunk c ^ (r & 7) ^ (r >> 3) 5.5.
PKV_DEVICE uint32_t kpe_swz(int r) { return (uint32_t)(r & 7); }

PKV_DEVICE void vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef short i16x4_t __attribute__((ext_vector_type(4)));
// Transposing 8-byte LDS read (see the header comment for the lane mapping).
PKV_DEVICE uint2 lds_read_tr16(const void* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(
      (__attribute__((address_space(3))) void*)p));
  return __builtin_bit_cast(uint2, v);
}

// 16 bytes per lane from global memory (scalar base + per-lane offset) straight into LDS
// (lane i -> lds_base + 16 i; lanes outside the exec mask move nothing). Written as inline
// assembly so the compiler does not see an LDS write: with the builtin it waits for every
// outstanding transfer before each later LDS read, which would stall the math on tile kt
// until tile kt + 1 has landed. The kernel itself waits (vmcnt(0)) and then barriers
// before any wave reads a buffer that a transfer filled.
PKV_DEVICE void lds_dma16_s(const void* sbase, uint32_t voff, const void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base);
  // M0 (the LDS destination) is an input operand, so the compiler writes it and knows its value
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0));
}

}  // namespace mla
}  // namespace pkv
