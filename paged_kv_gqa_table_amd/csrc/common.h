// Shared device helpers for the gfx950 kernels: bf16 packing, 16-byte loads,
// wavefront reductions (DPP inside a 16-lane row, cross-row permutes), exp2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define PKV_DEVICE __device__ __forceinline__

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------- bf16 <-> f32
PKV_DEVICE float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
PKV_DEVICE float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even f32 -> bf16 bits (NaN stays NaN).
PKV_DEVICE uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two floats to a bf16 pair with v_cvt_pk_bf16_f32 (round to nearest even).
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
PKV_DEVICE uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2v_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
}

// v_dot2c_f32_bf16: acc + a.lo*b.lo + a.hi*b.hi with bf16 pairs, f32 accumulate.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
PKV_DEVICE float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Byte permute: picks the low (sel_lo) or high (sel_hi) bf16 of a and b into one pair.
PKV_DEVICE uint32_t pair_lo(uint32_t a, uint32_t b) {  // (a.lo, b.lo)
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
PKV_DEVICE uint32_t pair_hi(uint32_t a, uint32_t b) {  // (a.hi, b.hi)
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// ---------------------------------------------------------------- loads
PKV_DEVICE uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
PKV_DEVICE uint4 ld16_nt(const void* p) {  // non-temporal: data read once (the KV stream)
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// K/V page loads of the decode kernels: every KV byte is read once per step, and on
// MI355X the non-temporal form streams faster (measured: 6.1-6.3 vs 5.4-5.7 TB/s for a
// plain read; 4-5 % less phase-1 time at 32 sequences x 2300 tokens).
PKV_DEVICE uint4 ld16_kv(const void* p) { return ld16_nt(p); }

// float8 e4m3 (OCP) K/V elements as bf16 pairs: every e4m3 value is exactly a bf16 value,
// so the conversion loses nothing. 8 elements (8 bytes) -> 8 bf16; 4 -> 4.
PKV_DEVICE uint4 as_bf16x8(const uint4& v) { return v; }
PKV_DEVICE uint4 as_bf16x8(const uint2& v) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, true);
  return make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(b[0], b[1]), pack_bf16x2(c[0], c[1]),
                    pack_bf16x2(d[0], d[1]));
}
PKV_DEVICE uint2 as_bf16x4(const uint2& v) { return v; }
PKV_DEVICE uint2 as_bf16x4(uint32_t v) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, true);
  return make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(b[0], b[1]));
}
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
PKV_DEVICE uint2 ld8_nt(const void* p) {  // non-temporal 8-byte load (float8 K/V)
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v[0], v[1]);
}
PKV_DEVICE uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

// ---------------------------------------------------------------- exp2
PKV_DEVICE float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- lane exchange
// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppQuadRev = 0x1B;       // quad_perm [3,2,1,0] (lane ^ 3)
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i inside each 8-lane half row
constexpr int kDppMirror = 0x140;       // lane i <-> 15-i inside each 16-lane row
constexpr int kDppRor8 = 0x128;         // lane i <- lane (i+8) mod 16 inside a row

template <int CTRL>
PKV_DEVICE float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Partner value across rows via ds_bpermute (lane ^ 16, lane ^ 32).
PKV_DEVICE float xor_lanes(float v, int mask) {
  int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

// All-reduce over groups of N consecutive lanes (N in {1,2,4,8,16}); every lane of a
// group ends with the group's sum / max.
template <int N>
PKV_DEVICE float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<kDppQuadXor1>(v);
  if constexpr (N >= 4) v += dpp<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppMirror>(v);
  return v;
}
template <int N>
PKV_DEVICE float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp<kDppQuadXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp<kDppQuadXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}

// All-reduce over lanes that agree modulo STRIDE (STRIDE in {1,...,32}, power of 2):
// combines lane l with lanes l ^ STRIDE, l ^ 2*STRIDE, ... up to 32.
template <int STRIDE>
PKV_DEVICE float strided_sum(float v) {
  if constexpr (STRIDE <= 1) v += dpp<kDppQuadXor1>(v);
  if constexpr (STRIDE <= 2) v += dpp<kDppQuadXor2>(v);
  if constexpr (STRIDE <= 4) v += xor_lanes(v, 4);
  if constexpr (STRIDE <= 8) v += dpp<kDppRor8>(v);
  if constexpr (STRIDE <= 16) v += xor_lanes(v, 16);
  if constexpr (STRIDE <= 32) v += xor_lanes(v, 32);
  return v;
}
template <int STRIDE>
PKV_DEVICE float strided_max(float v) {
  if constexpr (STRIDE <= 1) v = fmaxf(v, dpp<kDppQuadXor1>(v));
  if constexpr (STRIDE <= 2) v = fmaxf(v, dpp<kDppQuadXor2>(v));
  if constexpr (STRIDE <= 4) v = fmaxf(v, xor_lanes(v, 4));
  if constexpr (STRIDE <= 8) v = fmaxf(v, dpp<kDppRor8>(v));
  if constexpr (STRIDE <= 16) v = fmaxf(v, xor_lanes(v, 16));
  if constexpr (STRIDE <= 32) v = fmaxf(v, xor_lanes(v, 32));
  return v;
}

// Wave-wide max made uniform. `v` must already agree inside each group of STRIDE
// consecutive lanes (STRIDE in {1,...,16}, power of two); the remaining lane bits are
// folded with DPP (row_ror:8 inside a row, then row_bcast:15 / row_bcast:31 across rows,
// which leaves the full max in lane 63) and broadcast with readlane.
template <int STRIDE>
PKV_DEVICE float wave_max_uniform(float v) {
  if constexpr (STRIDE <= 1) v = fmaxf(v, dpp<kDppQuadXor1>(v));
  if constexpr (STRIDE <= 2) v = fmaxf(v, dpp<kDppQuadXor2>(v));
  if constexpr (STRIDE <= 4) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if constexpr (STRIDE <= 8) v = fmaxf(v, dpp<kDppRor8>(v));
  // rows 1 and 3 take lane 15 of the row below; then rows 2 and 3 take lane 31
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x142, 0xA, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x143, 0xC, 0xF, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

PKV_DEVICE float uniform(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
PKV_DEVICE int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

PKV_DEVICE void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pkv
