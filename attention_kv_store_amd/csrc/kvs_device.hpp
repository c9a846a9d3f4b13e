// Device-side helpers shared by the gfx950 kernels: vector types, MFMA
// wrappers, cross-lane reductions and bf16 packing.  CDNA4 only: wave64,
// 160 KB LDS per CU, bf16 MFMA with fp32 accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWave = 64;
constexpr int kPage = 16;               // tokens per KV block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for -inf in masked scores: exp2 of it minus any finite
// running max is exactly 0, and it never produces inf - inf.
constexpr float kMaskedScore = -3.0e38f;

// ---- bf16 <-> fp32 -------------------------------------------------------
// bf16 is the top half of an fp32 word, so widening is a shift / mask.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two fp32 values to bf16 (nearest even) and pack them, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// ---- MFMA wrappers (operand layouts are documented where they are used) ----
__device__ __forceinline__ f32x16 mfma32x32x16_bf16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16_bf16(const u32x2& a, const u32x2& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                    __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x2_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x4_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- cross-lane ------------------------------------------------------------
// Combine a value with the one in lane (lane ^ 32).  ds_bpermute through the
// LDS crossbar; one instruction per call.
// Cross-lane combines on the VALU (gfx950 permlane swaps): with both operands
// the same register, the pair returned holds this lane's value and the value
// of lane ^ 16 (resp. lane ^ 32), in an order that depends on the lane, so it
// is only ever combined symmetrically.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Value of lane (l & ~15) | ((l - n) & 15): a rotation inside each row of 16
// lanes (DPP row_ror, n in 1..15).
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  static_assert(N >= 1 && N <= 15, "row_ror takes 1..15");
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}
// Max over all 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, row_ror<1>(x));
  x = fmaxf(x, row_ror<2>(x));
  x = fmaxf(x, row_ror<4>(x));
  x = fmaxf(x, row_ror<8>(x));
  return max_xor32(max_xor16(x));
}
// Sum over all 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float x) {
  x += row_ror<1>(x);
  x += row_ror<2>(x);
  x += row_ror<4>(x);
  x += row_ror<8>(x);
  return sum_xor32(sum_xor16(x));
}
// Max / sum over the 16 lanes that share lane % 4.
__device__ __forceinline__ float max_mod4(float x) {
  x = fmaxf(x, row_ror<4>(x));
  x = fmaxf(x, row_ror<8>(x));
  return max_xor32(max_xor16(x));
}
__device__ __forceinline__ float sum_mod4(float x) {
  x += row_ror<4>(x);
  x += row_ror<8>(x);
  return sum_xor32(sum_xor16(x));
}
// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts inside rows
// of 16, then the last lane of a row added to the rows after it).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// ---- LDS transposing read (gfx950) -----------------------------------------
// In each group of 16 lanes, lane i receives 16-bit element i % 4 of the 8-byte
// rows addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12 of its group, in
// that order (checked on the device).
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(const_cast<char*>(p)));
  return __builtin_bit_cast(u32x2, v);
}

// 16-byte copy from global memory straight into LDS (gfx950): lane l's 16
// bytes land at lds_block + 16 * l; lds_block must be the same on every lane.
__device__ __forceinline__ void copy16_to_lds(const void* src, char* lds_block) {
  __builtin_amdgcn_global_load_lds(src, lds_block, 16, 0, 0);
}

// ---- memory --------------------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Load unconditionally (the address must be readable either way) and keep the
// data only where `keep` holds.  Branch-free, so the compiler can count the
// outstanding loads exactly and a prefetch is not waited on early.
__device__ __forceinline__ u32x4 ld16_keep(const void* p, bool keep) {
  const u32x4 v = ld16(p);
  return keep ? v : u32x4{0, 0, 0, 0};
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
// Non-temporal (streaming) loads, for K / V bytes that a decode launch reads
// exactly once: they carry the nt cache policy, which tells the caches not to
// keep the lines; the decode stream runs faster with them than with default
// loads.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 ld8_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}
__device__ __forceinline__ f32x4 ldf4_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

// Map a linear workgroup id so that each of the 8 XCDs (which receive
// workgroups round-robin) walks one contiguous range of the logical order;
// consecutive logical tiles then share an XCD and its L2.  A bijection on
// [0, n) for any n.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t n) {
  const uint32_t xcd = id & 7u, idx = id >> 3;
  const uint32_t per = n >> 3, rem = n & 7u;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Nearest E4M3 code of a finite y (ties to even), saturating at +-448: the
// OCP E4M3 format (bias 7, subnormal step 2^-9, largest finite 448).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.f);
  uint32_t c;
  if (a < 0.015625f) {                                  // below 2^-6: multiples of 2^-9
    c = (uint32_t)__builtin_rintf(a * 512.f);           // exact scaling, ties to even; 8 is 2^-6
  } else {
    const uint32_t b = __float_as_uint(a);
    const uint32_t e = (b >> 23) - 120u;                // E4M3 exponent field: (b >> 23) - 127 + 7
    const uint32_t mant = b & 0x7FFFFFu;
    uint32_t m = mant >> 20;                            // 3 kept mantissa bits
    const uint32_t rest = mant & 0xFFFFFu;
    m += (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) ? 1u : 0u;
    c = (e << 3) + m;                                   // m == 8 carries into the exponent
  }
  return c | sign;
}

// INT8 code of y: the nearest integer (ties to even), clamped to +-127, as
// the byte of its two's complement.
__device__ __forceinline__ uint32_t i8_code(float y) {
  const float r = fminf(fmaxf(__builtin_rintf(y), -127.f), 127.f);
  return (uint32_t)(int32_t)r & 0xFFu;
}

}  // namespace kvs
