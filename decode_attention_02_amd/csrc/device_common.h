// Device helpers shared by the MFA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mfa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlockTokens = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t p;
  p[0] = static_cast<__bf16>(lo);
  p[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, p);
}

// 16x16x32 bf16 matrix-core product: acc[m][n] += sum_k A[m][k] B[k][n].
// Operand layout (lane l, g = l/16, c = l%16): A lane holds A[c][8g..8g+7],
// B lane holds B[8g..8g+7][c]; the accumulator lane holds C[4g+i][c], i<4.
__device__ __forceinline__ f32x4_t mfma_16x16x32(const bf16x8_t& a, const bf16x8_t& b,
                                                 const f32x4_t& acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// 16x16x128 OCP-e4m3 matrix-core product (the f8f6f4 family, both operands
// e4m3, unit block scales: E8M0 exponent 127): acc[m][n] += sum_k A[m][k] *
// B[k][n] into the fp32 accumulator. Lane l holds 32 codes of row l%16 of A
// and of column l%16 of B; both operands give k the same (lane group, byte)
// positions, so pairing the bytes of the two operands the same way gives
// the dot product whatever the order of k within them.
__device__ __forceinline__ f32x4_t mfma_16x16x128_e4m3(const i32x8_t& a, const i32x8_t& b,
                                                       const f32x4_t& acc) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
}

// Non-temporal stores for results the next kernel reads: they leave the
// L2 write-back path early, so less dirty data is left for the write-back
// at the end of the kernel (measured: ~1.5 us less between back-to-back
// attention launches with 16 MB of split partials). They pay only for whole
// lines: lanes that store small pieces far apart (one head row each) write
// several times the bytes, so such results are gathered first (the
// attention kernel stages its rows in LDS).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt(void* p, uint2 v) {
  __builtin_nontemporal_store(u32x2_t{v.x, v.y}, static_cast<u32x2_t*>(p));
}
__device__ __forceinline__ void store_nt(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, static_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store_nt(void* p, float4 v) {
  __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w}, static_cast<f32x4_t*>(p));
}
__device__ __forceinline__ void store_nt(void* p, float2 v) {
  __builtin_nontemporal_store(f32x2_t{v.x, v.y}, static_cast<f32x2_t*>(p));
}
__device__ __forceinline__ void store_nt(void* p, uint32_t v) {
  __builtin_nontemporal_store(v, static_cast<uint32_t*>(p));
}
__device__ __forceinline__ void store_nt(void* p, float v) {
  __builtin_nontemporal_store(v, static_cast<float*>(p));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

// Two OCP e4m3 codes (the low or high 16 bits of `word`) -> two bf16. Every
// e4m3 value is exact in bf16, and the scale 1.0 makes the conversion exact.
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t word) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(word), 1.0f, HIGH);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight e4m3 codes (two dwords) -> eight bf16 as one matrix-core operand.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  uint4 u;
  u.x = e4m3x2_to_bf16x2<false>(w0);
  u.y = e4m3x2_to_bf16x2<true>(w0);
  u.z = e4m3x2_to_bf16x2<false>(w1);
  u.w = e4m3x2_to_bf16x2<true>(w1);
  return as_bf16x8(u);
}

// Round-to-nearest-even encode of a float into an OCP e4m3 code, from the
// format's definition: 3 mantissa bits, exponent bias 7, subnormal step
// 2^-9, largest finite 448. Magnitudes above 448 saturate to 448 (callers
// only pass |y| <= 448 * (1 + 2^-23)). The input's sign bit is kept.
__device__ __forceinline__ uint32_t encode_e4m3_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(u & 0x7fffffffu);
  uint32_t code;
  if (a < 0.015625f) {                      // below 2^-6: multiples of 2^-9
    code = static_cast<uint32_t>(rintf(a * 512.0f));   // 0..8, ties to even
  } else {
    const uint32_t ua = __float_as_uint(a);
    const int e = static_cast<int>(ua >> 23) - 127;    // >= -6
    uint32_t keep = (ua >> 20) & 7u;
    const uint32_t rem = ua & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) keep += 1;
    uint32_t ef = static_cast<uint32_t>(e + 7);
    if (keep == 8u) { keep = 0; ef += 1; }
    code = (ef << 3) | keep;
    if (code > 0x7eu) code = 0x7eu;
  }
  return code | sign;
}

// Maximum of non-NaN floats (finite or infinite) as one v_max_f32 / v_max3_f32.
// fmaxf must quiet signalling NaNs first, which costs one extra
// instruction per operand the compiler cannot prove canonical (every matrix-
// core result and LDS value); the callers below never hold NaNs.
__device__ __forceinline__ float max_nonan(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_nonan(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Max / sum over the four 16-lane rows of a wave: lane c of every row gets
// the result for column c (rows are swapped pairwise by the gfx950 permlane
// swaps, so no LDS round trip is involved). rows4_max takes non-NaN inputs.
__device__ __forceinline__ float rows4_max(float v) {
  const int iv = __float_as_int(v);
  auto p = __builtin_amdgcn_permlane16_swap(iv, iv, false, false);
  v = max_nonan(__int_as_float(p[0]), __int_as_float(p[1]));
  const int iw = __float_as_int(v);
  auto q = __builtin_amdgcn_permlane32_swap(iw, iw, false, false);
  return max_nonan(__int_as_float(q[0]), __int_as_float(q[1]));
}

// The 16-lane rows of the wave as rows 0..3. permlane32 / permlane16 swap
// (vdst a, vsrc b) exchange a's rows {2,3} with b's rows {0,1}, resp. a's odd
// rows with b's even rows; swap_max returns the lane-wise max of the two
// results:
//   32: rows (max(a0,a2), max(a1,a3), max(b0,b2), max(b1,b3))
//   16: rows (max(a0,a1), max(b0,b1), max(a2,a3), max(b2,b3))
__device__ __forceinline__ float swap32_max(float a, float b) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(a), __float_as_int(b), false, false);
  return max_nonan(__int_as_float(p[0]), __int_as_float(p[1]));
}
__device__ __forceinline__ float swap16_max(float a, float b) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(a), __float_as_int(b), false, false);
  return max_nonan(__int_as_float(p[0]), __int_as_float(p[1]));
}

// Column max of four per-lane values v[0..3] (one per 16-wide column tile)
// over the four rows, transposed: lane (row g, column c) returns
// max over rows of v[g] at column c. Three swaps instead of eight.
__device__ __forceinline__ float rows4_max_t4(float v0, float v1, float v2, float v3) {
  const float x = swap32_max(v0, v2);     // rows: v0(0,2) v0(1,3) v2(0,2) v2(1,3)
  const float y = swap32_max(v1, v3);     // rows: v1(0,2) v1(1,3) v3(0,2) v3(1,3)
  return swap16_max(x, y);                // rows: v0 v1 v2 v3, each over all rows
}

__device__ __forceinline__ float rows4_sum(float v) {
  const int iv = __float_as_int(v);
  auto p = __builtin_amdgcn_permlane16_swap(iv, iv, false, false);
  v = __int_as_float(p[0]) + __int_as_float(p[1]);
  const int iw = __float_as_int(v);
  auto q = __builtin_amdgcn_permlane32_swap(iw, iw, false, false);
  return __int_as_float(q[0]) + __int_as_float(q[1]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

}  // namespace mfa
