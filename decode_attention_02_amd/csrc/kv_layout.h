// Byte offsets inside one 64-token KV-cache block (see include/mfa.h).
//
// bf16 and FP8 blocks are stored in the order in which the 16x16x32
// matrix-core operands of the attention kernel consume them, so that each
// wave-wide 16-byte load reads 1 KB of contiguous memory:
//   bf16 K: unit (token group tg = t/16, k-step s = d/32) of 1 KB; inside it,
//           lane (g = (d%32)/8, c = t%16) holds 16 bytes = K[t][8 consecutive d]
//   bf16 V: unit (feature group fg = f/16, k-step s2 = t/32); inside it, lane
//           (g = (t%32)/8, c = f%16) holds V[8 consecutive t][f]
//   FP8 K:  unit (tg = t/16, u = d/64); lane (g = (d%64)/16, c = t%16) holds
//           K[t][16 consecutive d]
//   FP8 V:  unit (fg = f/16); lane (g = t/16, c = f%16) holds V[16 consecutive t][f]
// fp32 blocks keep plain rows: K [64][d] token-major, V [d][64] feature-major.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mfa {

__host__ __device__ __forceinline__ uint32_t k_off_bf16(int t, int d, int D) {
  const int unit = (t >> 4) * (D >> 5) + (d >> 5);
  const int ln = ((d >> 3) & 3) * 16 + (t & 15);
  return static_cast<uint32_t>((unit * 64 + ln) * 16 + (d & 7) * 2);
}

__host__ __device__ __forceinline__ uint32_t v_off_bf16(int t, int f) {
  const int unit = (f >> 4) * 2 + (t >> 5);
  const int ln = ((t >> 3) & 3) * 16 + (f & 15);
  return static_cast<uint32_t>((unit * 64 + ln) * 16 + (t & 7) * 2);
}

__host__ __device__ __forceinline__ uint32_t k_off_fp8(int t, int d, int D) {
  const int unit = (t >> 4) * (D >> 6) + (d >> 6);
  const int ln = ((d >> 4) & 3) * 16 + (t & 15);
  return static_cast<uint32_t>((unit * 64 + ln) * 16 + (d & 15));
}

__host__ __device__ __forceinline__ uint32_t v_off_fp8(int t, int f) {
  const int ln = (t >> 4) * 16 + (f & 15);
  return static_cast<uint32_t>(((f >> 4) * 64 + ln) * 16 + (t & 15));
}

__host__ __device__ __forceinline__ uint32_t k_off_f32(int t, int d, int D) {
  return static_cast<uint32_t>((t * D + d) * 4);
}

__host__ __device__ __forceinline__ uint32_t v_off_f32(int t, int f) {
  return static_cast<uint32_t>((f * 64 + t) * 4);
}

}  // namespace mfa
