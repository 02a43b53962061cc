// One new token of one sequence written into the KV cache by one wave
// (the decode-step case of the KV append): lane l owns features
// l*EPT .. l*EPT+EPT-1. F32/BF16 caches copy bits; FP8 caches quantise the
// token: amax over its d values, scale = amax/448 (one correctly rounded
// fp32 division, 1 when amax = 0), code = RNE e4m3 of the correctly rounded
// quotient x/scale ("Step-3 is Large yet Affordable" summary page, §5: the
// 8-bit cache that raises arithmetic intensity; §7: attention instances own
// their KV caches). Element positions follow kv_layout.h.
#pragma once

#include "device_common.h"
#include "kernels.h"
#include "kv_layout.h"

namespace mfa {

__device__ __forceinline__ float append_load_in(const void* p, size_t i, int in_f32) {
  return in_f32 ? reinterpret_cast<const float*>(p)[i]
                : bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}

// Token pos[b] of sequence b (n_new == 1); positions outside the table or
// mapped to no block write nothing.
// With a projected token (kv_part set), k_out / v_out are written even when
// the position maps to no block.
template <int CACHE, int EPT>   // CACHE: 0 f32, 1 bf16, 2 fp8
__device__ __forceinline__ void append_token_wave(const AppendArgs& a, int b, int lane) {
  const int p0 = a.pos[b];
  const int d = a.d;
  const size_t row = static_cast<size_t>(b) * d;
  float xk[EPT], xv[EPT];
  if (a.kv_part) {
    // projected token: sum the K-slice partials in slice order, round to the
    // activation dtype, keep a copy of the rounded values if asked
    const size_t prow = static_cast<size_t>(b - a.kv_row0) * a.kv_stride + a.kv_col0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) { xk[e] = 0.f; xv[e] = 0.f; }
    // slices in groups of 8 with all loads of a group in flight at once
    for (int k0 = 0; k0 < a.kv_ks; k0 += 8) {
      float tk[8][EPT], tv[8][EPT];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (k0 + u < a.kv_ks) {
          const float* pr = a.kv_part + static_cast<size_t>(k0 + u) * a.kv_rows * a.kv_stride + prow;
          if constexpr (EPT == 4) {   // 16-byte aligned: strides and column offsets are multiples of 4
            const float4 k4 = *reinterpret_cast<const float4*>(pr + lane * 4);
            const float4 v4 = *reinterpret_cast<const float4*>(pr + d + lane * 4);
            tk[u][0] = k4.x; tk[u][1] = k4.y; tk[u][2] = k4.z; tk[u][3] = k4.w;
            tv[u][0] = v4.x; tv[u][1] = v4.y; tv[u][2] = v4.z; tv[u][3] = v4.w;
          } else {
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
              tk[u][e] = pr[lane * EPT + e];
              tv[u][e] = pr[d + lane * EPT + e];
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (k0 + u < a.kv_ks) {
#pragma unroll
          for (int e = 0; e < EPT; ++e) { xk[e] += tk[u][e]; xv[e] += tv[u][e]; }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const size_t i = row + lane * EPT + e;
      if (a.kv_round_bf16) {
        const uint16_t kbits = f32_to_bf16(xk[e]), vbits = f32_to_bf16(xv[e]);
        xk[e] = bf16_to_f32(kbits);
        xv[e] = bf16_to_f32(vbits);
        if (a.k_out) static_cast<uint16_t*>(a.k_out)[i] = kbits;
        if (a.v_out) static_cast<uint16_t*>(a.v_out)[i] = vbits;
      } else {
        if (a.k_out) static_cast<float*>(a.k_out)[i] = xk[e];
        if (a.v_out) static_cast<float*>(a.v_out)[i] = xv[e];
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      xk[e] = append_load_in(a.k_new, row + lane * EPT + e, a.in_f32);
      xv[e] = append_load_in(a.v_new, row + lane * EPT + e, a.in_f32);
    }
  }
  if (p0 < 0) return;
  const int j = p0 / kBlockTokens;
  if (j >= a.max_blocks_per_seq) return;
  const int id = a.block_table ? a.block_table[static_cast<size_t>(b) * a.max_blocks_per_seq + j]
                               : b * a.max_blocks_per_seq + j;
  if (id < 0 || id >= a.num_blocks) return;
  const int off = p0 & 63;
  const size_t esz = CACHE == 0 ? 4 : (CACHE == 1 ? 2 : 1);
  uint8_t* kb = a.k + static_cast<size_t>(id) * kBlockTokens * d * esz;
  uint8_t* vb = a.v + static_cast<size_t>(id) * kBlockTokens * d * esz;
  if constexpr (CACHE == 2) {
    float ak = 0.f, av = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) { ak = fmaxf(ak, fabsf(xk[e])); av = fmaxf(av, fabsf(xv[e])); }
    ak = wave_max(ak);
    av = wave_max(av);
    const float sk = ak > 0.f ? ak / 448.0f : 1.0f;
    const float sv = av > 0.f ? av / 448.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int f = lane * EPT + e;
      kb[k_off_fp8(off, f, d)] = static_cast<uint8_t>(encode_e4m3_rne(xk[e] / sk));
      vb[v_off_fp8(off, f)] = static_cast<uint8_t>(encode_e4m3_rne(xv[e] / sv));
    }
    if (lane == 0) {
      a.k_scale[static_cast<size_t>(id) * kBlockTokens + off] = sk;
      a.v_scale[static_cast<size_t>(id) * kBlockTokens + off] = sv;
    }
  } else if constexpr (CACHE == 1) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int f = lane * EPT + e;
      *reinterpret_cast<uint16_t*>(kb + k_off_bf16(off, f, d)) = f32_to_bf16(xk[e]);  // exact
      *reinterpret_cast<uint16_t*>(vb + v_off_bf16(off, f)) = f32_to_bf16(xv[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int f = lane * EPT + e;
      *reinterpret_cast<float*>(kb + k_off_f32(off, f, d)) = xk[e];
      *reinterpret_cast<float*>(vb + v_off_f32(off, f)) = xv[e];
    }
  }
}

// Runtime dispatch over cache dtype and head dim.
__device__ __forceinline__ void append_token(const AppendArgs& a, int b, int lane) {
  const int ept = a.d >> 6;
  if (a.cache_dtype == 1) {
    if (ept == 4) append_token_wave<1, 4>(a, b, lane);
    else if (ept == 2) append_token_wave<1, 2>(a, b, lane);
    else append_token_wave<1, 1>(a, b, lane);
  } else if (a.cache_dtype == 2) {
    if (ept == 4) append_token_wave<2, 4>(a, b, lane);
    else if (ept == 2) append_token_wave<2, 2>(a, b, lane);
    else append_token_wave<2, 1>(a, b, lane);
  } else {
    if (ept == 4) append_token_wave<0, 4>(a, b, lane);
    else if (ept == 2) append_token_wave<0, 2>(a, b, lane);
    else append_token_wave<0, 1>(a, b, lane);
  }
}

}  // namespace mfa
