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

// Cache slot of sequence b's token at position p0: block id and offset in
// the block; id = -1 where the append writes nothing (negative position, a
// position past the table, or a block the table does not map). In two
// steps, token_block_raw (the table entry, or -1) and token_slot_of (the
// checks), so that the table read can be in flight with the token's own.
struct TokenSlot {
  int id, off;
};
__device__ __forceinline__ int token_block_raw(const AppendArgs& a, int b, int p0) {
  if (p0 < 0) return -1;
  const int j = p0 / kBlockTokens;
  if (j >= a.max_blocks_per_seq) return -1;
  return a.block_table ? a.block_table[static_cast<size_t>(b) * a.max_blocks_per_seq + j]
                       : b * a.max_blocks_per_seq + j;
}
__device__ __forceinline__ TokenSlot token_slot_of(const AppendArgs& a, int raw, int p0) {
  TokenSlot ts{-1, 0};
  if (raw < 0 || raw >= a.num_blocks) return ts;
  ts.id = raw;
  ts.off = p0 & 63;
  return ts;
}

// Features lane*EPT .. +EPT-1 of row b of a [B][d] input (fp32 or bf16) as
// raw words, one load per lane (rows of d = 64, 128, 256 elements from a
// 16-byte aligned base keep every lane's piece aligned), and their fp32
// values. Raw words first: nothing uses them until the stores, so the
// loads stay in flight with the position and block-table reads. The input
// dtype is a template parameter: chosen at run time per element, it made
// the compiler issue both kinds of load for every element, each behind its
// own wait.
template <int EPT, bool INF32>
struct RowPiece {
  uint32_t w[INF32 ? EPT : (EPT + 1) / 2];
};
template <int EPT, bool INF32>
__device__ __forceinline__ RowPiece<EPT, INF32> load_row_piece(const void* p, int b, int d, int lane) {
  RowPiece<EPT, INF32> r;
  const size_t i = static_cast<size_t>(b) * d + lane * EPT;
  if constexpr (INF32) {
    const uint32_t* s = static_cast<const uint32_t*>(p) + i;
    if constexpr (EPT == 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(s);
      r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else if constexpr (EPT == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(s);
      r.w[0] = v.x; r.w[1] = v.y;
    } else {
      r.w[0] = s[0];
    }
  } else {
    const uint16_t* s = static_cast<const uint16_t*>(p) + i;
    if constexpr (EPT == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(s);
      r.w[0] = v.x; r.w[1] = v.y;
    } else if constexpr (EPT == 2) {
      r.w[0] = *reinterpret_cast<const uint32_t*>(s);
    } else {
      r.w[0] = s[0];
    }
  }
  return r;
}
template <int EPT, bool INF32>
__device__ __forceinline__ void row_piece_f32(const RowPiece<EPT, INF32>& r, float (&x)[EPT]) {
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if constexpr (INF32) x[e] = __uint_as_float(r.w[e]);
    else x[e] = __uint_as_float(e & 1 ? (r.w[e >> 1] & 0xffff0000u) : (r.w[e >> 1] << 16));
  }
}

// FP8 scale of one token (the wave holds its d values): amax / 448, one
// correctly rounded division; 1 when amax = 0.
template <int EPT>
__device__ __forceinline__ float token_scale(const float (&x)[EPT]) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) m = fmaxf(m, fabsf(x[e]));
  m = wave_max(m);
  return m > 0.f ? m / 448.0f : 1.0f;
}

// The stored form of this lane's EPT K features: bf16 bits (two per word)
// or e4m3 codes of x / sk (four per word); f32 caches store x itself.
template <int CACHE, int EPT>
__device__ __forceinline__ void token_words(const float (&x)[EPT], float s, uint32_t (&w)[2]) {
  w[0] = w[1] = 0u;
  if constexpr (CACHE == 2) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) w[0] |= encode_e4m3_rne(x[e] / s) << (8 * e);
  } else if constexpr (CACHE == 1) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) w[e >> 1] |= static_cast<uint32_t>(f32_to_bf16(x[e])) << (16 * (e & 1));
  }
}

// K features lane*EPT .. +EPT-1 of the token into its slot (one store: the
// EPT features are adjacent in every layout).
template <int CACHE, int EPT>
__device__ __forceinline__ void store_token_k(const AppendArgs& a, const TokenSlot& ts,
                                              const float (&xk)[EPT], float sk, int lane) {
  const int d = a.d, f = lane * EPT;
  const size_t esz = CACHE == 0 ? 4 : (CACHE == 1 ? 2 : 1);
  uint8_t* kb = a.k + static_cast<size_t>(ts.id) * kBlockTokens * d * esz;
  uint32_t w[2];
  token_words<CACHE, EPT>(xk, sk, w);
  if constexpr (CACHE == 2) {
    uint8_t* p = kb + k_off_fp8(ts.off, f, d);
    if constexpr (EPT == 4) *reinterpret_cast<uint32_t*>(p) = w[0];
    else if constexpr (EPT == 2) *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(w[0]);
    else *p = static_cast<uint8_t>(w[0]);
  } else if constexpr (CACHE == 1) {
    uint8_t* p = kb + k_off_bf16(ts.off, f, d);
    if constexpr (EPT == 4) *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    else if constexpr (EPT == 2) *reinterpret_cast<uint32_t*>(p) = w[0];
    else *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(w[0]);
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) *reinterpret_cast<float*>(kb + k_off_f32(ts.off, f + e, d)) = xk[e];
  }
}

// V features lane*EPT .. +EPT-1 of the token (one element per store: in
// the bf16 and FP8 layouts a token's features are 16 bytes apart).
template <int CACHE, int EPT>
__device__ __forceinline__ void store_token_v(const AppendArgs& a, const TokenSlot& ts,
                                              const float (&xv)[EPT], float sv, int lane) {
  const int d = a.d;
  const size_t esz = CACHE == 0 ? 4 : (CACHE == 1 ? 2 : 1);
  uint8_t* vb = a.v + static_cast<size_t>(ts.id) * kBlockTokens * d * esz;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int f = lane * EPT + e;
    if constexpr (CACHE == 2) {
      vb[v_off_fp8(ts.off, f)] = static_cast<uint8_t>(encode_e4m3_rne(xv[e] / sv));
    } else if constexpr (CACHE == 1) {
      *reinterpret_cast<uint16_t*>(vb + v_off_bf16(ts.off, f)) = f32_to_bf16(xv[e]);  // exact
    } else {
      *reinterpret_cast<float*>(vb + v_off_f32(ts.off, f)) = xv[e];
    }
  }
}

// Token pos[b] of sequence b (n_new == 1); positions outside the table or
// mapped to no block write nothing.
// With a projected token (kv_part set), k_out / v_out are written even when
// the position maps to no block.
template <int CACHE, int EPT, bool INF32>   // CACHE: 0 f32, 1 bf16, 2 fp8; INF32: k_new, v_new dtype
__device__ __forceinline__ void append_token_wave(const AppendArgs& a, int b, int lane) {
  const int d = a.d;
  const size_t row = static_cast<size_t>(b) * d;
  float xk[EPT], xv[EPT];
  // the token's reads first (they need no position), then the position and
  // its table entry, all in flight together
  const bool proj = a.kv_part != nullptr;
  RowPiece<EPT, INF32> rk{}, rv{};
  if (!proj) {
    rk = load_row_piece<EPT, INF32>(a.k_new, b, d, lane);
    rv = load_row_piece<EPT, INF32>(a.v_new, b, d, lane);
  }
  const int p0 = a.pos[b];
  const int raw = token_block_raw(a, b, p0);
  if (proj) {
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
    row_piece_f32(rk, xk);
    row_piece_f32(rv, xv);
  }
  const TokenSlot ts = token_slot_of(a, raw, p0);
  if (ts.id < 0) return;
  float sk = 1.f, sv = 1.f;
  if constexpr (CACHE == 2) {
    sk = token_scale(xk);
    sv = token_scale(xv);
    if (lane == 0) {
      a.k_scale[static_cast<size_t>(ts.id) * kBlockTokens + ts.off] = sk;
      a.v_scale[static_cast<size_t>(ts.id) * kBlockTokens + ts.off] = sv;
    }
  }
  store_token_k<CACHE, EPT>(a, ts, xk, sk, lane);
  store_token_v<CACHE, EPT>(a, ts, xv, sv, lane);
}

// Token pos[b] of sequence b (n_new == 1) from k_new / v_new, no
// projection: the same reads, arithmetic and stores as append_token_wave.
template <int CACHE, int EPT, bool INF32>
__device__ __forceinline__ void append_token_plain(const AppendArgs& a, int b, int lane) {
  const RowPiece<EPT, INF32> rk = load_row_piece<EPT, INF32>(a.k_new, b, a.d, lane);
  const RowPiece<EPT, INF32> rv = load_row_piece<EPT, INF32>(a.v_new, b, a.d, lane);
  const int p0 = a.pos[b];
  const TokenSlot ts = token_slot_of(a, token_block_raw(a, b, p0), p0);
  if (ts.id < 0) return;
  float xk[EPT], xv[EPT];
  row_piece_f32(rk, xk);
  row_piece_f32(rv, xv);
  float sk = 1.f, sv = 1.f;
  if constexpr (CACHE == 2) {
    sk = token_scale(xk);
    sv = token_scale(xv);
    if (lane == 0) {
      a.k_scale[static_cast<size_t>(ts.id) * kBlockTokens + ts.off] = sk;
      a.v_scale[static_cast<size_t>(ts.id) * kBlockTokens + ts.off] = sv;
    }
  }
  store_token_k<CACHE, EPT>(a, ts, xk, sk, lane);
  store_token_v<CACHE, EPT>(a, ts, xv, sv, lane);
}

// Runtime dispatch over cache dtype, head dim and input dtype.
template <bool INF32>
__device__ __forceinline__ void append_token_in(const AppendArgs& a, int b, int lane) {
  const int ept = a.d >> 6;
  if (a.cache_dtype == 1) {
    if (ept == 4) append_token_wave<1, 4, INF32>(a, b, lane);
    else if (ept == 2) append_token_wave<1, 2, INF32>(a, b, lane);
    else append_token_wave<1, 1, INF32>(a, b, lane);
  } else if (a.cache_dtype == 2) {
    if (ept == 4) append_token_wave<2, 4, INF32>(a, b, lane);
    else if (ept == 2) append_token_wave<2, 2, INF32>(a, b, lane);
    else append_token_wave<2, 1, INF32>(a, b, lane);
  } else {
    if (ept == 4) append_token_wave<0, 4, INF32>(a, b, lane);
    else if (ept == 2) append_token_wave<0, 2, INF32>(a, b, lane);
    else append_token_wave<0, 1, INF32>(a, b, lane);
  }
}
__device__ __forceinline__ void append_token(const AppendArgs& a, int b, int lane) {
  if (a.in_f32) append_token_in<true>(a, b, lane);
  else append_token_in<false>(a, b, lane);
}

}  // namespace mfa
