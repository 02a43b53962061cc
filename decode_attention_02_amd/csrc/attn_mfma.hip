// MFA decode attention on the matrix cores: 64 query heads of width 256
// against one shared K/V head, bf16 or OCP-e4m3 KV cache.
//
// The method: "Step-3 is Large yet Affordable" (summary page), §2 Step-3
// Model Card (many query heads share a small KV cache through MFA's
// low-rank QK circuit) and §5 Model-System Co-design (one KV head read once
// for all 64 heads: 128 flop per byte of an 8-bit cache, 64 per byte of a
// bf16 cache). §6 states the attention stays memory-bandwidth bound, so the
// kernel is built around streaming K and V once at full HBM rate.
//
// One workgroup (8 waves, 2 per SIMD) owns one (sequence, split) pair and
// walks it in tiles of 128 tokens (two 64-token cache blocks). Per tile:
//   * wave w loads K rows 16w..16w+15 of the tile and the V^T rows
//     (features) 32w..32w+31 for all 128 tokens straight into registers. The
//     cache blocks are stored in matrix-core operand order (kv_layout.h), so
//     each wave-wide load reads 1 KB of contiguous memory and lands in the
//     operand registers as is. Every K and V byte is read from HBM once;
//   * S^T[token][head] = K . Q^T on the matrix cores: the 16 tokens are the
//     row side, the 64 heads sharing the KV head are four 16-column tiles of
//     Q staged once in LDS in operand order;
//   * online softmax: per-head tile max across the 8 waves through LDS,
//     p = exp2(s - m) in registers, lane-partial row sums;
//   * P^T (bf16, operand order) goes through LDS so every wave can apply all
//     128 tokens to its 32 features: O^T[feature][head] += V^T . P^T.
// FP8 codes are widened to bf16 in registers (exact); per-token K scales
// multiply the logits, per-token V scales multiply P before its bf16
// rounding. The next tile's loads are issued before the current tile's
// math, so each wave keeps one tile (16 KB) in flight: 128 KB per CU.
#include "device_common.h"
#include "kernels.h"

namespace mfa {

namespace {

constexpr int kH = 64;
constexpr int kD = 256;
constexpr int kWaves = 8;
constexpr int kTile = 128;              // tokens per tile (two cache blocks)

template <bool FP8>
struct Layout {
  static constexpr int kElem = FP8 ? 1 : 2;
  static constexpr int kBlockBytes = kBlockTokens * kD * kElem;
  static constexpr int kKLoads = FP8 ? 4 : 8;    // 16-byte loads per lane per tile
  static constexpr int kVLoads = FP8 ? 4 : 8;
};

// d offset of operand k-step s for lane group g (the K and Q sides agree).
template <bool FP8>
__device__ __forceinline__ int qk_dim(int s, int g) {
  return FP8 ? ((s >> 1) * 64 + g * 16 + (s & 1) * 8) : (s * 32 + g * 8);
}

// Loads of one wave for one tile. Blocks are stored in operand order (see
// kv_layout.h), so every load below reads 1 KB of contiguous memory per wave.
// kblk: the block holding this wave's 16 K rows (token group tg); vb0/vb1:
// the tile's two blocks (nullptr: block past the end).
template <bool FP8>
__device__ __forceinline__ void load_tile(const uint8_t* kblk, int tg, const uint8_t* vb0,
                                          const uint8_t* vb1, int w, int lane,
                                          uint4 (&kr)[Layout<FP8>::kKLoads],
                                          uint4 (&vr)[Layout<FP8>::kVLoads]) {
  if constexpr (FP8) {
    if (kblk) {   // units (tg, u), u = 0..3: K[16tg + c][64u + 16g .. +16]
      const uint8_t* kp = kblk + (tg * 4) * 1024 + lane * 16;
#pragma unroll
      for (int u = 0; u < 4; ++u) kr[u] = *reinterpret_cast<const uint4*>(kp + u * 1024);
    }
    // vr[bb*2 + dt]: unit fg = 2w + dt: V^T[16fg + c][16g .. +16] of block bb
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const uint8_t* vb = bb ? vb1 : vb0;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        vr[bb * 2 + dt] = vb ? *reinterpret_cast<const uint4*>(vb + ((2 * w + dt) * 64 + lane) * 16)
                             : make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
    if (kblk) {   // units (tg, s), s = 0..7: K[16tg + c][32s + 8g .. +8]
      const uint8_t* kp = kblk + (tg * 8) * 1024 + lane * 16;
#pragma unroll
      for (int s = 0; s < 8; ++s) kr[s] = *reinterpret_cast<const uint4*>(kp + s * 1024);
    }
    // vr[(bb*2 + dt)*2 + s2]: unit (fg = 2w + dt, s2): V^T[16fg + c][32s2 + 8g .. +8]
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const uint8_t* vb = bb ? vb1 : vb0;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          vr[(bb * 2 + dt) * 2 + s2] =
              vb ? *reinterpret_cast<const uint4*>(vb + (((2 * w + dt) * 2 + s2) * 64 + lane) * 16)
                 : make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

__device__ __forceinline__ uint32_t keep_bf16(uint32_t word, bool lo_ok, bool hi_ok) {
  return (lo_ok ? (word & 0xffffu) : 0u) | (hi_ok ? (word & 0xffff0000u) : 0u);
}

}  // namespace

template <bool FP8>
__global__ __launch_bounds__(512) void mfa_decode_mfma_kernel(AttnArgs a) {
  using LT = Layout<FP8>;
  __shared__ __attribute__((aligned(16))) uint4 q_lds[4 * 8 * 64];   // 32 KB, operand order
  __shared__ __attribute__((aligned(16))) uint4 p_lds[4 * 4 * 64];   // 16 KB, operand order
  __shared__ __attribute__((aligned(16))) float red[kH * kWaves];    // [head][wave]

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int split = blockIdx.x % a.num_splits;
  const int b = blockIdx.x / a.num_splits;

  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int t0 = split * a.chunk_tokens;
  const int t1 = min(t0 + a.chunk_tokens, L);

  f32x4_t o_acc[2][4];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) o_acc[dt][ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) { m_run[ht] = -INFINITY; l_run[ht] = 0.f; }

  if (t0 < t1) {
    // Q -> LDS in operand order: block (ht, s), lane (gg, cc) holds
    // Q[ht*16+cc][qk_dim(s, gg) .. +8].
    const uint16_t* qb = a.q + static_cast<size_t>(b) * kH * kD;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int idx = tid + 512 * r;
      const int ln = idx & 63, blk = idx >> 6;
      const int ht = blk >> 3, s = blk & 7;
      const int gg = ln >> 4, cc = ln & 15;
      q_lds[idx] = *reinterpret_cast<const uint4*>(qb + (ht * 16 + cc) * kD + qk_dim<FP8>(s, gg));
    }

    const int blk0 = t0 >> 6;                          // first logical block
    const int blk_end = (t1 + kBlockTokens - 1) >> 6;  // one past the last
    const int* bt_row = a.block_table ? a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq
                                      : nullptr;
    auto phys = [&](int j) -> size_t {
      int id = bt_row ? bt_row[j] : b * a.max_blocks_per_seq + j;
      id = id < 0 ? 0 : (id >= a.num_blocks ? a.num_blocks - 1 : id);
      return static_cast<size_t>(id);
    };
    // this wave's K rows within a tile: block (w >> 2), token group w & 3
    const int kbb = w >> 2, tg = w & 3, krow = 16 * tg;

    uint4 kr[LT::kKLoads], vr[LT::kVLoads];
#pragma unroll
    for (int i = 0; i < LT::kKLoads; ++i) kr[i] = make_uint4(0u, 0u, 0u, 0u);
    float4 ksc = make_float4(1.f, 1.f, 1.f, 1.f), vsc = ksc;
    auto issue = [&](int j0) {                         // tile starting at logical block j0
      const bool has1 = j0 + 1 < blk_end;
      const size_t p0 = phys(j0);
      const size_t p1 = has1 ? phys(j0 + 1) : p0;
      const uint8_t* vb0 = a.v + p0 * LT::kBlockBytes;
      const uint8_t* vb1 = has1 ? a.v + p1 * LT::kBlockBytes : nullptr;
      const size_t pk = kbb ? p1 : p0;
      const uint8_t* kb = (kbb == 0 || has1) ? a.k + pk * LT::kBlockBytes : nullptr;
      load_tile<FP8>(kb, tg, vb0, vb1, w, lane, kr, vr);
      if constexpr (FP8) {
        if (kbb == 0 || has1) {
          ksc = *reinterpret_cast<const float4*>(a.k_scale + pk * kBlockTokens + krow + 4 * g);
          vsc = *reinterpret_cast<const float4*>(a.v_scale + pk * kBlockTokens + krow + 4 * g);
        }
      }
    };
    issue(blk0);
    __syncthreads();   // Q staged

    for (int j0 = blk0; j0 < blk_end; j0 += 2) {
      uint4 kc[LT::kKLoads], vc[LT::kVLoads];
#pragma unroll
      for (int i = 0; i < LT::kKLoads; ++i) kc[i] = kr[i];
#pragma unroll
      for (int i = 0; i < LT::kVLoads; ++i) vc[i] = vr[i];
      const float4 kscc = ksc, vscc = vsc;
      if (j0 + 2 < blk_end) issue(j0 + 2);

      const int tile_t0 = j0 * kBlockTokens;           // token index of tile row 0
      const int lim = t1 - tile_t0;                    // valid tokens in this tile (> 0)

      // ---- S^T = K . Q^T  (tokens 16w..16w+15 of the tile, all 64 heads)
      f32x4_t s_acc[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) s_acc[ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        bf16x8_t kop;
        if constexpr (FP8) {
          const uint4 u = kc[s >> 1];
          kop = (s & 1) ? e4m3x8_to_bf16x8(u.z, u.w) : e4m3x8_to_bf16x8(u.x, u.y);
        } else {
          kop = as_bf16x8(kc[s]);
        }
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
          s_acc[ht] = mfma_16x16x32(kop, as_bf16x8(q_lds[(ht * 8 + s) * 64 + lane]), s_acc[ht]);
      }

      // ---- scale, mask, tile max per head
      const int tt0 = 16 * w + 4 * g;                  // tile token of s_acc[.][0]
      const float kscv[4] = {kscc.x, kscc.y, kscc.z, kscc.w};
      const float vscv[4] = {vscc.x, vscc.y, vscc.z, vscc.w};
      float mx[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sv = s_acc[ht][i] * a.scale_log2;
          if constexpr (FP8) sv *= kscv[i];
          sv = (tt0 + i < lim) ? sv : -INFINITY;
          s_acc[ht][i] = sv;
          m = fmaxf(m, sv);
        }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        mx[ht] = m;
      }
      if (g == 0) {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) red[(ht * 16 + c) * kWaves + w] = mx[ht];
      }
      __syncthreads();

      float alpha[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const float4 r0 = reinterpret_cast<const float4*>(red)[(ht * 16 + c) * 2];
        const float4 r1 = reinterpret_cast<const float4*>(red)[(ht * 16 + c) * 2 + 1];
        const float tmax = fmaxf(fmaxf(fmaxf(r0.x, r0.y), fmaxf(r0.z, r0.w)),
                                 fmaxf(fmaxf(r1.x, r1.y), fmaxf(r1.z, r1.w)));
        const float mnew = fmaxf(m_run[ht], tmax);
        alpha[ht] = __builtin_amdgcn_exp2f(m_run[ht] - mnew);
        m_run[ht] = mnew;
        float p[4], psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = tt0 + i < lim;
          const float e = __builtin_amdgcn_exp2f(s_acc[ht][i] - mnew);
          psum += ok ? e : 0.f;
          float pv = e;
          if constexpr (FP8) pv *= vscv[i];
          p[i] = ok ? pv : 0.f;
        }
        l_run[ht] = l_run[ht] * alpha[ht] + psum;
        // P^T into the operand block (ht, k-step ks) of the p.V product
        int ks, gr;
        if constexpr (FP8) { ks = (w >> 2) * 2 + (g >> 1); gr = w & 3; }
        else { ks = w >> 1; gr = 2 * (w & 1) + (g >> 1); }
        uint2 pk;
        pk.x = pack_bf16x2(p[0], p[1]);
        pk.y = pack_bf16x2(p[2], p[3]);
        uint8_t* dst = reinterpret_cast<uint8_t*>(p_lds) +
                       ((ht * 4 + ks) * 64 + gr * 16 + c) * 16 + (g & 1) * 8;
        *reinterpret_cast<uint2*>(dst) = pk;
      }
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) o_acc[dt][ht] *= alpha[ht];

      // Tokens past the end: their V bytes are whatever the block holds; zero
      // them so that 0 * (garbage) cannot reach O.
      if (lim < kTile) {
        if constexpr (FP8) {
#pragma unroll
          for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
              uint4 u = vc[bb * 2 + dt];
              uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) {
                uint32_t msk = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (bb * 64 + g * 16 + q4 * 4 + e < lim) msk |= 0xffu << (8 * e);
                wd[q4] &= msk;
              }
              vc[bb * 2 + dt] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
            }
        } else {
#pragma unroll
          for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
#pragma unroll
              for (int s2 = 0; s2 < 2; ++s2) {
                const int base = bb * 64 + s2 * 32 + g * 8;
                uint4 u = vc[(bb * 2 + dt) * 2 + s2];
                u.x = keep_bf16(u.x, base + 0 < lim, base + 1 < lim);
                u.y = keep_bf16(u.y, base + 2 < lim, base + 3 < lim);
                u.z = keep_bf16(u.z, base + 4 < lim, base + 5 < lim);
                u.w = keep_bf16(u.w, base + 6 < lim, base + 7 < lim);
                vc[(bb * 2 + dt) * 2 + s2] = u;
              }
        }
      }
      __syncthreads();

      // ---- O^T[feature][head] += V^T . P^T   (features 32w..32w+31)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int bb = ks >> 1, s2 = ks & 1;
        bf16x8_t pop[4];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) pop[ht] = as_bf16x8(p_lds[(ht * 4 + ks) * 64 + lane]);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          bf16x8_t vop;
          if constexpr (FP8) {
            const uint4 u = vc[bb * 2 + dt];
            vop = s2 ? e4m3x8_to_bf16x8(u.z, u.w) : e4m3x8_to_bf16x8(u.x, u.y);
          } else {
            vop = as_bf16x8(vc[(bb * 2 + dt) * 2 + s2]);
          }
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) o_acc[dt][ht] = mfma_16x16x32(vop, pop[ht], o_acc[dt][ht]);
        }
      }
    }
  }

  // ---- row sums: lane partials -> wave -> workgroup
  float lsum[4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    float l = l_run[ht];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    lsum[ht] = l;
  }
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) red[(ht * 16 + c) * kWaves + w] = lsum[ht];
  }
  __syncthreads();
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const float4 r0 = reinterpret_cast<const float4*>(red)[(ht * 16 + c) * 2];
    const float4 r1 = reinterpret_cast<const float4*>(red)[(ht * 16 + c) * 2 + 1];
    lsum[ht] = ((r0.x + r0.y) + (r0.z + r0.w)) + ((r1.x + r1.y) + (r1.z + r1.w));
  }

  // ---- write: lane holds O^T[32w + 16dt + 4g + i][16ht + c]
  if (a.num_splits == 1) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const float inv = lsum[ht] > 0.f ? 1.0f / lsum[ht] : 0.f;
      const int head = ht * 16 + c;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int f = 32 * w + 16 * dt + 4 * g;
        const size_t o = (static_cast<size_t>(b) * kH + head) * kD + f;
        const f32x4_t v = o_acc[dt][ht] * inv;
        if (a.out_f32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + o) =
              make_float4(v[0], v[1], v[2], v[3]);
        } else {
          uint2 pk;
          pk.x = pack_bf16x2(v[0], v[1]);
          pk.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + o) = pk;
        }
      }
    }
  } else {
    const size_t row = static_cast<size_t>(b) * a.num_splits + split;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const int head = ht * 16 + c;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int f = 32 * w + 16 * dt + 4 * g;
        const f32x4_t v = o_acc[dt][ht];
        *reinterpret_cast<float4*>(a.part_o + (row * kH + head) * kD + f) =
            make_float4(v[0], v[1], v[2], v[3]);
      }
      if (w == 0 && g == 0) {
        float2 ml;
        ml.x = m_run[ht] * kLn2;     // natural-log units of the scaled logits
        ml.y = lsum[ht];
        *reinterpret_cast<float2*>(a.part_ml + (row * kH + head) * 2) = ml;
      }
    }
  }
}

hipError_t launch_decode_mfma(const AttnArgs& a, bool fp8, int B, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(B * a.num_splits)), block(64 * kWaves);
  if (fp8)
    hipLaunchKernelGGL(mfa_decode_mfma_kernel<true>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(mfa_decode_mfma_kernel<false>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mfa
