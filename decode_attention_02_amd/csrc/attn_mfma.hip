// MFA decode attention on the matrix cores: 64 query heads of width 256
// against one shared K/V head, bf16 or OCP-e4m3 KV cache.
//
// The method: "Step-3 is Large yet Affordable" (summary page), §2 Step-3
// Model Card (many query heads share a small KV cache through MFA's
// low-rank QK circuit) and §5 Model-System Co-design (one KV head read once
// for all 64 heads: 128 flop per byte of an 8-bit cache, 64 per byte of a
// bf16 cache). §6 states the attention stays memory-bandwidth bound, so the
// kernel is built around keeping HBM busy: every K and V byte is read once,
// with several cache blocks in flight per compute unit at all times.
//
// One workgroup (8 waves, 2 per SIMD) owns one (sequence, split) pair and
// walks it one 64-token cache block at a time. The waves split by role:
//   * QK waves 0..3: wave w holds K rows 16w..16w+15 of each block and
//     computes S^T[token][head] = K . Q^T on the 16x16x32 matrix cores (the
//     16 tokens are the row side, the 64 heads sharing the KV head four
//     16-column tiles of Q, staged once in LDS in operand order); then the
//     online softmax: per-head block max across the four QK waves through
//     LDS, p = exp2(s - m), lane-partial row sums, P^T (bf16) into LDS;
//   * PV waves 4..7: wave 4+j holds the V^T rows (features) 64j..64j+63 of
//     each block and accumulates O^T[feature][head] += V^T . P^T.
// Each wave only ever holds its own role's operands, so a ring of R blocks
// of registers keeps R-1 blocks of loads in flight per wave (bf16: R = 4,
// 192 KB per compute unit). The three stages are skewed across iterations
// separated by one barrier each: iteration i computes S of block i, the
// softmax of block i-1 and the P.V product of block i-2.
// The running max is updated lazily: only when a block's max exceeds it by
// more than 2^8 (log2 units) are O and the row sums rescaled, so p <= 256;
// the result is the same softmax, normalised by the same reference at the end.
// Cache blocks are stored in operand order (kv_layout.h): every wave-wide
// 16-byte load reads 1 KB of contiguous memory and lands in the operand
// registers as is. FP8 codes are widened to bf16 in registers (exact);
// per-token K scales multiply the logits, V scales multiply P before its
// bf16 rounding.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mfa {

namespace {

constexpr int kH = 64;
constexpr int kD = 256;
constexpr float kLazy = 8.0f;           // rescale only when the max grows by > 2^8

template <bool FP8, int RING>
struct Cfg {
  static constexpr int kBlockBytes = kBlockTokens * kD * (FP8 ? 1 : 2);
  static constexpr int kLoads = FP8 ? 4 : 8;     // 16-byte loads per lane per block (K or V)
  static constexpr int kSlot = kLoads + (FP8 ? 2 : 0);   // + K and V scales (QK waves, FP8)
  static constexpr int kRing = RING;             // blocks of registers per wave
  static constexpr int kUnroll = RING % 2 ? 2 * RING : RING;   // multiple of the ring and of 2
};

// d offset of operand k-step s for lane group g (the K and Q sides agree).
template <bool FP8>
__device__ __forceinline__ int qk_dim(int s, int g) {
  return FP8 ? ((s >> 1) * 64 + g * 16 + (s & 1) * 8) : (s * 32 + g * 8);
}

// Calls f(std::integral_constant<int, I>) for I = I0 .. I1-1 (a compile-time
// unrolled loop: register arrays indexed by I stay in registers).
template <int I0, int I1, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < I1) {
    f(std::integral_constant<int, I0>{});
    static_for<I0 + 1, I1>(f);
  }
}

__device__ __forceinline__ uint32_t keep_bf16(uint32_t word, bool lo_ok, bool hi_ok) {
  return (lo_ok ? (word & 0xffffu) : 0u) | (hi_ok ? (word & 0xffff0000u) : 0u);
}

}  // namespace

template <bool FP8, int RING>
__global__ __launch_bounds__(512) void mfa_decode_mfma_kernel(AttnArgs a) {
  using C = Cfg<FP8, RING>;
  constexpr int R = C::kRing;
  constexpr int U = C::kUnroll;
  __shared__ __attribute__((aligned(16))) uint4 q_lds[4 * 8 * 64];      // 32 KB, operand order
  __shared__ __attribute__((aligned(16))) uint4 p_lds[2][4 * 2 * 64];   // 2 x 8 KB, operand order
  __shared__ __attribute__((aligned(16))) float red[2][kH * 4];         // block max [head][QK wave]
  __shared__ __attribute__((aligned(16))) float alpha_lds[2][kH];
  __shared__ int flag_lds[2];
  __shared__ __attribute__((aligned(16))) float lred[kH * 4];           // row sums [head][QK wave]
  __shared__ float m_lds[kH];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const bool is_qk = w < 4;
  const int ww = w & 3;                 // QK: token group; PV: feature group of 64
  const int split = blockIdx.x % a.num_splits;
  const int b = blockIdx.x / a.num_splits;

  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int t0 = split * a.chunk_tokens;
  const int t1 = min(t0 + a.chunk_tokens, L);
  const int blk0 = t0 >> 6;
  const int N = t0 < t1 ? ((t1 + kBlockTokens - 1) >> 6) - blk0 : 0;   // blocks to walk

  // QK state (lane holds heads 16ht + c)
  float m_run[4], l_run[4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) { m_run[ht] = -INFINITY; l_run[ht] = 0.f; }
  // acc: PV waves: O^T, lane holds O^T[64ww + 16dt + 4g + i][16ht + c];
  // QK waves: acc[parity][ht] keeps S of the last block until its softmax.
  // One array for both roles keeps the register budget of either role.
  f32x4_t acc[4][4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) acc[dt][ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (N > 0) {
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

    const int* bt_row = a.block_table ? a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq
                                      : nullptr;
    auto phys = [&](int n) -> size_t {   // physical id of the workgroup's n-th block
      const int j = blk0 + n;
      int id = bt_row ? bt_row[j] : b * a.max_blocks_per_seq + j;
      id = id < 0 ? 0 : (id >= a.num_blocks ? a.num_blocks - 1 : id);
      return static_cast<size_t>(id);
    };

    // Register rings: QK waves keep K blocks (+ FP8 scales), PV waves V blocks.
    uint4 ring[R][C::kSlot];
    auto issue = [&](auto slot_c, int n) __attribute__((always_inline)) {
      constexpr int slot = decltype(slot_c)::value;
      const size_t pb = phys(n);
      if (is_qk) {
        // units (tg = ww, s): K[16ww + c][..], 1 KB contiguous per load
        const uint8_t* kp = a.k + pb * C::kBlockBytes + (ww * C::kLoads) * 1024 + lane * 16;
        static_for<0, C::kLoads>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          ring[slot][s] = *reinterpret_cast<const uint4*>(kp + s * 1024);
        });
        if constexpr (FP8) {
          ring[slot][4] = *reinterpret_cast<const uint4*>(a.k_scale + pb * kBlockTokens + 16 * ww + 4 * g);
          ring[slot][5] = *reinterpret_cast<const uint4*>(a.v_scale + pb * kBlockTokens + 16 * ww + 4 * g);
        }
      } else {
        // bf16 units (fg = 4ww + s/2, ks = s%2); FP8 units fg = 4ww + s
        const uint8_t* vp = a.v + pb * C::kBlockBytes + (ww * C::kLoads) * 1024 + lane * 16;
        static_for<0, C::kLoads>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          ring[slot][s] = *reinterpret_cast<const uint4*>(vp + s * 1024);
        });
      }
    };
    static_for<0, R>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      if (r < N) issue(rc, r);
    });
    __syncthreads();   // Q staged

    uint4 vkeep[2];                       // FP8: V scales of the last two blocks, by parity
    vkeep[0] = vkeep[1] = make_uint4(0u, 0u, 0u, 0u);
    for (int base = 0; base < N + 2; base += U) {
      static_for<0, U>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        constexpr int rs = r % R;                 // ring slot of block i
        constexpr int rs2 = (r + 2 * R - 2) % R;  // ... of block i-2
        constexpr int par = r & 1, par1 = (r + 1) & 1;
        const int i = base + r;                   // base is a multiple of U: i = r mod R, mod 2
        if (i < N + 2) {
          if (is_qk) {
            // ---- S^T of block i
            if (i < N) {
              f32x4_t s_acc[4];
#pragma unroll
              for (int ht = 0; ht < 4; ++ht) s_acc[ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
              static_for<0, 8>([&](auto sc) {
                constexpr int s = decltype(sc)::value;
                bf16x8_t kop;
                if constexpr (FP8) {
                  const uint4 u = ring[rs][s >> 1];
                  kop = (s & 1) ? e4m3x8_to_bf16x8(u.z, u.w) : e4m3x8_to_bf16x8(u.x, u.y);
                } else {
                  kop = as_bf16x8(ring[rs][s]);
                }
#pragma unroll
                for (int ht = 0; ht < 4; ++ht)
                  s_acc[ht] = mfma_16x16x32(kop, as_bf16x8(q_lds[(ht * 8 + s) * 64 + lane]), s_acc[ht]);
              });
              // scale, mask, local max over this wave's 16 tokens
              const int lim = t1 - (blk0 + i) * kBlockTokens;
              const int tt0 = 16 * ww + 4 * g;
              float kscv[4] = {1.f, 1.f, 1.f, 1.f};
              if constexpr (FP8) {
                const uint4 k4 = ring[rs][4];
                kscv[0] = __uint_as_float(k4.x); kscv[1] = __uint_as_float(k4.y);
                kscv[2] = __uint_as_float(k4.z); kscv[3] = __uint_as_float(k4.w);
              }
#pragma unroll
              for (int ht = 0; ht < 4; ++ht) {
                float m = -INFINITY;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  float sv = s_acc[ht][e] * a.scale_log2;
                  if constexpr (FP8) sv *= kscv[e];
                  sv = (tt0 + e < lim) ? sv : -INFINITY;
                  s_acc[ht][e] = sv;
                  m = fmaxf(m, sv);
                }
                m = rows4_max(m);
                if (g == 0) red[i & 1][(ht * 16 + c) * 4 + ww] = m;
              }
#pragma unroll
              for (int ht = 0; ht < 4; ++ht) acc[par][ht] = s_acc[ht];
              // the slot is refilled below; the softmax of this block (next
              // iteration) still needs its V scales
              if constexpr (FP8) vkeep[par] = ring[rs][5];
              if (i + R < N) issue(std::integral_constant<int, rs>{}, i + R);
            }
            // ---- softmax of block i-1
            if (i >= 1 && i - 1 < N) {
              const int n = i - 1;
              const int lim = t1 - (blk0 + n) * kBlockTokens;
              const int tt0 = 16 * ww + 4 * g;
              float vscv[4] = {1.f, 1.f, 1.f, 1.f};
              if constexpr (FP8) {
                const uint4 v4 = vkeep[par1];
                vscv[0] = __uint_as_float(v4.x); vscv[1] = __uint_as_float(v4.y);
                vscv[2] = __uint_as_float(v4.z); vscv[3] = __uint_as_float(v4.w);
              }
              bool rescale = false;
              float4 rr[4];
#pragma unroll
              for (int ht = 0; ht < 4; ++ht) rr[ht] = reinterpret_cast<const float4*>(red[n & 1])[ht * 16 + c];
#pragma unroll
              for (int ht = 0; ht < 4; ++ht) {
                const float4 r4 = rr[ht];
                const float tmax = fmaxf(fmaxf(r4.x, r4.y), fmaxf(r4.z, r4.w));
                float alpha = 1.0f;
                if (tmax > m_run[ht] + kLazy) {          // also true for the first block
                  alpha = __builtin_amdgcn_exp2f(m_run[ht] - tmax);
                  m_run[ht] = tmax;
                  rescale = true;
                }
                float p[4], psum = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const bool ok = tt0 + e < lim;
                  const float ex = __builtin_amdgcn_exp2f(acc[par1][ht][e] - m_run[ht]);
                  psum += ok ? ex : 0.f;
                  float pv = ex;
                  if constexpr (FP8) pv *= vscv[e];
                  p[e] = ok ? pv : 0.f;
                }
                l_run[ht] = l_run[ht] * alpha + psum;
                if (ww == 0 && g == 0) alpha_lds[n & 1][ht * 16 + c] = alpha;
                // P^T into operand block (ht, ks) of buffer n&1
                int ks, gr;
                if constexpr (FP8) { ks = g >> 1; gr = ww; }
                else { ks = ww >> 1; gr = 2 * (ww & 1) + (g >> 1); }
                uint2 pk;
                pk.x = pack_bf16x2(p[0], p[1]);
                pk.y = pack_bf16x2(p[2], p[3]);
                uint8_t* dst = reinterpret_cast<uint8_t*>(p_lds[n & 1]) +
                               ((ht * 2 + ks) * 64 + gr * 16 + c) * 16 + (g & 1) * 8;
                *reinterpret_cast<uint2*>(dst) = pk;
              }
              if (ww == 0) {
                const bool any = __ballot(rescale) != 0ull;
                if (lane == 0) flag_lds[n & 1] = any ? 1 : 0;
              }
            }
          } else {
            // ---- O^T += V^T . P^T of block i-2
            if (i >= 2 && i - 2 < N) {
              const int n = i - 2;
              constexpr int slot = rs2;
              if (flag_lds[n & 1]) {
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) {
                  const float al = alpha_lds[n & 1][ht * 16 + c];
#pragma unroll
                  for (int dt = 0; dt < 4; ++dt) acc[dt][ht] *= al;
                }
              }
              const int lim = t1 - (blk0 + n) * kBlockTokens;
              if (lim < kBlockTokens) {
                // tokens past the end: zero their V so 0 * (garbage) cannot reach O
                static_for<0, C::kLoads>([&](auto sc) {
                  constexpr int s = decltype(sc)::value;
                  uint4 u = ring[slot][s];
                  if constexpr (FP8) {
                    uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                      uint32_t msk = 0;
#pragma unroll
                      for (int e = 0; e < 4; ++e)
                        if (g * 16 + q4 * 4 + e < lim) msk |= 0xffu << (8 * e);
                      wd[q4] &= msk;
                    }
                    u = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                  } else {
                    const int tb = (s & 1) * 32 + g * 8;      // unit (dt = s/2, ks = s%2)
                    u.x = keep_bf16(u.x, tb + 0 < lim, tb + 1 < lim);
                    u.y = keep_bf16(u.y, tb + 2 < lim, tb + 3 < lim);
                    u.z = keep_bf16(u.z, tb + 4 < lim, tb + 5 < lim);
                    u.w = keep_bf16(u.w, tb + 6 < lim, tb + 7 < lim);
                  }
                  ring[slot][s] = u;
                });
              }
              static_for<0, 2>([&](auto ksc) {
                constexpr int ks = decltype(ksc)::value;
                bf16x8_t pop[4];
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) pop[ht] = as_bf16x8(p_lds[n & 1][(ht * 2 + ks) * 64 + lane]);
                static_for<0, 4>([&](auto dtc) {
                  constexpr int dt = decltype(dtc)::value;
                  bf16x8_t vop;
                  if constexpr (FP8) {
                    const uint4 u = ring[slot][dt];
                    vop = ks ? e4m3x8_to_bf16x8(u.z, u.w) : e4m3x8_to_bf16x8(u.x, u.y);
                  } else {
                    vop = as_bf16x8(ring[slot][dt * 2 + ks]);
                  }
#pragma unroll
                  for (int ht = 0; ht < 4; ++ht) acc[dt][ht] = mfma_16x16x32(vop, pop[ht], acc[dt][ht]);
                });
              });
              if (n + R < N) issue(std::integral_constant<int, slot>{}, n + R);
            }
          }
          __syncthreads();
        }
      });
    }
  }

  // ---- row sums (QK waves) -> LDS -> PV waves normalise and write
  if (is_qk) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const float l = rows4_sum(l_run[ht]);
      if (g == 0) lred[(ht * 16 + c) * 4 + ww] = l;
      if (ww == 0 && g == 0) m_lds[ht * 16 + c] = m_run[ht];
    }
  }
  __syncthreads();
  if (!is_qk) {
    float lsum[4], mh[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const float4 r4 = reinterpret_cast<const float4*>(lred)[ht * 16 + c];
      lsum[ht] = (r4.x + r4.y) + (r4.z + r4.w);
      mh[ht] = m_lds[ht * 16 + c];
    }
    if (a.num_splits == 1) {
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const float inv = lsum[ht] > 0.f ? 1.0f / lsum[ht] : 0.f;
        const int head = ht * 16 + c;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int f = 64 * ww + 16 * dt + 4 * g;
          const size_t o = (static_cast<size_t>(b) * kH + head) * kD + f;
          const f32x4_t v = acc[dt][ht] * inv;
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
        for (int dt = 0; dt < 4; ++dt) {
          const int f = 64 * ww + 16 * dt + 4 * g;
          const f32x4_t v = acc[dt][ht];
          *reinterpret_cast<float4*>(a.part_o + (row * kH + head) * kD + f) =
              make_float4(v[0], v[1], v[2], v[3]);
        }
        if (ww == 0 && g == 0) {
          float2 ml;
          ml.x = mh[ht] * kLn2;     // natural-log units of the scaled logits
          ml.y = lsum[ht];
          *reinterpret_cast<float2*>(a.part_ml + (row * kH + head) * 2) = ml;
        }
      }
    }
  }
}

hipError_t launch_decode_mfma(const AttnArgs& a, bool fp8, int B, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(B * a.num_splits)), block(512);
  if (fp8)
    hipLaunchKernelGGL((mfa_decode_mfma_kernel<true, 4>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((mfa_decode_mfma_kernel<false, 3>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mfa
