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
// One workgroup (4 waves) owns one (sequence, split) pair and walks its
// 64-token cache blocks. Per block:
//   * wave w loads K rows 16w..16w+15 straight into registers in the
//     matrix-core operand layout (each lane: 16 contiguous bytes of a row),
//     and the V^T rows (features) 64w..64w+63: V blocks are stored
//     feature-major, so one lane's 8 tokens of one feature are contiguous;
//   * S^T[token][head] = K . Q^T on the matrix cores: tokens are the 16-row
//     side, the 64 heads sharing the KV head are four 16-column tiles read
//     from Q staged once in LDS in operand order;
//   * online softmax: per-head block max across the 4 waves through LDS,
//     p = exp2(s - m) in registers, lane-partial row sums;
//   * P^T goes through LDS (8 KB, in operand order) so every wave can apply
//     all 64 tokens to its 64 features: O^T[feature][head] += V^T . P^T.
// Each K and V byte is read from HBM exactly once per workgroup; FP8 codes
// are widened to bf16 in registers; per-token K scales multiply the logits,
// per-token V scales multiply P before its bf16 rounding.
// The next block's loads are issued before the current block's math.
#include "device_common.h"
#include "kernels.h"

namespace mfa {

namespace {

constexpr int kH = 64;
constexpr int kD = 256;

template <bool FP8>
struct Layout {
  // bytes per element / per cache block
  static constexpr int kElem = FP8 ? 1 : 2;
  static constexpr int kBlockBytes = kBlockTokens * kD * kElem;
  // 16-byte loads per lane per block
  static constexpr int kKLoads = FP8 ? 4 : 8;
  static constexpr int kVLoads = FP8 ? 4 : 8;
};

// d offset of operand k-step s for lane group g (the K and Q sides agree).
template <bool FP8>
__device__ __forceinline__ int qk_dim(int s, int g) {
  return FP8 ? ((s >> 1) * 64 + g * 16 + (s & 1) * 8) : (s * 32 + g * 8);
}

template <bool FP8>
__device__ __forceinline__ void load_block(const uint8_t* __restrict__ kblk,
                                           const uint8_t* __restrict__ vblk, int w, int g,
                                           int c, uint4 (&kr)[Layout<FP8>::kKLoads],
                                           uint4 (&vr)[Layout<FP8>::kVLoads]) {
  if constexpr (FP8) {
    // K row (16w+c), bytes u*64 + g*16 .. +16 ; V^T row (64w + dt*16 + c), bytes g*16 .. +16
    const uint8_t* kp = kblk + (16 * w + c) * kD + g * 16;
#pragma unroll
    for (int u = 0; u < 4; ++u) kr[u] = *reinterpret_cast<const uint4*>(kp + u * 64);
    const uint8_t* vp = vblk + (64 * w + c) * kBlockTokens + g * 16;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      vr[dt] = *reinterpret_cast<const uint4*>(vp + dt * 16 * kBlockTokens);
  } else {
    const uint8_t* kp = kblk + (16 * w + c) * (kD * 2) + g * 16;
#pragma unroll
    for (int s = 0; s < 8; ++s) kr[s] = *reinterpret_cast<const uint4*>(kp + s * 64);
    const uint8_t* vp = vblk + (64 * w + c) * (kBlockTokens * 2) + g * 16;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        vr[dt * 2 + s2] = *reinterpret_cast<const uint4*>(vp + dt * 16 * kBlockTokens * 2 + s2 * 64);
    }
  }
}

__device__ __forceinline__ uint32_t zero_bf16_lanes(uint32_t word, bool lo_ok, bool hi_ok) {
  return (lo_ok ? (word & 0xffffu) : 0u) | (hi_ok ? (word & 0xffff0000u) : 0u);
}

}  // namespace

template <bool FP8>
__global__ __launch_bounds__(256) void mfa_decode_mfma_kernel(AttnArgs a) {
  using LT = Layout<FP8>;
  __shared__ __attribute__((aligned(16))) uint4 q_lds[4 * 8 * 64];   // 32 KB
  __shared__ __attribute__((aligned(16))) uint4 p_lds[4 * 2 * 64];   // 8 KB
  __shared__ __attribute__((aligned(16))) float red[kH * 4];         // [head][wave]

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int split = blockIdx.x % a.num_splits;
  const int b = blockIdx.x / a.num_splits;

  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int t0 = split * a.chunk_tokens;
  const int t1 = min(t0 + a.chunk_tokens, L);

  f32x4_t o_acc[4][4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
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
    for (int r = 0; r < 8; ++r) {
      const int idx = tid + 256 * r;
      const int ln = idx & 63, blk = idx >> 6;
      const int ht = blk >> 3, s = blk & 7;
      const int gg = ln >> 4, cc = ln & 15;
      q_lds[idx] = *reinterpret_cast<const uint4*>(qb + (ht * 16 + cc) * kD + qk_dim<FP8>(s, gg));
    }

    const int tb0 = t0 >> 6;
    const int tb1 = (t1 + kBlockTokens - 1) >> 6;
    const int* bt_row = a.block_table ? a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq
                                      : nullptr;
    auto phys = [&](int tb) -> size_t {
      int id = bt_row ? bt_row[tb] : b * a.max_blocks_per_seq + tb;
      id = id < 0 ? 0 : (id >= a.num_blocks ? a.num_blocks - 1 : id);
      return static_cast<size_t>(id);
    };

    uint4 kr[LT::kKLoads], vr[LT::kVLoads];
    float4 ksc = make_float4(1.f, 1.f, 1.f, 1.f), vsc = ksc;
    {
      const size_t pb = phys(tb0);
      load_block<FP8>(a.k + pb * LT::kBlockBytes, a.v + pb * LT::kBlockBytes, w, g, c, kr, vr);
      if constexpr (FP8) {
        ksc = *reinterpret_cast<const float4*>(a.k_scale + pb * kBlockTokens + 16 * w + 4 * g);
        vsc = *reinterpret_cast<const float4*>(a.v_scale + pb * kBlockTokens + 16 * w + 4 * g);
      }
    }
    __syncthreads();   // Q staged

    for (int tb = tb0; tb < tb1; ++tb) {
      uint4 kc[LT::kKLoads], vc[LT::kVLoads];
#pragma unroll
      for (int i = 0; i < LT::kKLoads; ++i) kc[i] = kr[i];
#pragma unroll
      for (int i = 0; i < LT::kVLoads; ++i) vc[i] = vr[i];
      const float4 kscc = ksc, vscc = vsc;
      if (tb + 1 < tb1) {
        const size_t pb = phys(tb + 1);
        load_block<FP8>(a.k + pb * LT::kBlockBytes, a.v + pb * LT::kBlockBytes, w, g, c, kr, vr);
        if constexpr (FP8) {
          ksc = *reinterpret_cast<const float4*>(a.k_scale + pb * kBlockTokens + 16 * w + 4 * g);
          vsc = *reinterpret_cast<const float4*>(a.v_scale + pb * kBlockTokens + 16 * w + 4 * g);
        }
      }

      // ---- S^T = K . Q^T  (tokens 16w..16w+15 of this block, all 64 heads)
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

      // ---- scale, mask, block max per head
      const int tok0 = tb * kBlockTokens + 16 * w + 4 * g;   // token of s_acc[.][0]
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
          sv = (tok0 + i < t1) ? sv : -INFINITY;
          s_acc[ht][i] = sv;
          m = fmaxf(m, sv);
        }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        mx[ht] = m;
      }
      if (g == 0) {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) red[(ht * 16 + c) * 4 + w] = mx[ht];
      }
      __syncthreads();

      float alpha[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const float4 r4 = reinterpret_cast<const float4*>(red)[ht * 16 + c];
        const float tmax = fmaxf(fmaxf(r4.x, r4.y), fmaxf(r4.z, r4.w));
        const float mnew = fmaxf(m_run[ht], tmax);
        alpha[ht] = __builtin_amdgcn_exp2f(m_run[ht] - mnew);
        m_run[ht] = mnew;
        float p[4], psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = tok0 + i < t1;
          const float e = __builtin_amdgcn_exp2f(s_acc[ht][i] - mnew);
          psum += ok ? e : 0.f;
          float pv = e;
          if constexpr (FP8) pv *= vscv[i];
          p[i] = ok ? pv : 0.f;
        }
        l_run[ht] = l_run[ht] * alpha[ht] + psum;
        // P^T into the operand block of the p.V product
        int s2, gr;
        if constexpr (FP8) { s2 = g >> 1; gr = w; }
        else { s2 = w >> 1; gr = 2 * (w & 1) + (g >> 1); }
        uint2 pk;
        pk.x = pack_bf16x2(p[0], p[1]);
        pk.y = pack_bf16x2(p[2], p[3]);
        uint8_t* dst = reinterpret_cast<uint8_t*>(p_lds) +
                       ((ht * 2 + s2) * 64 + gr * 16 + c) * 16 + (g & 1) * 8;
        *reinterpret_cast<uint2*>(dst) = pk;
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) o_acc[dt][ht] *= alpha[ht];

      // Tokens past the end of the sequence: their V bytes are whatever the
      // block holds; zero them so that 0 * (garbage) cannot reach O.
      if (tb * kBlockTokens + kBlockTokens > t1) {
        const int lim = t1 - tb * kBlockTokens;   // valid tokens in this block
        if constexpr (FP8) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            uint32_t wd[4] = {vc[dt].x, vc[dt].y, vc[dt].z, vc[dt].w};
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              uint32_t m = 0;
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (g * 16 + q4 * 4 + e < lim) m |= 0xffu << (8 * e);
              wd[q4] &= m;
            }
            vc[dt] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
          }
        } else {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              const int base = s2 * 32 + g * 8;
              uint4 u = vc[dt * 2 + s2];
              u.x = zero_bf16_lanes(u.x, base + 0 < lim, base + 1 < lim);
              u.y = zero_bf16_lanes(u.y, base + 2 < lim, base + 3 < lim);
              u.z = zero_bf16_lanes(u.z, base + 4 < lim, base + 5 < lim);
              u.w = zero_bf16_lanes(u.w, base + 6 < lim, base + 7 < lim);
              vc[dt * 2 + s2] = u;
            }
        }
      }
      __syncthreads();

      // ---- O^T[feature][head] += V^T . P^T   (features 64w..64w+63)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8_t pop[4];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) pop[ht] = as_bf16x8(p_lds[(ht * 2 + s2) * 64 + lane]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          bf16x8_t vop;
          if constexpr (FP8) {
            const uint4 u = vc[dt];
            vop = s2 ? e4m3x8_to_bf16x8(u.z, u.w) : e4m3x8_to_bf16x8(u.x, u.y);
          } else {
            vop = as_bf16x8(vc[dt * 2 + s2]);
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
    for (int ht = 0; ht < 4; ++ht) red[(ht * 16 + c) * 4 + w] = lsum[ht];
  }
  __syncthreads();
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const float4 r4 = reinterpret_cast<const float4*>(red)[ht * 16 + c];
    lsum[ht] = (r4.x + r4.y) + (r4.z + r4.w);
  }

  // ---- write: lane holds O^T[64w + 16dt + 4g + i][16ht + c]
  if (a.num_splits == 1) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const float inv = lsum[ht] > 0.f ? 1.0f / lsum[ht] : 0.f;
      const int head = ht * 16 + c;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int f = 64 * w + 16 * dt + 4 * g;
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
      for (int dt = 0; dt < 4; ++dt) {
        const int f = 64 * w + 16 * dt + 4 * g;
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
  dim3 grid(static_cast<unsigned>(B * a.num_splits)), block(256);
  if (fp8)
    hipLaunchKernelGGL(mfa_decode_mfma_kernel<true>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(mfa_decode_mfma_kernel<false>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mfa
