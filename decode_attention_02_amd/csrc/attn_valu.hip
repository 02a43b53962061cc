// MFA decode attention on the vector ALUs, for head shapes the matrix-core
// kernel does not cover (any H <= 64 with H*d <= 8192, d in {64,128,256})
// and for fp32 caches. All arithmetic is fp32. Same semantics as the
// matrix-core kernel: all H heads attend to the one shared K/V head
// ("Step-3 is Large yet Affordable" summary page, §2 and §5), online softmax
// over 16- or 32-token tiles, natural exp.
#include "device_common.h"
#include "kernels.h"
#include "kv_layout.h"

namespace mfa {

namespace {
constexpr int kMaxHD = 8192;     // H*d limit (q staged in LDS)
constexpr int kMaxPerThread = kMaxHD / 256;
}

// KT tokens per tile; the next tile's K and V are loaded into registers
// while the current one is computed.
template <int D, int KT>
__global__ __launch_bounds__(256) void mfa_decode_valu_kernel(AttnArgs a) {
  constexpr int kPer = KT * D / 256;           // K (and V) elements per thread per tile
  __shared__ float q_s[kMaxHD];
  // K rows padded by one float: the score loop reads k_s[t][j] for the KT
  // tokens of a wave at once, which without the pad all fall in one bank
  __shared__ float k_s[KT][D + 1];
  __shared__ float v_s[KT][D];
  __shared__ float p_s[64][KT];
  __shared__ float alpha_s[64], m_s[64], l_s[64];

  const int H = a.heads;
  const int HD = H * D;
  const int tid = threadIdx.x;
  const int split = blockIdx.x % a.num_splits;
  const int b = blockIdx.x / a.num_splits;          // virtual row (q, partials, out)
  const int ql = a.q_len > 0 ? a.q_len : 1;
  const int bs = b / ql;                            // its sequence (cache, lengths)
  const int jq = b - bs * ql;                       // its query token: sees the sequence up to itself
  int L = a.seq_lens[bs] - (ql - 1 - jq);
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int t0 = split * a.chunk_tokens;
  const int t1 = min(t0 + a.chunk_tokens, L);

  for (int i = tid; i < HD; i += 256) {
    const size_t qi = static_cast<size_t>(b) * HD + i;
    q_s[i] = a.q_f32 ? reinterpret_cast<const float*>(a.q)[qi] : bf16_to_f32(a.q[qi]);
  }
  if (tid < H) { m_s[tid] = -INFINITY; l_s[tid] = 0.f; }
  float o[kMaxPerThread];
#pragma unroll
  for (int r = 0; r < kMaxPerThread; ++r) o[r] = 0.f;
  const int* bt_row = a.block_table ? a.block_table + static_cast<size_t>(bs) * a.max_blocks_per_seq
                                    : nullptr;
  float kr[kPer], vr[kPer];
  auto load_tile = [&](int tt) {               // element i = tid + 256 r: token i / D, dim i % D
    const int n = min(KT, t1 - tt);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = tid + 256 * r;
      const int t = i / D, j = i % D;
      float kv = 0.f, vv = 0.f;
      if (t < n) {
        const int tok = tt + t;
        int id = bt_row ? bt_row[tok >> 6] : bs * a.max_blocks_per_seq + (tok >> 6);
        id = id < 0 ? 0 : (id >= a.num_blocks ? a.num_blocks - 1 : id);
        const int off = tok & 63;
        if (a.kv_f32) {
          const uint8_t* kb = a.k + static_cast<size_t>(id) * kBlockTokens * D * 4;
          const uint8_t* vb = a.v + static_cast<size_t>(id) * kBlockTokens * D * 4;
          kv = *reinterpret_cast<const float*>(kb + k_off_f32(off, j, D));
          vv = *reinterpret_cast<const float*>(vb + v_off_f32(off, j));
        } else {
          const uint8_t* kb = a.k + static_cast<size_t>(id) * kBlockTokens * D * 2;
          const uint8_t* vb = a.v + static_cast<size_t>(id) * kBlockTokens * D * 2;
          kv = bf16_to_f32(*reinterpret_cast<const uint16_t*>(kb + k_off_bf16(off, j, D)));
          vv = bf16_to_f32(*reinterpret_cast<const uint16_t*>(vb + v_off_bf16(off, j)));
        }
      }
      kr[r] = kv;
      vr[r] = vv;
    }
  };
  if (t0 < t1) load_tile(t0);
  __syncthreads();

  for (int tt = t0; tt < t1; tt += KT) {
    const int n = min(KT, t1 - tt);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = tid + 256 * r;
      k_s[i / D][i % D] = kr[r];
      v_s[i / D][i % D] = vr[r];
    }
    __syncthreads();
    if (tt + KT < t1) load_tile(tt + KT);       // in flight during this tile
    for (int i = tid; i < H * KT; i += 256) {
      const int h = i / KT, t = i % KT;
      float s = -INFINITY;
      if (t < n) {
        float acc = 0.f;
        for (int j = 0; j < D; ++j) acc = fmaf(q_s[h * D + j], k_s[t][j], acc);
        s = acc * a.sm_scale;
      }
      p_s[h][t] = s;
    }
    __syncthreads();
    // online softmax of the tile, one thread per (head, token): the KT
    // threads of a head are adjacent lanes of one wave (KT divides 64), so
    // the tile's max and sum are butterfly reductions over them
    for (int i = tid; i < H * KT; i += 256) {
      const int h = i / KT, t = i % KT;
      const float s = p_s[h][t];                      // -inf past the end
      float mx = s;
#pragma unroll
      for (int off = 1; off < KT; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float mold = m_s[h];
      mx = fmaxf(mx, mold);
      const float p = t < n ? expf(s - mx) : 0.f;
      float sum = p;
#pragma unroll
      for (int off = 1; off < KT; off <<= 1) sum += __shfl_xor(sum, off);
      p_s[h][t] = p;
      if (t == 0) {
        const float al = expf(mold - mx);
        l_s[h] = l_s[h] * al + sum;
        m_s[h] = mx;
        alpha_s[h] = al;
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kMaxPerThread; ++r) {
      const int e = tid + 256 * r;
      if (e < HD) {
        const int h = e / D, j = e % D;
        float acc = o[r] * alpha_s[h];
        for (int t = 0; t < n; ++t) acc = fmaf(p_s[h][t], v_s[t][j], acc);
        o[r] = acc;
      }
    }
    __syncthreads();
  }

  if (a.num_splits == 1) {
#pragma unroll
    for (int r = 0; r < kMaxPerThread; ++r) {
      const int e = tid + 256 * r;
      if (e < HD) {
        const int h = e / D;
        const float l = l_s[h];
        const float val = l > 0.f ? o[r] / l : 0.f;
        const size_t oi = static_cast<size_t>(b) * HD + e;
        if (a.out_f32) reinterpret_cast<float*>(a.out)[oi] = val;
        else reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16(val);
      }
    }
  } else {
    const size_t row = static_cast<size_t>(b) * a.num_splits + split;
#pragma unroll
    for (int r = 0; r < kMaxPerThread; ++r) {
      const int e = tid + 256 * r;
      if (e < HD) {
        a.part_o[row * HD + e] = o[r];
      }
    }
    if (tid < H) {
      a.part_ml[(row * H + tid) * 2 + 0] = m_s[tid];
      a.part_ml[(row * H + tid) * 2 + 1] = l_s[tid];
    }
  }
}

hipError_t launch_decode_valu(const AttnArgs& a, int B, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(B * a.num_splits)), block(256);
  switch (a.head_dim) {
    case 64: hipLaunchKernelGGL((mfa_decode_valu_kernel<64, 32>), grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL((mfa_decode_valu_kernel<128, 32>), grid, block, 0, stream, a); break;
    case 256: hipLaunchKernelGGL((mfa_decode_valu_kernel<256, 16>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mfa
