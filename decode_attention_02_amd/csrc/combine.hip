// Split-KV combine: log-sum-exp merge of per-split partials (o_j, m_j, l_j)
// of every (sequence, head):
//   m* = max_j m_j,  w_j = exp(m_j - m*),  out = sum_j w_j o_j / sum_j w_j l_j.
// Splits with l_j == 0 are empty and carry no weight; a head with only empty
// splits gives zeros. This is the exact re-association of the softmax sum
// that lets long contexts be spread over many workgroups (long contexts are
// where MFA's decoding cost lives: "Step-3 is Large yet Affordable" summary
// page, §4 Cost Analysis for LLM Decoding, attention dominating from 8K on).
#include "device_common.h"
#include "kernels.h"

namespace mfa {

__global__ __launch_bounds__(256) void mfa_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int S, int H, int d, void* out,
                                                          int out_f32) {
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const size_t row0 = static_cast<size_t>(b) * S;
  float mstar = -INFINITY;
  for (int s = 0; s < S; ++s) {
    const float2 ml = *reinterpret_cast<const float2*>(part_ml + ((row0 + s) * H + h) * 2);
    if (ml.y > 0.f) mstar = fmaxf(mstar, ml.x);
  }
  for (int j = threadIdx.x; j < d; j += blockDim.x) {
    float num = 0.f, den = 0.f;
    for (int s = 0; s < S; ++s) {
      const float2 ml = *reinterpret_cast<const float2*>(part_ml + ((row0 + s) * H + h) * 2);
      if (ml.y > 0.f) {
        const float wgt = expf(ml.x - mstar);
        den = fmaf(wgt, ml.y, den);
        num = fmaf(wgt, part_o[((row0 + s) * H + h) * d + j], num);
      }
    }
    const float val = den > 0.f ? num / den : 0.f;
    const size_t oi = (static_cast<size_t>(b) * H + h) * d + j;
    if (out_f32) reinterpret_cast<float*>(out)[oi] = val;
    else reinterpret_cast<uint16_t*>(out)[oi] = f32_to_bf16(val);
  }
}

hipError_t launch_combine(const float* part_o, const float* part_ml, int B, int H, int d,
                          int num_splits, void* out, int out_f32, hipStream_t stream) {
  const int threads = d >= 256 ? 256 : ((d + 63) / 64) * 64;
  hipLaunchKernelGGL(mfa_combine_kernel, dim3(static_cast<unsigned>(B * H)), dim3(threads), 0,
                     stream, part_o, part_ml, num_splits, H, d, out, out_f32);
  return hipGetLastError();
}

}  // namespace mfa
