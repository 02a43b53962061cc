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

// One workgroup of 256 threads covers 1024/d heads of one sequence; a thread
// owns 4 consecutive features of one head and reads one float4 per split.
// Partials are fp32 (o, m and l). Row b's partials are the S slots from
// b * S on, or, with meta (the balanced partition), meta[b] = (first slot,
// slot count).
// Workgroups are dispatched round-robin over the 8 XCDs (id % 8); the remap
// gives each XCD a contiguous range of sequences, the same range whose
// splits the attention kernel ran there.
// kBatch partials are loaded at once per batch; its registers (6 per
// partial) bound the occupancy, so rows with few partials (the balanced
// partition's 1..3, short split plans) use batches of 4, which fit every
// workgroup of the grid on the chip at once.
template <int kBatch>
__global__ __launch_bounds__(256) void mfa_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          const int* __restrict__ meta,
                                                          int S, int H, int d, void* out,
                                                          int out_f32) {
  const int tpb = d >> 2;                        // threads per head
  const int hpb = 256 / tpb;                     // heads per workgroup
  const int groups = (H + hpb - 1) / hpb;
  int id = blockIdx.x;
  if ((gridDim.x & 7) == 0) id = (id & 7) * (gridDim.x >> 3) + (id >> 3);
  const int b = id / groups;
  const int h = (id % groups) * hpb + threadIdx.x / tpb;
  const int f = (threadIdx.x % tpb) * 4;
  if (h >= H) return;
  size_t row0 = static_cast<size_t>(b) * S;
  if (meta) {
    using cint = const __attribute__((address_space(4))) int;
    row0 = static_cast<size_t>(((cint*)meta)[2 * b]);
    S = ((cint*)meta)[2 * b + 1];
  }
  // One pass: each batch of up to kBatch splits is loaded at once (every split's
  // partials are valid memory, empty ones too), then merged against a running
  // max; when a batch raises the max, the sums so far are rescaled by
  // exp(old - new), the same identity that merges the splits themselves.
  float mrun = -INFINITY, den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    float2 ml[kBatch];
    float4 o[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool in = s0 + j < S;
      ml[j] = in ? *reinterpret_cast<const float2*>(part_ml + ((row0 + s0 + j) * H + h) * 2)
                 : make_float2(-INFINITY, 0.f);
      const size_t po = ((row0 + s0 + j) * H + h) * d + f;
      o[j] = in ? *reinterpret_cast<const float4*>(part_o + po) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (ml[j].y > 0.f) bmax = fmaxf(bmax, ml[j].x);   // empty splits carry no weight
    if (bmax > mrun) {
      const float sc = mrun == -INFINITY ? 0.f : expf(mrun - bmax);
      den *= sc;
      num.x *= sc; num.y *= sc; num.z *= sc; num.w *= sc;
      mrun = bmax;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (ml[j].y > 0.f) {
        const float wgt = expf(ml[j].x - mrun);
        den = fmaf(wgt, ml[j].y, den);
        num.x = fmaf(wgt, o[j].x, num.x);
        num.y = fmaf(wgt, o[j].y, num.y);
        num.z = fmaf(wgt, o[j].z, num.z);
        num.w = fmaf(wgt, o[j].w, num.w);
      }
    }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  const size_t oi = (static_cast<size_t>(b) * H + h) * d + f;
  if (out_f32) {
    store_nt(reinterpret_cast<float*>(out) + oi, make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv));
  } else {
    uint2 pk;
    pk.x = pack_bf16x2(num.x * inv, num.y * inv);
    pk.y = pack_bf16x2(num.z * inv, num.w * inv);
    store_nt(reinterpret_cast<uint16_t*>(out) + oi, pk);
  }
}

hipError_t launch_combine(const float* part_o, const float* part_ml, const int* meta, int B,
                          int H, int d, int num_splits, void* out, int out_f32,
                          hipStream_t stream) {
  if (d % 4 || d > 1024) return hipErrorInvalidValue;
  const int hpb = 256 / (d / 4);
  const int groups = (H + hpb - 1) / hpb;
  const dim3 grid(static_cast<unsigned>(B * groups));
  if (meta || num_splits <= 4)
    hipLaunchKernelGGL(mfa_combine_kernel<4>, grid, dim3(256), 0, stream, part_o, part_ml, meta,
                       num_splits, H, d, out, out_f32);
  else
    hipLaunchKernelGGL(mfa_combine_kernel<16>, grid, dim3(256), 0, stream, part_o, part_ml, meta,
                       num_splits, H, d, out, out_f32);
  return hipGetLastError();
}

}  // namespace mfa
