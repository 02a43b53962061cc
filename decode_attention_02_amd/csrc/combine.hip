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

// One workgroup of 256 threads covers 1024/(d*NS) heads of one sequence; a
// thread owns 4 consecutive features of one head and reads one float4 per
// split. With NS > 1 (rows with many splits and too few rows to fill the
// chip), NS thread groups share each head: group i merges the i-th contiguous
// run of its splits, and the NS running states are merged in LDS, in group
// order, with the same identity.
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
// NTL: non-temporal loads of the partials (split plans: 64K steps 80.6-81.8
// -> 79.8-80.8 us; no gain for the balanced partition's, which keep plain
// loads).
template <bool NTL>
__device__ __forceinline__ float2 load_ml(const float* p) {
  if constexpr (NTL) {
    const f32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x2_t*>(p));
    return make_float2(v[0], v[1]);
  }
  return *reinterpret_cast<const float2*>(p);
}
template <bool NTL>
__device__ __forceinline__ float4 load_o(const float* p) {
  if constexpr (NTL) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
  }
  return *reinterpret_cast<const float4*>(p);
}

template <int kBatch, int NS, bool NTL>
__global__ __launch_bounds__(256) void mfa_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          const int* __restrict__ meta,
                                                          int S, int H, int d, void* out,
                                                          int out_f32) {
  const int tpb = d >> 2;                        // threads per head and split group
  const int hpb = 256 / (tpb * NS);              // heads per workgroup
  const int groups = (H + hpb - 1) / hpb;
  int id = blockIdx.x;
  if ((gridDim.x & 7) == 0) id = (id & 7) * (gridDim.x >> 3) + (id >> 3);
  const int b = id / groups;
  const int q = threadIdx.x / tpb;               // (head slot, split group)
  const int sg = q % NS;
  const int h = (id % groups) * hpb + q / NS;
  const int f = (threadIdx.x % tpb) * 4;
  const bool live = q < hpb * NS && h < H;
  if (NS == 1 && !live) return;
  size_t row0 = static_cast<size_t>(b) * S;
  if (meta) {
    using cint = const __attribute__((address_space(4))) int;
    row0 = static_cast<size_t>(((cint*)meta)[2 * b]);
    S = ((cint*)meta)[2 * b + 1];
  }
  // this group's splits [s_lo, s_hi)
  const int per = (S + NS - 1) / NS;
  const int s_lo = min(S, sg * per), s_hi = live ? min(S, s_lo + per) : s_lo;
  // One pass: each batch of up to kBatch splits is loaded at once (every split's
  // partials are valid memory, empty ones too), then merged against a running
  // max; when a batch raises the max, the sums so far are rescaled by
  // exp(old - new), the same identity that merges the splits themselves.
  float mrun = -INFINITY, den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = s_lo; s0 < s_hi; s0 += kBatch) {
    float2 ml[kBatch];
    float4 o[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool in = s0 + j < s_hi;
      ml[j] = in ? load_ml<NTL>(part_ml + ((row0 + s0 + j) * H + h) * 2) : make_float2(-INFINITY, 0.f);
      const size_t po = ((row0 + s0 + j) * H + h) * d + f;
      o[j] = in ? load_o<NTL>(part_o + po) : make_float4(0.f, 0.f, 0.f, 0.f);
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
  if constexpr (NS > 1) {
    // group 0 of each head merges the other groups' states in group order
    __shared__ float4 st_num[256];
    __shared__ float2 st_md[256];
    st_num[threadIdx.x] = num;
    st_md[threadIdx.x] = make_float2(mrun, den);
    __syncthreads();
    if (!live || sg != 0) return;
    float mall = mrun;
#pragma unroll
    for (int i = 1; i < NS; ++i) mall = fmaxf(mall, st_md[threadIdx.x + i * tpb].x);
    if (mall > -INFINITY) {
      // a group with no weight has mrun = -inf and den = num = 0
      const float w0 = expf(mrun - mall);
      den *= w0;
      num.x *= w0; num.y *= w0; num.z *= w0; num.w *= w0;
#pragma unroll
      for (int i = 1; i < NS; ++i) {
        const float2 md = st_md[threadIdx.x + i * tpb];
        const float4 ni = st_num[threadIdx.x + i * tpb];
        const float wi = expf(md.x - mall);
        den = fmaf(wi, md.y, den);
        num.x = fmaf(wi, ni.x, num.x);
        num.y = fmaf(wi, ni.y, num.y);
        num.z = fmaf(wi, ni.z, num.z);
        num.w = fmaf(wi, ni.w, num.w);
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

// Split groups per head: rows with many splits spread over NS thread groups
// while the grid is small (4 rows of 64 splits give 64 workgroups at
// NS = 1); each group keeps at least two splits.
static int combine_groups(long long grid1, int S, int tpb) {
  int ns = 1;
  while (ns < 4 && 2 * ns * tpb <= 256 && grid1 * ns < 1024 && S >= 4 * ns) ns *= 2;
  return ns;
}

template <int NS>
static void launch_combine_ns(const float* part_o, const float* part_ml, int B, int H, int d,
                              int S, void* out, int out_f32, hipStream_t stream) {
  const int hpb = 256 / ((d / 4) * NS);
  const dim3 grid(static_cast<unsigned>(B * ((H + hpb - 1) / hpb)));
  if ((S + NS - 1) / NS <= 4)
    hipLaunchKernelGGL((mfa_combine_kernel<4, NS, true>), grid, dim3(256), 0, stream, part_o, part_ml,
                       nullptr, S, H, d, out, out_f32);
  else
    hipLaunchKernelGGL((mfa_combine_kernel<16, NS, true>), grid, dim3(256), 0, stream, part_o, part_ml,
                       nullptr, S, H, d, out, out_f32);
}

hipError_t launch_combine(const float* part_o, const float* part_ml, const int* meta, int B,
                          int H, int d, int num_splits, void* out, int out_f32,
                          hipStream_t stream) {
  if (d % 4 || d > 1024) return hipErrorInvalidValue;
  const int tpb = d / 4;
  const int hpb = 256 / tpb;
  const int groups = (H + hpb - 1) / hpb;
  if (meta) {
    hipLaunchKernelGGL((mfa_combine_kernel<4, 1, false>), dim3(static_cast<unsigned>(B * groups)), dim3(256),
                       0, stream, part_o, part_ml, meta, num_splits, H, d, out, out_f32);
    return hipGetLastError();
  }
  const int ns = combine_groups(static_cast<long long>(B) * groups, num_splits, tpb);
  if (ns == 4) launch_combine_ns<4>(part_o, part_ml, B, H, d, num_splits, out, out_f32, stream);
  else if (ns == 2) launch_combine_ns<2>(part_o, part_ml, B, H, d, num_splits, out, out_f32, stream);
  else launch_combine_ns<1>(part_o, part_ml, B, H, d, num_splits, out, out_f32, stream);
  return hipGetLastError();
}

}  // namespace mfa
