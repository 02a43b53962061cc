// KV append: writes new tokens of every sequence into the paged (or
// contiguous) cache. Attention instances own their KV caches ("Step-3 is
// Large yet Affordable" summary page, §7 Implementation and Results); the
// 8-bit cache option is the one §5 (Model-System Co-design) credits with
// raising arithmetic intensity.
//
// One workgroup covers the new tokens of one sequence that fall into one
// 64-token block. F32/BF16 caches copy bits; FP8 caches quantise each token:
// amax over the token's d values, scale = amax/448 (correctly rounded fp32
// division, 1 when amax = 0), code = RNE e4m3 of the correctly rounded
// quotient x/scale. Element positions inside a block follow kv_layout.h.
#include "device_common.h"
#include "kernels.h"
#include "kv_layout.h"
#include "append_one.h"

namespace mfa {

namespace {

__device__ __forceinline__ float load_in(const void* p, size_t i, int in_f32) {
  return in_f32 ? reinterpret_cast<const float*>(p)[i]
                : bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}

// Range of new tokens of sequence b that land in the workgroup's block.
struct Span {
  int lo, hi, blk, p0;
};

__device__ __forceinline__ Span block_span(const AppendArgs& a, int b, int jj) {
  Span s{0, 0, -1, 0};
  int p0 = a.pos[b];
  if (p0 < 0) return s;
  const int cap = a.max_blocks_per_seq * kBlockTokens;
  const int j = p0 / kBlockTokens + jj;
  if (j >= a.max_blocks_per_seq) return s;
  s.lo = max(p0, j * kBlockTokens);
  s.hi = min(min(p0 + a.n_new, (j + 1) * kBlockTokens), cap);
  s.p0 = p0;
  const int id = a.block_table ? a.block_table[static_cast<size_t>(b) * a.max_blocks_per_seq + j]
                               : b * a.max_blocks_per_seq + j;
  s.blk = (id < 0 || id >= a.num_blocks) ? -1 : id;   // unmapped: nothing written
  return s;
}

}  // namespace

template <typename T>
__device__ __forceinline__ uint32_t k_off(int t, int d, int D) {
  if constexpr (sizeof(T) == 4) return k_off_f32(t, d, D);
  else return k_off_bf16(t, d, D);
}

template <typename T>
__device__ __forceinline__ uint32_t v_off(int t, int f) {
  if constexpr (sizeof(T) == 4) return v_off_f32(t, f);
  else return v_off_bf16(t, f);
}

template <typename T>
__global__ __launch_bounds__(256) void kv_append_copy_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const Span sp = block_span(a, b, blockIdx.y);
  if (sp.lo >= sp.hi || sp.blk < 0) return;
  const int n = sp.hi - sp.lo, off0 = sp.lo & 63, i0 = sp.lo - sp.p0, d = a.d;
  const T* kin = reinterpret_cast<const T*>(a.k_new) + (static_cast<size_t>(b) * a.n_new + i0) * d;
  const T* vin = reinterpret_cast<const T*>(a.v_new) + (static_cast<size_t>(b) * a.n_new + i0) * d;
  const size_t block_bytes = static_cast<size_t>(kBlockTokens) * d * sizeof(T);
  uint8_t* kc = a.k + static_cast<size_t>(sp.blk) * block_bytes;
  uint8_t* vc = a.v + static_cast<size_t>(sp.blk) * block_bytes;
  for (int idx = threadIdx.x; idx < n * d; idx += 256) {
    const int t = idx / d, jd = idx % d;
    *reinterpret_cast<T*>(kc + k_off<T>(off0 + t, jd, d)) = kin[idx];
    *reinterpret_cast<T*>(vc + v_off<T>(off0 + t, jd)) = vin[idx];
  }
}

template <int EPT>   // elements per lane: d / 64
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(AppendArgs a) {
  __shared__ uint8_t vt[256][kBlockTokens];
  const int b = blockIdx.x;
  const Span sp = block_span(a, b, blockIdx.y);
  if (sp.lo >= sp.hi || sp.blk < 0) return;
  const int n = sp.hi - sp.lo, off0 = sp.lo & 63, i0 = sp.lo - sp.p0, d = a.d;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint8_t* kc = a.k + static_cast<size_t>(sp.blk) * kBlockTokens * d;
  for (int t = w; t < n; t += 4) {
    const size_t row = (static_cast<size_t>(b) * a.n_new + i0 + t) * d;
    float xk[EPT], xv[EPT];
    float ak = 0.f, av = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      xk[e] = load_in(a.k_new, row + lane * EPT + e, a.in_f32);
      xv[e] = load_in(a.v_new, row + lane * EPT + e, a.in_f32);
      ak = fmaxf(ak, fabsf(xk[e]));
      av = fmaxf(av, fabsf(xv[e]));
    }
    ak = wave_max(ak);
    av = wave_max(av);
    const float sk = ak > 0.f ? ak / 448.0f : 1.0f;
    const float sv = av > 0.f ? av / 448.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int jd = lane * EPT + e;
      kc[k_off_fp8(off0 + t, jd, d)] = static_cast<uint8_t>(encode_e4m3_rne(xk[e] / sk));
      vt[jd][t] = static_cast<uint8_t>(encode_e4m3_rne(xv[e] / sv));
    }
    if (lane == 0) {
      a.k_scale[static_cast<size_t>(sp.blk) * kBlockTokens + off0 + t] = sk;
      a.v_scale[static_cast<size_t>(sp.blk) * kBlockTokens + off0 + t] = sv;
    }
  }
  __syncthreads();
  uint8_t* vc = a.v + static_cast<size_t>(sp.blk) * d * kBlockTokens;
  for (int idx = threadIdx.x; idx < n * d; idx += 256) {
    const int jd = idx / n, t = idx % n;
    vc[v_off_fp8(off0 + t, jd)] = vt[jd][t];
  }
}

// Decode-step append (one new token per sequence): one wave per sequence.
template <int CACHE, int EPT, bool INF32>   // CACHE: 0 f32, 1 bf16, 2 fp8
__global__ __launch_bounds__(64) void kv_append_one_kernel(AppendArgs a) {
  append_token_wave<CACHE, EPT, INF32>(a, blockIdx.x, threadIdx.x);
}

template <int CACHE, bool INF32>
static void launch_one_in(const AppendArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(a.B)), block(64);
  if (a.d == 64) hipLaunchKernelGGL((kv_append_one_kernel<CACHE, 1, INF32>), grid, block, 0, stream, a);
  else if (a.d == 128) hipLaunchKernelGGL((kv_append_one_kernel<CACHE, 2, INF32>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((kv_append_one_kernel<CACHE, 4, INF32>), grid, block, 0, stream, a);
}
template <int CACHE>
static void launch_one(const AppendArgs& a, hipStream_t stream) {
  if (a.in_f32) launch_one_in<CACHE, true>(a, stream);
  else launch_one_in<CACHE, false>(a, stream);
}

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(a.B), static_cast<unsigned>((a.n_new + kBlockTokens - 1) / kBlockTokens + 1));
  dim3 block(256);
  if (a.d != 64 && a.d != 128 && a.d != 256) return hipErrorInvalidValue;
  if (a.n_new == 1) {
    if (a.cache_dtype == 0) launch_one<0>(a, stream);
    else if (a.cache_dtype == 1) launch_one<1>(a, stream);
    else launch_one<2>(a, stream);
    return hipGetLastError();
  }
  switch (a.cache_dtype) {
    case 0: hipLaunchKernelGGL(kv_append_copy_kernel<float>, grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL(kv_append_copy_kernel<uint16_t>, grid, block, 0, stream, a); break;
    case 2:
      if (a.d == 64) hipLaunchKernelGGL(kv_append_fp8_kernel<1>, grid, block, 0, stream, a);
      else if (a.d == 128) hipLaunchKernelGGL(kv_append_fp8_kernel<2>, grid, block, 0, stream, a);
      else if (a.d == 256) hipLaunchKernelGGL(kv_append_fp8_kernel<4>, grid, block, 0, stream, a);
      else return hipErrorInvalidValue;
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mfa
