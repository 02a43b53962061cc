// MFA query path: c = x W_qdown^T, n = RMSNorm(c; g), q = n W_qup^T.
//
// "Step-3 is Large yet Affordable" (summary page), §2 Step-3 Model Card:
// MFA factorises the QK circuit at low rank; the reading implemented is a
// down-projection to the query rank, an RMSNorm with gain, and an
// up-projection into the H query heads. §4 (Cost Analysis) counts these
// linear projections on top of the attention's own cost.
//
// At decode batch sizes (M <= 64 rows) both products are skinny: every
// weight byte is used by at most 64 rows, so they are bound by the weight
// stream from HBM. The bf16 kernel streams each weight row slice straight
// into registers in matrix-core operand layout (16 contiguous bytes per
// lane), stages the small activation panel through LDS, splits K across
// workgroups so that the grid covers the chip, and leaves fp32 partials;
// the RMSNorm (for the down product) or the bf16 cast (for the up product)
// sums them in a second pass.
#include "device_common.h"
#include "kernels.h"

namespace mfa {

namespace {
constexpr int kKC = 256;                 // K per LDS stage (8 k-steps of 32)
constexpr int kRow = kKC * 2 + 16;       // padded LDS row: conflict-free 16-lane reads
}

template <int MT>   // M tiles of 16 rows
__global__ __launch_bounds__(256) void gemm_bf16_splitk_kernel(const uint16_t* __restrict__ A,
                                                               const uint16_t* __restrict__ W,
                                                               float* __restrict__ part, int M,
                                                               int N, int K, int kchunk) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[MT * 16 * kRow];
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int n0 = blockIdx.x * 64 + w * 16;
  const int ks = blockIdx.y;
  const int kbeg = ks * kchunk, kend = kbeg + kchunk;

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // B operand: lane holds W[n0 + c][k + 8g .. +8]
  const uint16_t* wrow = W + static_cast<size_t>(n0 + c) * K + g * 8;
  uint4 wcur[8], wnxt[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) wcur[s] = *reinterpret_cast<const uint4*>(wrow + kbeg + s * 32);

  for (int k0 = kbeg; k0 < kend; k0 += kKC) {
    if (k0 + kKC < kend) {
#pragma unroll
      for (int s = 0; s < 8; ++s)
        wnxt[s] = *reinterpret_cast<const uint4*>(wrow + k0 + kKC + s * 32);
    }
    // A panel rows [0, MT*16) x [k0, k0+256): 32 pieces of 16 B per row
#pragma unroll
    for (int r = 0; r < MT * 2; ++r) {
      const int idx = tid + 256 * r;
      const int m = idx >> 5, piece = idx & 31;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < M) v = *reinterpret_cast<const uint4*>(A + static_cast<size_t>(m) * K + k0 + piece * 8);
      *reinterpret_cast<uint4*>(a_lds + m * kRow + piece * 16) = v;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8_t bop = as_bf16x8(wcur[s]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint4 av = *reinterpret_cast<const uint4*>(a_lds + (mt * 16 + c) * kRow + (s * 32 + g * 8) * 2);
        acc[mt] = mfma_16x16x32(as_bf16x8(av), bop, acc[mt]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 8; ++s) wcur[s] = wnxt[s];
  }
  // accumulator lane holds C[mt*16 + 4g + i][n0 + c]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + 4 * g + i;
      if (m < M) part[(static_cast<size_t>(ks) * M + m) * N + n0 + c] = acc[mt][i];
    }
}

__global__ __launch_bounds__(256) void rmsnorm_reduce_kernel(const float* __restrict__ part,
                                                             int ksplit, const float* __restrict__ g,
                                                             int M, int R, float eps, void* out,
                                                             int out_f32) {
  constexpr int kMaxPer = 32;          // R <= 8192
  __shared__ float wsum[4];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  float cv[kMaxPer];
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxPer; ++r) {
    const int j = tid + 256 * r;
    float cj = 0.f;
    if (j < R) {
      for (int ks = 0; ks < ksplit; ++ks) cj += part[(static_cast<size_t>(ks) * M + m) * R + j];
    }
    cv[r] = cj;
    ss = fmaf(cj, cj, ss);
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(R) + eps);
#pragma unroll
  for (int r = 0; r < kMaxPer; ++r) {
    const int j = tid + 256 * r;
    if (j < R) {
      const float v = cv[r] * inv * g[j];
      const size_t o = static_cast<size_t>(m) * R + j;
      if (out_f32) reinterpret_cast<float*>(out)[o] = v;
      else reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16(v);
    }
  }
}

__global__ __launch_bounds__(256) void reduce_cast_kernel(const float* __restrict__ part, int ksplit,
                                                          int M, int N, void* out, int out_f32) {
  const size_t total = static_cast<size_t>(M) * N;
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < total; i += static_cast<size_t>(gridDim.x) * 256) {
    float v = 0.f;
    for (int ks = 0; ks < ksplit; ++ks) v += part[static_cast<size_t>(ks) * total + i];
    if (out_f32) reinterpret_cast<float*>(out)[i] = v;
    else reinterpret_cast<uint16_t*>(out)[i] = f32_to_bf16(v);
  }
}

// fp32 path: one wave per output element, lanes stride K.
__global__ __launch_bounds__(256) void gemv_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ W,
                                                       float* __restrict__ out, int M, int N,
                                                       int K) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= M * N) return;
  const int m = wid / N, n = wid % N;
  const float* a = A + static_cast<size_t>(m) * K;
  const float* wr = W + static_cast<size_t>(n) * K;
  float acc = 0.f;
  for (int k = lane; k < K; k += 64) acc = fmaf(a[k], wr[k], acc);
  acc = wave_sum(acc);
  if (lane == 0) out[static_cast<size_t>(m) * N + n] = acc;
}

hipError_t launch_gemm_bf16_splitk(const uint16_t* A, const uint16_t* W, float* part, int M,
                                   int N, int K, int ksplit, hipStream_t stream) {
  const int kchunk = K / ksplit;
  dim3 grid(static_cast<unsigned>(N / 64), static_cast<unsigned>(ksplit)), block(256);
  if (M <= 16)
    hipLaunchKernelGGL(gemm_bf16_splitk_kernel<1>, grid, block, 0, stream, A, W, part, M, N, K, kchunk);
  else if (M <= 32)
    hipLaunchKernelGGL(gemm_bf16_splitk_kernel<2>, grid, block, 0, stream, A, W, part, M, N, K, kchunk);
  else
    hipLaunchKernelGGL(gemm_bf16_splitk_kernel<4>, grid, block, 0, stream, A, W, part, M, N, K, kchunk);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_reduce(const float* part, int ksplit, const float* g, int M, int R,
                                 float eps, void* out, int out_f32, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_reduce_kernel, dim3(static_cast<unsigned>(M)), dim3(256), 0, stream,
                     part, ksplit, g, M, R, eps, out, out_f32);
  return hipGetLastError();
}

hipError_t launch_reduce_cast(const float* part, int ksplit, int M, int N, void* out, int out_f32,
                              hipStream_t stream) {
  const size_t total = static_cast<size_t>(M) * N;
  size_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(reduce_cast_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     part, ksplit, M, N, out, out_f32);
  return hipGetLastError();
}

hipError_t launch_gemv_f32(const float* A, const float* W, float* out, int M, int N, int K,
                           hipStream_t stream) {
  const size_t waves = static_cast<size_t>(M) * N;
  hipLaunchKernelGGL(gemv_f32_kernel, dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0,
                     stream, A, W, out, M, N, K);
  return hipGetLastError();
}

}  // namespace mfa
