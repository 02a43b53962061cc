// Read-bandwidth probe for the benchmark: not part of the MFA method.
//
// Streams a buffer once with 16-byte buffer loads (4 per lane in flight),
// optionally marked non-temporal, so that a kernel's achieved bandwidth can
// be set beside what a pure stream of the same bytes reaches on the same
// device. Each workgroup reads one contiguous range of bytes / grid.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

template <int CP>
__global__ __launch_bounds__(512) void stream_probe_kernel(const uint8_t* __restrict__ base, int per,
                                                           uint4* __restrict__ sink) {
  constexpr int kUnroll = 4;
  const uint8_t* p = base + static_cast<size_t>(blockIdx.x) * per;
  // loads past the workgroup's range read nothing and return zeros
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), 0, per, 0x00020000);
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int off = threadIdx.x * 16; off < per; off += 512 * 16 * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off + u * 512 * 16, 0, CP));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      acc.x ^= v[u].x; acc.y ^= v[u].y; acc.z ^= v[u].z; acc.w ^= v[u].w;
    }
  }
  // keeps the loads live; a write happens only for one improbable value
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

}  // namespace

// Streams bytes of buf (bytes % (16 * grid) == 0, bytes / grid < 2^31) with
// grid workgroups of 512 threads; sink: 512 x 16 bytes of device memory.
// Returns 0, or -1 for bad arguments, -2 for a launch error.
extern "C" int mfa_probe_stream(const void* buf, size_t bytes, int grid, int nontemporal,
                                void* sink, void* stream) {
  if (!buf || !sink || grid < 1 || bytes % (16ull * grid) || bytes / grid >= (1ull << 31)) return -1;
  const int per = static_cast<int>(bytes / grid);
  auto st = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(stream_probe_kernel<2>, dim3(grid), dim3(512), 0, st,
                       static_cast<const uint8_t*>(buf), per, static_cast<uint4*>(sink));
  else
    hipLaunchKernelGGL(stream_probe_kernel<0>, dim3(grid), dim3(512), 0, st,
                       static_cast<const uint8_t*>(buf), per, static_cast<uint4*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
