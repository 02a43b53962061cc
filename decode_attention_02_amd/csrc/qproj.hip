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
// stream from HBM. The bf16 kernel streams weight row slices straight into
// registers in matrix-core operand layout (16 contiguous bytes per lane),
// splits K across workgroups when the output alone cannot fill the chip,
// and leaves fp32 partials that the RMSNorm pass sums (down product) or
// writes bf16 directly (up product, one K slice).
#include <type_traits>

#include "append_one.h"
#include "device_common.h"
#include "kernels.h"

namespace mfa {

// Skinny bf16 product on the matrix cores: part[ks][m][n] = sum over the K
// slice ks of A[m][k] * W[n][k] for m < M <= 128.
//
// A workgroup of 8 waves owns NT*16 output columns and one K slice; the
// waves take interleaved 32-wide k-steps of that slice, so every wave
// streams distinct weight bytes. Per k-step a wave loads NT weight fragments
// (lane: 16 contiguous bytes of one weight row) through buffer resources and
// MT activation fragments (lane: 16 bytes of one activation row; the
// activations are small and stay in L2), keeping PD k-steps of loads in
// flight. The eight waves' accumulators are summed through LDS at the end;
// the sum is written as fp32 partials, or as bf16 directly when the product
// has a single K slice.
// Weights: row-major [N][K] (PACKED = false) or packed in operand order
// (PACKED = true): 1 KB unit (nt = n/16, kt = k/32) at unit index
// nt*(K/32) + kt, lane 16*((k%32)/8) + n%16 holding W[n][8*(k/8) .. +8], so
// that each wave-wide weight load reads 1 KB of contiguous memory.
// Activations: row-major [M][K] (PA = false) or packed in operand order
// (PA = true, written so by the RMSNorm pass): 1 KB unit (kt = k/32,
// mt = m/16) at unit index kt*MT + mt, lane 16*((k%32)/8) + m%16 holding
// A[m][8*(k/8) .. +8]; rows M .. 16*MT-1 of the last tile are don't-care
// (they feed only output rows that are not written).
constexpr int kGemmWaves = 8;

// Sum the waves' accumulators for rows r0 .. r0+TM-1 of the tile (red[w]
// holds them at row r - r0) and write rows below M: fp32 partials of slice
// ks, or bf16 when out_bf16 is set.
template <int TM, int TN, int kPad>
__device__ __forceinline__ void gemm_store_rows(const float (*red)[TM * kPad], int tid, int r0,
                                                int M, int N, int n0, int ks,
                                                float* __restrict__ part,
                                                uint16_t* __restrict__ out_bf16) {
  constexpr int kOut = TM * TN;
  if constexpr (kOut % (kGemmWaves * 64) != 0 || (kOut / (kGemmWaves * 64)) % 2 == 1) {
    // tile sizes that do not split into pairs per thread: one output at a time
    for (int e = tid; e < kOut; e += kGemmWaves * 64) {
      const int ml = e / TN, nl = e % TN, m = r0 + ml;
      if (m >= M) continue;
      float sum = 0.f;
#pragma unroll
      for (int ww = 0; ww < kGemmWaves; ++ww) sum += red[ww][ml * kPad + nl];
      if (out_bf16)
        __builtin_nontemporal_store(f32_to_bf16(sum), out_bf16 + static_cast<size_t>(m) * N + n0 + nl);
      else
        store_nt(part + (static_cast<size_t>(ks) * M + m) * N + n0 + nl, sum);
    }
  } else {
    constexpr int kPer = kOut / (kGemmWaves * 64);   // outputs per thread (contiguous in n)
    const int e0 = tid * kPer;
    const int ml = e0 / TN, nl = e0 % TN, m = r0 + ml;
    if (m >= M) return;
    float v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int o = ml * kPad + nl + j;
      float sum = 0.f;
#pragma unroll
      for (int ww = 0; ww < kGemmWaves; ++ww) sum += red[ww][o];
      v[j] = sum;
    }
    if (out_bf16) {
      uint16_t* dst = out_bf16 + static_cast<size_t>(m) * N + n0 + nl;
#pragma unroll
      for (int j = 0; j < kPer; j += 2) store_nt(dst + j, pack_bf16x2(v[j], v[j + 1]));
    } else {
      float* dst = part + (static_cast<size_t>(ks) * M + m) * N + n0 + nl;
#pragma unroll
      for (int j = 0; j < kPer; j += 2) store_nt(dst + j, make_float2(v[j], v[j + 1]));
    }
  }
}

// NTW marks the weight loads non-temporal: a weight that is read once per
// call streams through L2 without pushing out the activations and partials
// (measured: the down-projection's 29 MB this way saves 2.5 us per decode
// step, the up-projection's 67 MB costs 1 us, the output projection's 235 MB
// saves 3-5 %).
// Columns N1 .. N-1 may come from a second weight matrix W2 (rows 0 ..
// N-N1-1 of it; null W2: all from W), so two products that share A run as
// one launch (the down-projection and the K/V projection share x).
template <int MT, int NT, int PD, bool PACKED, bool PA, bool NTW>
__global__ __launch_bounds__(kGemmWaves * 64) void gemm_skinny_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, float* __restrict__ part,
    uint16_t* __restrict__ out_bf16, int M, int N, int K, int kchunk,
    const uint16_t* __restrict__ W2, int N1) {
  constexpr int TN = NT * 16;
  constexpr int RG = MT < 4 ? MT : 4;                // row tiles per LDS reduction round
  constexpr int kPad = TN + 4;                       // padded LDS row (floats)
  __shared__ __attribute__((aligned(16))) float red[kGemmWaves][RG * 16 * kPad];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int n0 = blockIdx.x * TN;
  const int ks = blockIdx.y;
  const int kbeg = ks * kchunk;
  const int nsteps = kchunk / 32;                    // k-steps in the slice
  const int mine = (nsteps - w + kGemmWaves - 1) / kGemmWaves;   // k-steps w, w+8, ...

  // one buffer resource per 16-row weight tile, covering this K slice; the
  // lane offset of k-step kk is wofs + kk * kstep_bytes
  __amdgpu_buffer_rsrc_t wr[NT];
  int wofs;
  constexpr int kStepBytes = PACKED ? 1024 : 64;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    // 16-row group nt of the tile: from W2 at and past column N1
    const int col = n0 + nt * 16;
    const bool second = W2 != nullptr && col >= N1;
    const uint16_t* Wt = second ? W2 : W;
    const int nw = second ? col - N1 : col;          // its first row in Wt
    const uint16_t* base;
    int bytes;
    if constexpr (PACKED) {
      base = Wt + static_cast<size_t>((nw / 16) * (K / 32) + kbeg / 32) * 64 * 8;
      bytes = nsteps * 1024;
    } else {
      base = Wt + static_cast<size_t>(nw) * K + kbeg;
      bytes = (15 * K + kchunk) * 2;
    }
    wr[nt] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, bytes, 0x00020000);
  }
  if constexpr (PACKED) wofs = lane * 16;
  else wofs = (c * K + g * 8) * 2;
  const uint16_t* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + c, M - 1);           // rows >= M feed only rows >= M of C
    ap[mt] = A + static_cast<size_t>(m) * K + kbeg + g * 8;
  }

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 wb[PD][NT], ab[PD][MT];
  auto issue = [&](int slot, int j) {                // j-th k-step of this wave
    const int kk = w + kGemmWaves * j;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      wb[slot][nt] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(wr[nt], wofs + kk * kStepBytes, 0, NTW ? 2 : 0));
    if constexpr (PA) {
      const uint16_t* au = A + static_cast<size_t>((kbeg / 32 + kk) * MT) * 64 * 8 + lane * 8;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) ab[slot][mt] = *reinterpret_cast<const uint4*>(au + mt * 64 * 8);
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) ab[slot][mt] = *reinterpret_cast<const uint4*>(ap[mt] + kk * 32);
    }
  };
#pragma unroll
  for (int p = 0; p < PD; ++p)
    if (p < mine) issue(p, p);
  for (int j0 = 0; j0 < mine; j0 += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int j = j0 + p;
      if (j < mine) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt][nt] = mfma_16x16x32(as_bf16x8(ab[p][mt]), as_bf16x8(wb[p][nt]), acc[mt][nt]);
        if (j + PD < mine) issue(p, j + PD);
      }
    }
  }

  // accumulator lane holds C[mt*16 + 4g + i][nt*16 + c]; the waves' sums
  // meet in LDS, RG row tiles at a time
#pragma unroll
  for (int mg = 0; mg < MT; mg += RG) {
    if (mg) __syncthreads();                         // previous group's reads are done
#pragma unroll
    for (int mt = 0; mt < RG; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[w][(mt * 16 + 4 * g + i) * kPad + nt * 16 + c] = acc[mg + mt][nt][i];
    __syncthreads();
    gemm_store_rows<RG * 16, TN, kPad>(red, tid, mg * 16, M, N, n0, ks, part, out_bf16);
  }
}

// c[m][:] = sum of the K-slice partials; n = c / sqrt(mean(c^2) + eps) * g.
// One workgroup per row; each thread owns 8 consecutive columns per 2048.
// With APPEND, workgroups M.. of the grid write the decode step's new KV
// tokens instead (wave w of workgroup M + j appends sequences 4j + w,
// 4j + w + 4*(gridDim.x - M), ...): the two small, latency-bound jobs share
// one launch and their memory latencies overlap.
template <bool APPEND>
__global__ __launch_bounds__(256) void rmsnorm_reduce_kernel(const float* __restrict__ part,
                                                             int ksplit, const float* __restrict__ g,
                                                             int M, int R, int pstride, float eps,
                                                             void* out, int out_f32, int out_tiles,
                                                             AppendArgs app) {
  constexpr int kMaxChunks = 4;        // R <= 8192 = 4 chunks of 2048
  __shared__ float wsum[4];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  if constexpr (APPEND) {
    if (m >= M) {
      const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
      if (app.kv_part) {
        // projected tokens: one sequence per workgroup (wave 0), so the K-slice
        // partials of the rows are read by as many compute units as rows
        if (w == 0) append_token(app, app.kv_row0 + (m - M), tid & 63);
        return;
      }
      const int per = (gridDim.x - M) * 4;
      for (int b = (m - M) * 4 + w; b < app.B; b += per) append_token(app, b, tid & 63);
      return;
    }
  }
  float cv[kMaxChunks][8];
  // the gain is loaded with the partials, not after the barrier, so its
  // latency overlaps theirs
  float4 gv[kMaxChunks][2];
#pragma unroll
  for (int ch = 0; ch < kMaxChunks; ++ch) {
    const int j0 = ch * 2048 + tid * 8;
    if (j0 < R) {
      gv[ch][0] = *reinterpret_cast<const float4*>(g + j0);
      gv[ch][1] = *reinterpret_cast<const float4*>(g + j0 + 4);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int ch = 0; ch < kMaxChunks; ++ch) {
    const int j0 = ch * 2048 + tid * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) cv[ch][j] = 0.f;
    if (j0 < R) {
      // slices in groups of 8 with all loads of a group in flight at once
      // (the sum stays in slice order)
      for (int k0 = 0; k0 < ksplit; k0 += 8) {
        float4 a[8], b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (k0 + u < ksplit) {
            const float* p = part + (static_cast<size_t>(k0 + u) * M + m) * pstride + j0;
            a[u] = *reinterpret_cast<const float4*>(p);
            b[u] = *reinterpret_cast<const float4*>(p + 4);
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (k0 + u < ksplit) {
            cv[ch][0] += a[u].x; cv[ch][1] += a[u].y; cv[ch][2] += a[u].z; cv[ch][3] += a[u].w;
            cv[ch][4] += b[u].x; cv[ch][5] += b[u].y; cv[ch][6] += b[u].z; cv[ch][7] += b[u].w;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(cv[ch][j], cv[ch][j], ss);
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(R) + eps);
#pragma unroll
  for (int ch = 0; ch < kMaxChunks; ++ch) {
    const int j0 = ch * 2048 + tid * 8;
    if (j0 < R) {
      const float gg[8] = {gv[ch][0].x, gv[ch][0].y, gv[ch][0].z, gv[ch][0].w,
                           gv[ch][1].x, gv[ch][1].y, gv[ch][1].z, gv[ch][1].w};
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = cv[ch][j] * inv * gg[j];
      const size_t o = static_cast<size_t>(m) * R + j0;
      if (out_f32) {
        float* d = reinterpret_cast<float*>(out) + o;
        *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(d + 4) = make_float4(v[4], v[5], v[6], v[7]);
      } else {
        uint4 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        pk.z = pack_bf16x2(v[4], v[5]);
        pk.w = pack_bf16x2(v[6], v[7]);
        // packed: unit (kt, mt) = (j0 / 32, m / 16), lane 16 * ((j0 % 32) / 8) + m % 16
        const size_t po = out_tiles
            ? (static_cast<size_t>((j0 >> 5) * out_tiles + (m >> 4)) * 64 + ((j0 >> 3) & 3) * 16 + (m & 15)) * 8
            : o;
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + po) = pk;
      }
    }
  }
}

// Attention output projection, second half: y[m][:] = sum of the K-slice
// partials, rounded to bf16; then the per-token FP8 pack of the bf16 row for
// the attention-to-FFN hand-off ("Step-3 is Large yet Affordable" summary
// page, §7: FP8 tokens with their scales go from attention to FFN):
// amax over the row, scale = amax / 448 (1 when amax = 0), code = RNE e4m3
// of the correctly rounded quotient. One 1024-thread workgroup per row, 8
// consecutive columns per thread, so every load of the row is issued at once.
constexpr int kPackThreads = 1024;
__global__ __launch_bounds__(kPackThreads) void outproj_pack_kernel(const float* __restrict__ part,
                                                                    int ksplit, int M, int N,
                                                                    uint16_t* __restrict__ y,
                                                                    uint8_t* __restrict__ codes,
                                                                    float* __restrict__ scales) {
  __shared__ float wmax[kPackThreads / 64];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const int j0 = tid * 8;
  float yv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) yv[j] = 0.f;
  float amax = 0.f;
  if (j0 < N) {
    for (int k0 = 0; k0 < ksplit; k0 += 8) {         // slices in slice order, 8 in flight
      float4 a[8], b[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (k0 + u < ksplit) {
          const float* p = part + (static_cast<size_t>(k0 + u) * M + m) * N + j0;
          a[u] = *reinterpret_cast<const float4*>(p);
          b[u] = *reinterpret_cast<const float4*>(p + 4);
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (k0 + u < ksplit) {
          yv[0] += a[u].x; yv[1] += a[u].y; yv[2] += a[u].z; yv[3] += a[u].w;
          yv[4] += b[u].x; yv[5] += b[u].y; yv[6] += b[u].z; yv[7] += b[u].w;
        }
      }
    }
    uint32_t bits[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      bits[j / 2] = pack_bf16x2(yv[j], yv[j + 1]);
      yv[j] = __uint_as_float(bits[j / 2] << 16);                     // the bf16 values
      yv[j + 1] = __uint_as_float(bits[j / 2] & 0xffff0000u);
      amax = fmaxf(amax, fmaxf(fabsf(yv[j]), fabsf(yv[j + 1])));
    }
    if (y) store_nt(y + static_cast<size_t>(m) * N + j0, make_uint4(bits[0], bits[1], bits[2], bits[3]));
  }
  if (!codes) return;                  // uniform: no pack asked for
  amax = wave_max(amax);
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = wmax[0];
#pragma unroll
  for (int w = 1; w < kPackThreads / 64; ++w) amax = fmaxf(amax, wmax[w]);
  const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
  if (j0 < N) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w0 |= encode_e4m3_rne(yv[j] / sc) << (8 * j);
      w1 |= encode_e4m3_rne(yv[4 + j] / sc) << (8 * j);
    }
    store_nt(codes + static_cast<size_t>(m) * N + j0, make_uint2(w0, w1));
  }
  if (tid == 0) scales[m] = sc;
}

hipError_t launch_outproj_pack(const float* part, int ksplit, int M, int N, uint16_t* y,
                               uint8_t* codes, float* scales, hipStream_t stream) {
  if (N % 8 || N > 8 * kPackThreads || M < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(outproj_pack_kernel, dim3(static_cast<unsigned>(M)), dim3(kPackThreads), 0,
                     stream, part, ksplit, M, N, y, codes, scales);
  return hipGetLastError();
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

struct GemmCall {
  const uint16_t *A, *W, *W2;
  float* part;
  uint16_t* out_bf16;
  int M, N, K, kchunk, N1;
};

template <int MT, int NT, int PD, bool PACKED, bool PA, bool NTW>
static void launch_gemm_shape(dim3 grid, const GemmCall& c, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_skinny_kernel<MT, NT, PD, PACKED, PA, NTW>), grid, dim3(kGemmWaves * 64), 0,
                     stream, c.A, c.W, c.part, c.out_bf16, c.M, c.N, c.K, c.kchunk, c.W2, c.N1);
}

template <bool PACKED, bool PA, bool NTW>
static void launch_gemm_variant(const GemmCall& c, int ksplit, int ntiles, hipStream_t stream) {
  const int M = c.M;
  if (ntiles == 4) {
    dim3 grid(static_cast<unsigned>(c.N / 64), static_cast<unsigned>(ksplit));
    if (M <= 16) launch_gemm_shape<1, 4, 4, PACKED, PA, NTW>(grid, c, stream);
    else if (M <= 32) launch_gemm_shape<2, 4, 4, PACKED, PA, NTW>(grid, c, stream);
    else if (M <= 64) launch_gemm_shape<4, 4, 3, PACKED, PA, NTW>(grid, c, stream);
    else launch_gemm_shape<8, 4, 2, PACKED, PA, NTW>(grid, c, stream);
  } else if (ntiles == 7) {
    // 112-column tiles: 7168 columns are 64 of them, x 4 K slices = 256 workgroups
    dim3 grid(static_cast<unsigned>(c.N / 112), static_cast<unsigned>(ksplit));
    if (M <= 16) launch_gemm_shape<1, 7, 4, PACKED, PA, NTW>(grid, c, stream);
    else launch_gemm_shape<2, 7, 4, PACKED, PA, NTW>(grid, c, stream);
  } else if (ntiles == 5) {
    dim3 grid(static_cast<unsigned>(c.N / 80), static_cast<unsigned>(ksplit));
    // (64 rows x 80 columns would need more LDS than a CU has for the reduction)
    if (M <= 16) launch_gemm_shape<1, 5, 4, PACKED, PA, NTW>(grid, c, stream);
    else launch_gemm_shape<2, 5, 4, PACKED, PA, NTW>(grid, c, stream);
  } else {
    dim3 grid(static_cast<unsigned>(c.N / 32), static_cast<unsigned>(ksplit));
    if (M <= 16) launch_gemm_shape<1, 2, 8, PACKED, PA, NTW>(grid, c, stream);
    else if (M <= 32) launch_gemm_shape<2, 2, 6, PACKED, PA, NTW>(grid, c, stream);
    else if (M <= 64) launch_gemm_shape<4, 2, 4, PACKED, PA, NTW>(grid, c, stream);
    else launch_gemm_shape<8, 2, 4, PACKED, PA, NTW>(grid, c, stream);
  }
}

int gemm_row_tiles(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : (M <= 64 ? 4 : 8)); }

hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* W, float* part, uint16_t* out_bf16,
                            int M, int N, int K, int ksplit, int ntiles, bool packed, bool a_packed,
                            hipStream_t stream, const uint16_t* W2, int N1, bool stream_w) {
  if (M < 1 || M > 128) return hipErrorInvalidValue;
  if (ntiles != 2 && ntiles != 4 && ntiles != 5 && ntiles != 7) return hipErrorInvalidValue;
  if ((ntiles == 5 || ntiles == 7) && M > 32) return hipErrorInvalidValue;
  if (N % (16 * ntiles)) return hipErrorInvalidValue;
  if (W2 && (N1 <= 0 || N1 >= N || N1 % 16)) return hipErrorInvalidValue;
  const GemmCall c{A, W, W2, part, out_bf16, M, N, K, K / ksplit, W2 ? N1 : N};
  if (a_packed && stream_w) return hipErrorInvalidValue;   // not instantiated
  if (a_packed) {
    if (packed) launch_gemm_variant<true, true, false>(c, ksplit, ntiles, stream);
    else launch_gemm_variant<false, true, false>(c, ksplit, ntiles, stream);
  } else if (stream_w) {
    if (packed) launch_gemm_variant<true, false, true>(c, ksplit, ntiles, stream);
    else launch_gemm_variant<false, false, true>(c, ksplit, ntiles, stream);
  } else {
    if (packed) launch_gemm_variant<true, false, false>(c, ksplit, ntiles, stream);
    else launch_gemm_variant<false, false, false>(c, ksplit, ntiles, stream);
  }
  return hipGetLastError();
}

// Skinny bf16 product for 65 .. 128 rows (packed weights, row-major A):
// part[ks][m][n] = sum over K slice ks of A[m][k] * W[n][k].
//
// The K-split kernel above keeps every wave's full 128 x 64 fp32 tile in
// registers (half the register file at 128 rows), which leaves room for only
// two k-steps of weights in flight per wave. Here the waves split the rows
// instead: wave w owns rows 16w .. 16w+15 over the whole K slice, so its
// accumulators are the NT 16x16 tiles of its own rows (32 registers at
// NT = 8). The weight tile goes through LDS: chunks of CH k-steps (NT*CH KB)
// are loaded by all 512 threads, P chunks in flight in registers, staged into
// one of two LDS buffers and read by every wave; one barrier per chunk. The
// 128-column tile halves the activation reads of a 64-column one (every
// workgroup reads all of its rows of A through L2).
template <int NT, int CH, int P>
struct RowsCfg {
  static constexpr int kUnits = NT * CH;               // 1 KB weight units per chunk
  static constexpr int kPer = kUnits * 64 / 512;       // 16-byte pieces per thread per chunk
  static_assert(kPer * 512 == kUnits * 64, "a chunk splits evenly over 512 threads");
};

template <int I0, int I1, typename F>
__device__ __forceinline__ void rows_static_for(F&& f) {
  if constexpr (I0 < I1) {
    f(std::integral_constant<int, I0>{});
    rows_static_for<I0 + 1, I1>(f);
  }
}

template <int NT, int CH, int P, bool NTW>
__global__ __launch_bounds__(512) void gemm_rows_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ W,
                                                        float* __restrict__ part, int M, int N,
                                                        int K, int kchunk) {
  using C = RowsCfg<NT, CH, P>;
  __shared__ __attribute__((aligned(16))) uint4 wl[2][C::kUnits * 64];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int n0 = blockIdx.x * NT * 16;
  const int ks = blockIdx.y;
  const int kbeg = ks * kchunk;
  const int nchunks = kchunk / (32 * CH);
  // the tile's NT row groups, this K slice: unit (nt, kt) at nt*(K/32) + kt
  // from the first; the resource ends after the last unit the tile reads
  const uint16_t* wbase = W + (static_cast<size_t>(n0 / 16) * (K / 32) + kbeg / 32) * 512;
  const int wbytes = ((NT - 1) * (K / 32) + nchunks * CH) * 1024;
  const auto wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wbase), 0, wbytes,
                                                    0x00020000);
  // piece q = tid + 512 i of a chunk: unit u = q / 64 = (nt = u / CH, kt = u % CH), lane q % 64
  int voff[C::kPer];
#pragma unroll
  for (int i = 0; i < C::kPer; ++i) {
    const int q = tid + 512 * i, u = q >> 6;
    voff[i] = (((u / CH) * (K / 32) + u % CH) * 64 + (q & 63)) * 16;
  }
  const int m = min(16 * w + c, M - 1);            // rows >= M feed only rows >= M of C
  const uint16_t* arow = A + static_cast<size_t>(m) * K + kbeg + g * 8;
  uint4 wreg[P][C::kPer];
  uint4 areg[2][CH];
  f32x4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto issue_w = [&](auto slot_c, int ch) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    // past the end: an offset beyond the resource, which reads nothing (zeros, unused)
    const int co = ch < nchunks ? ch * CH * 1024 : wbytes;
#pragma unroll
    for (int i = 0; i < C::kPer; ++i)
      wreg[slot][i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, voff[i] + co, 0, NTW ? 2 : 0));
  };
  auto issue_a = [&](auto buf_c, int ch) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    const int cc = ch < nchunks ? ch : 0;
#pragma unroll
    for (int kt = 0; kt < CH; ++kt)
      areg[buf][kt] = *reinterpret_cast<const uint4*>(arow + (cc * CH + kt) * 32);
  };
  auto stage = [&](auto slot_c, auto buf_c) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value, buf = decltype(buf_c)::value;
#pragma unroll
    for (int i = 0; i < C::kPer; ++i) wl[buf][tid + 512 * i] = wreg[slot][i];
  };
  auto compute = [&](auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
#pragma unroll
    for (int kt = 0; kt < CH; ++kt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[nt] = mfma_16x16x32(as_bf16x8(areg[buf][kt]), as_bf16x8(wl[buf][(nt * CH + kt) * 64 + lane]),
                                acc[nt]);
  };
  // prologue: chunks 0 .. P-1 in flight, A of chunk 0, chunk 0 staged
  rows_static_for<0, P>([&](auto sc) { issue_w(sc, decltype(sc)::value); });
  issue_a(std::integral_constant<int, 0>{}, 0);
  stage(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
  __syncthreads();
  // chunk ch: refill its register slot with chunk ch+P, load A of ch+1,
  // multiply from LDS buffer ch%2, stage chunk ch+1 into the other buffer
  // (read last in chunk ch-1, before the previous barrier), barrier. Groups
  // of U keep slots and buffers static.
  constexpr int U = (P % 2) ? 2 * P : P;
  for (int base = 0; base < nchunks; base += U) {
    rows_static_for<0, U>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      const int ch = base + r;
      if (ch < nchunks) {
        issue_w(std::integral_constant<int, r % P>{}, ch + P);
        issue_a(std::integral_constant<int, (r + 1) & 1>{}, ch + 1);
        compute(std::integral_constant<int, r & 1>{});
        if (ch + 1 < nchunks)
          stage(std::integral_constant<int, (r + 1) % P>{}, std::integral_constant<int, (r + 1) & 1>{});
        __syncthreads();
      }
    });
  }
  // lane (g, c) of tile nt: rows 16w + 4g + i, column n0 + 16nt + c
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mm = 16 * w + 4 * g + i;
      if (mm < M) part[(static_cast<size_t>(ks) * M + mm) * N + n0 + 16 * nt + c] = acc[nt][i];
    }
}

// 128-column tiles, 4 k-steps per chunk, 3 chunks in flight (measured at
// 128 x 7168 x 16384 with 4 K slices: 56 us against 87 us for the K-split
// kernel with 128-row tiles).
constexpr int kRowsNT = 8, kRowsCH = 4, kRowsP = 3;

hipError_t launch_gemm_rows_bf16(const uint16_t* A, const uint16_t* Wp, float* part, int M, int N,
                                 int K, int ksplit, bool stream_w, hipStream_t stream) {
  if (M <= 64 || M > 128 || N % (16 * kRowsNT) || ksplit < 1 || K % ksplit ||
      (K / ksplit) % (32 * kRowsCH))
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(N / (16 * kRowsNT)), static_cast<unsigned>(ksplit));
  if (stream_w)
    hipLaunchKernelGGL((gemm_rows_kernel<kRowsNT, kRowsCH, kRowsP, true>), grid, dim3(512), 0,
                       stream, A, Wp, part, M, N, K, K / ksplit);
  else
    hipLaunchKernelGGL((gemm_rows_kernel<kRowsNT, kRowsCH, kRowsP, false>), grid, dim3(512), 0,
                       stream, A, Wp, part, M, N, K, K / ksplit);
  return hipGetLastError();
}

int gemm_rows_splits(int N, int K) {
  // fill the 256 compute units once with N/128 column tiles
  const int tiles = N / (16 * kRowsNT);
  int ks = 1;
  while (tiles * ks * 2 <= 256 && K % (ks * 2) == 0 && (K / (ks * 2)) % (32 * kRowsCH) == 0) ks *= 2;
  return ks;
}

// Pack a row-major bf16 weight [N][K] into operand order (see above); one
// thread per 16-byte lane slot.
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint16_t* __restrict__ W,
                                                          uint16_t* __restrict__ P, int N, int K) {
  const int ksteps = K / 32;
  const size_t slots = static_cast<size_t>(N / 16) * ksteps * 64;
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < slots; i += static_cast<size_t>(gridDim.x) * 256) {
    const int lane = static_cast<int>(i & 63);
    const size_t unit = i >> 6;
    const int nt = static_cast<int>(unit / ksteps), kt = static_cast<int>(unit % ksteps);
    const int n = nt * 16 + (lane & 15), k = kt * 32 + (lane >> 4) * 8;
    *reinterpret_cast<uint4*>(P + i * 8) = *reinterpret_cast<const uint4*>(W + static_cast<size_t>(n) * K + k);
  }
}

hipError_t launch_pack_weight(const uint16_t* W, uint16_t* P, int N, int K, hipStream_t stream) {
  const size_t slots = static_cast<size_t>(N / 16) * (K / 32) * 64;
  size_t blocks = (slots + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_weight_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, W, P, N, K);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_reduce(const float* part, int ksplit, const float* g, int M, int R,
                                 float eps, void* out, int out_f32, int out_tiles,
                                 const AppendArgs* append, hipStream_t stream, int part_stride) {
  if (out_tiles && (out_f32 || out_tiles * 16 < M || R % 32)) return hipErrorInvalidValue;
  const int ps = part_stride > 0 ? part_stride : R;
  if (ps < R) return hipErrorInvalidValue;
  if (append) {
    // given tokens: one wave per sequence, at most 16 workgroups; projected
    // tokens (<= 64 rows per pass): one workgroup per sequence
    const int extra = append->kv_part ? append->kv_rows
                                      : ((append->B + 3) / 4 < 16 ? (append->B + 3) / 4 : 16);
    hipLaunchKernelGGL(rmsnorm_reduce_kernel<true>, dim3(static_cast<unsigned>(M + extra)),
                       dim3(256), 0, stream, part, ksplit, g, M, R, ps, eps, out, out_f32,
                       out_tiles, *append);
  } else {
    hipLaunchKernelGGL(rmsnorm_reduce_kernel<false>, dim3(static_cast<unsigned>(M)), dim3(256), 0,
                       stream, part, ksplit, g, M, R, ps, eps, out, out_f32, out_tiles,
                       AppendArgs{});
  }
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
