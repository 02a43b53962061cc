// Launch interfaces of the MFA kernels (internal to libmfa; the public ABI
// is include/mfa.h). Every launcher enqueues on `stream` and returns the
// launch status from hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mfa {

// Equal-work ("balanced") partition of the matrix-core attention: the grid
// is kBalancedWorkgroups workgroups, which split the concatenated 64-token
// blocks of all rows (at most kBalancedMaxRows) evenly; workgroup w writes
// one partial per row it touches, in partial slot w + row.
constexpr int kBalancedWorkgroups = 256;
constexpr int kBalancedMaxRows = 1024;

// Decode attention arguments (shared by the matrix-core and VALU kernels).
struct AttnArgs {
  const uint16_t* q;          // bf16 bits or (VALU kernel, f32 q) reinterpret
  const uint8_t* k;           // cache blocks, bytes
  const uint8_t* v;
  const float* k_scale;       // FP8 only
  const float* v_scale;
  const int* block_table;     // nullable
  const int* seq_lens;
  int max_blocks_per_seq;
  int num_blocks;
  int max_seq_len;
  int chunk_tokens;           // multiple of 64
  int num_splits;
  int heads;                  // VALU kernel only (matrix-core kernel: 64)
  int head_dim;               // VALU kernel only (matrix-core kernel: 256)
  int q_f32;                  // VALU kernel: q dtype
  int kv_f32;                 // VALU kernel: cache dtype (else bf16)
  float sm_scale;             // VALU kernel (natural exp)
  float scale_log2;           // matrix-core kernel: sm_scale * log2(e)
  float* part_o;              // [B][S][H][d] fp32 when num_splits > 1
  float* part_ml;             // [B][S][H][2]
  // balanced partition (num_splits == 0): part_o / part_ml hold
  // kBalancedWorkgroups + B slots; bal_meta[row] = (first slot, slot count)
  int* bal_meta;
  int bal_rows;               // rows of the balanced walk (virtual rows)
  void* out;                  // [B][H][d] when num_splits == 1
  int out_f32;
  // Query tokens per sequence (>= 1). Rows of q, the partials and out are
  // virtual rows r = b * q_len + j (query token j of sequence b); row r reads
  // sequence b's cache (block table row b, seq_lens[b]) and attends to its
  // first seq_lens[b] - (q_len - 1 - j) tokens: causal among the new tokens,
  // which are the last q_len of the sequence.
  int q_len;
  // Matrix-core kernel, FP8 cache: quantize each (row, head) of q to e4m3
  // (scale amax/448) and run Q.K^T on the FP8 matrix cores.
  int fp8_queries;
};


hipError_t launch_decode_valu(const AttnArgs& a, int B, hipStream_t stream);

// meta (nullable): per row (first partial slot, slot count), the balanced
// partition's layout; otherwise row b's partials are slots b*num_splits ..
hipError_t launch_combine(const float* part_o, const float* part_ml, const int* meta, int B,
                          int H, int d, int num_splits, void* out, int out_f32,
                          hipStream_t stream);

struct AppendArgs {
  const void* k_new;          // [B][n_new][d]
  const void* v_new;
  int in_f32;                 // else bf16
  const int* pos;             // [B]
  int n_new;
  int B;
  uint8_t* k;                 // cache
  uint8_t* v;
  float* k_scale;
  float* v_scale;
  const int* block_table;
  int num_blocks;
  int max_blocks_per_seq;
  int d;
  int cache_dtype;            // 0 f32, 1 bf16, 2 fp8
  // K/V projection (decode step only, n_new == 1): when kv_part is set, the
  // token of sequence b (kv_row0 <= b < kv_row0 + kv_rows) is not read from
  // k_new / v_new but summed over kv_ks fp32 partial slices
  //   k[f] = sum_ks kv_part[(ks * kv_rows + b - kv_row0) * kv_stride + kv_col0 + f]
  // (v: columns kv_col0 + d + f), rounded to bf16 when kv_round_bf16, and
  // also written to k_out / v_out ([B][d], the rounded dtype) when set.
  const float* kv_part;
  int kv_ks;
  int kv_rows;
  int kv_row0;
  int kv_stride;
  int kv_col0;
  int kv_round_bf16;
  void* k_out;
  void* v_out;
};

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);

// Matrix-core kernel with the decode step's KV append in the same launch
// (q_len == 1, one token per row, app.n_new == 1, bf16 k_new / v_new, no
// projection): the workgroup that walks a token's block writes the token
// before its waves read that block.
struct AttnAppArgs : AttnArgs {
  AppendArgs app;
};

// B: virtual rows (sequences x q_len). app (nullable): the decode step's KV
// append, done in the same launch.
hipError_t launch_decode_mfma(const AttnArgs& a, bool fp8, int B, hipStream_t stream,
                              const AppendArgs* app = nullptr);

// Query path.
// bf16: C[m][n] = A[M][K] . W[N][K]^T, M <= 128. With ksplit > 1 writes fp32
// partials part[ks][M][N] (K slice ks); with ksplit == 1 and out_bf16 set,
// writes bf16 C directly. ntiles (2, 4, or 5 or 7 with M <= 32) = 16-column tiles
// per workgroup.
// Requires N % (16*ntiles) == 0 and (K/ksplit) % 32 == 0. packed / a_packed:
// W / A in operand order (qproj.hip); a packed A holds gemm_row_tiles(M)
// 16-row tiles per 32-wide k-step.
int gemm_row_tiles(int M);
// W2 (nullable): columns N1 .. N-1 come from W2 (its rows 0 .. N-N1-1)
// instead of W; N1 % 16 == 0. stream_w: non-temporal weight loads (row-major
// A only).
hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* W, float* part, uint16_t* out_bf16,
                            int M, int N, int K, int ksplit, int ntiles, bool packed, bool a_packed,
                            hipStream_t stream, const uint16_t* W2 = nullptr, int N1 = 0,
                            bool stream_w = false);
// Row-major bf16 W [N][K] -> operand-order packed weight (N % 16 == 0, K % 32 == 0).
hipError_t launch_pack_weight(const uint16_t* W, uint16_t* P, int N, int K, hipStream_t stream);
// n[m][j] = bf16(c / sqrt(mean c^2 + eps) * g), c = sum over ksplit partials.
// out_tiles > 0 (bf16 only): n is written as the packed GEMM activation
// operand with out_tiles 16-row tiles; 0: row-major [M][R].
// With append set, the same launch also writes one new KV token per
// sequence (append->n_new == 1, see append_one.h).
// part_stride: row stride of the partials (>= R; R when 0).
hipError_t launch_rmsnorm_reduce(const float* part, int ksplit, const float* g, int M, int R,
                                 float eps, void* out, int out_f32, int out_tiles,
                                 const AppendArgs* append, hipStream_t stream, int part_stride = 0);
// y[m][n] = bf16(sum over ksplit partials) (y nullable); with codes set,
// also the per-row FP8 pack of the bf16 row: scales[m] = amax / 448 (1 when
// 0), codes = RNE e4m3(y / scale). N % 8 == 0, N <= 8192.
hipError_t launch_outproj_pack(const float* part, int ksplit, int M, int N, uint16_t* y,
                               uint8_t* codes, float* scales, hipStream_t stream);
// 65 .. 128 rows, packed weights, row-major A: fp32 partials part[ks][M][N]
// from the row-split kernel (waves own 16-row slices, the weight tile is
// shared through LDS). N % 128 == 0, (K / ksplit) % 128 == 0.
hipError_t launch_gemm_rows_bf16(const uint16_t* A, const uint16_t* Wp, float* part, int M, int N,
                                 int K, int ksplit, bool stream_w, hipStream_t stream);
// its K split for N columns (fills the 256 compute units once)
int gemm_rows_splits(int N, int K);
// out[m][n] = sum over ksplit partials, cast to bf16 or kept f32.
hipError_t launch_reduce_cast(const float* part, int ksplit, int M, int N, void* out,
                              int out_f32, hipStream_t stream);
// f32: out[m][n] = A[m][K] . W[n][K]  (one wave per output).
hipError_t launch_gemv_f32(const float* A, const float* W, float* out, int M, int N, int K,
                           hipStream_t stream);

}  // namespace mfa
