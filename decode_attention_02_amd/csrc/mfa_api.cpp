// libmfa C ABI (include/mfa.h): host-side validation, planning and dispatch.
// Every check runs before any HIP call, so a rejected call touches neither
// the device nor the runtime.
#include "mfa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "kernels.h"

namespace {

constexpr int kBlock = MFA_BLOCK_TOKENS;
constexpr int kMaxQueryTokens = MFA_MAX_QUERY_TOKENS;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

mfa_status from_hip(hipError_t e) { return e == hipSuccess ? MFA_OK : MFA_ERR_HIP; }

// ---- query path planning -------------------------------------------------
constexpr int kRowsPerPass = 64;     // rows per pass of the query path
constexpr int kOutProjRows = 128;    // rows per pass of the output projection (GEMM limit)

struct GemmPlan {
  int ntiles;        // 16-column tiles per workgroup (2, 4, 5 or 7)
  int ks;            // K slices
};

// Wide outputs (>= 512 tiles of 32 columns) run one K slice on 32-column
// tiles; narrower ones use 64-column tiles (80 when that fills the 256
// compute units better: the down-projection with the K/V columns, 2560
// columns, is 32 x 8 workgroups of 80 columns instead of 40 x 4 of 64) and
// halve K while the grid stays within one round of 256 workgroups (one per
// compute unit) and a slice keeps at least 16 k-steps of 32 (two per wave).
// A second, partial round costs more than the compute units one round
// leaves idle: the 7168-column output projection runs 112 x 2 workgroups
// (K slices of 8192) in 43.0 / 49.4 / 63.3 us at 16 / 32 / 64 tokens, and
// 112 x 4 in 48.1 / 52.5 / 66 us.
GemmPlan plan_gemm(int N, int K, int rows) {
  if (N % 32 == 0 && N / 32 >= 512) return GemmPlan{2, 1};
  auto split = [&](int ntiles) {
    GemmPlan p{ntiles, 1};
    const int tiles = N / (16 * ntiles);
    const int steps = K / 32;
    while (static_cast<long long>(tiles) * p.ks * 2 <= 256 && steps % (p.ks * 2) == 0 &&
           steps / (p.ks * 2) >= 16)
      p.ks *= 2;
    return p;
  };
  // fraction of the last round of 256 workgroups that is busy
  auto fill = [&](const GemmPlan& p) {
    const long long wg = static_cast<long long>(N / (16 * p.ntiles)) * p.ks;
    return static_cast<double>(wg) / (256.0 * static_cast<double>((wg + 255) / 256));
  };
  GemmPlan best = split(N % 64 == 0 ? 4 : 2);
  if (N % 80 == 0 && rows <= 32) {      // 80-column tiles hold at most 32 rows
    const GemmPlan p5 = split(5);
    if (fill(p5) > fill(best) + 1e-9) best = p5;
  }
  if (N % 112 == 0 && rows <= 32) {     // so do 112-column tiles
    const GemmPlan p7 = split(7);
    if (fill(p7) > fill(best) + 1e-9) best = p7;
  }
  return best;
}

struct QprojPlan {
  int rows;          // rows per pass
  GemmPlan down, down_kv, up;   // down_kv: down-projection with the K/V columns appended
  size_t off_part_down, off_n, off_part_up, off_kv, total;
};

// kvc: K/V projection columns (2d) the workspace must also hold.
QprojPlan plan_qproj(int B, int hidden, int q_rank, int HD, int dtype, int kvc) {
  QprojPlan p{};
  p.rows = B < kRowsPerPass ? B : kRowsPerPass;
  if (dtype == MFA_BF16) {
    p.down = plan_gemm(q_rank, hidden, p.rows);
    p.down_kv = plan_gemm(q_rank + kvc, hidden, p.rows);
    p.up = plan_gemm(HD, q_rank, p.rows);
    p.off_part_down = 0;
    const size_t part_q = static_cast<size_t>(p.down.ks) * p.rows * q_rank * 4;
    const size_t part_kv = static_cast<size_t>(p.down_kv.ks) * p.rows * (q_rank + kvc) * 4;
    p.off_n = round_up(part_q > part_kv ? part_q : part_kv, 256);
    // n is the up-projection's packed activation operand: whole 16-row tiles
    p.off_part_up = p.off_n + round_up(static_cast<size_t>(16 * mfa::gemm_row_tiles(p.rows)) *
                                           q_rank * 2, 256);
    p.total = p.off_part_up +
              (p.up.ks > 1 ? round_up(static_cast<size_t>(p.up.ks) * p.rows * HD * 4, 256) : 0);
    p.off_kv = 0;      // the K/V columns live in the down-projection's partials
  } else {
    p.down = p.down_kv = p.up = GemmPlan{0, 1};
    p.off_part_down = 0;
    p.off_n = round_up(static_cast<size_t>(p.rows) * q_rank * 4, 256);
    p.off_part_up = p.off_n + round_up(static_cast<size_t>(p.rows) * q_rank * 4, 256);
    p.off_kv = p.off_part_up;                 // [rows][kvc] fp32 K/V projection
    p.total = p.off_kv + round_up(static_cast<size_t>(p.rows) * kvc * 4, 256);
  }
  return p;
}

mfa_status check_qproj_shape(int B, int hidden, int q_rank, int H, int d, int dtype) {
  if (dtype != MFA_BF16 && dtype != MFA_F32) return MFA_ERR_DTYPE;
  if (B < 1 || B > 256 || hidden < 1 || q_rank < 1 || H < 1 || d < 1) return MFA_ERR_SHAPE;
  if (q_rank > 8192) return MFA_ERR_SHAPE;
  const long long hd = static_cast<long long>(H) * d;
  if (hd > (1 << 24)) return MFA_ERR_SHAPE;
  if (dtype == MFA_BF16) {
    if (hidden % 256 || q_rank % 256 || hd % 64) return MFA_ERR_SHAPE;
  } else {
    if (hidden % 4 || q_rank % 8 || hd % 4) return MFA_ERR_SHAPE;
  }
  return MFA_OK;
}

// ---- attention planning --------------------------------------------------
// Split workspace: part_o fp32 [rows][d] (rows = partial slots x heads) at
// 0, part_ml fp32 [rows][2] at off_ml; for the balanced partition also the
// per-row metadata int32 [B][2] at off_meta.
struct SplitLayout {
  size_t off_ml, off_meta, total;
};
SplitLayout split_layout(size_t rows, int d, size_t meta_rows = 0) {
  SplitLayout l;
  l.off_ml = round_up(rows * static_cast<size_t>(d) * 4, 256);
  l.off_meta = round_up(l.off_ml + rows * 2 * 4, 16);
  l.total = meta_rows ? l.off_meta + meta_rows * 8 : l.off_ml + rows * 2 * 4;
  return l;
}
// Splits walked as two halves each: when B * num_splits workgroups would
// leave at least half of the 256 compute units idle (and the XCD remap's
// multiple of 8 holds), every split runs as two workgroups of 64 heads over
// half its tokens (two partials per split) instead of one per split. Two
// head groups reading the same blocks were the earlier answer; the halves
// read every byte once and were faster (64K workload: 48.7 against 52.0 us).
bool halves(long long B, int num_splits) {
  return num_splits > 1 && B * num_splits * 2 <= mfa::kBalancedWorkgroups &&
         (B * num_splits) % 8 == 0;
}
int effective_splits(long long B, int num_splits) {
  return halves(B, num_splits) ? 2 * num_splits : num_splits;
}
// The workspace of B rows and num_splits (0: balanced partition).
SplitLayout workspace_layout(int B, int H, int d, int num_splits) {
  if (num_splits == 0)
    return split_layout(static_cast<size_t>(mfa::kBalancedWorkgroups + B) * H, d,
                        static_cast<size_t>(B));
  return split_layout(static_cast<size_t>(B) * effective_splits(B, num_splits) * H, d);
}

bool mfma_shape(int H, int d, int kv_dtype) {
  return H == 64 && d == 256 && (kv_dtype == MFA_BF16 || kv_dtype == MFA_FP8_E4M3);
}

bool valu_shape(int H, int d, int kv_dtype) {
  return (kv_dtype == MFA_F32 || kv_dtype == MFA_BF16) && H >= 1 && H <= 64 &&
         (d == 64 || d == 128 || d == 256) && H * d <= 8192;
}

mfa_status check_cache(const mfa_kv_cache* c) {
  if (!c) return MFA_ERR_NULL;
  if (!c->k || !c->v) return MFA_ERR_NULL;
  if (!aligned16(c->k) || !aligned16(c->v)) return MFA_ERR_ALIGN;
  if (c->dtype != MFA_F32 && c->dtype != MFA_BF16 && c->dtype != MFA_FP8_E4M3) return MFA_ERR_DTYPE;
  if (c->dtype == MFA_FP8_E4M3) {
    if (!c->k_scale || !c->v_scale) return MFA_ERR_NULL;
    if (!aligned16(c->k_scale) || !aligned16(c->v_scale)) return MFA_ERR_ALIGN;
  }
  if (c->num_blocks < 1 || c->max_blocks_per_seq < 1) return MFA_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return MFA_ERR_SHAPE;
  if (c->block_table && !aligned4(c->block_table)) return MFA_ERR_ALIGN;
  if (static_cast<long long>(c->max_blocks_per_seq) * kBlock > (1ll << 30)) return MFA_ERR_SHAPE;
  return MFA_OK;
}

}  // namespace

extern "C" {

int mfa_abi_version(void) { return MFA_ABI_VERSION; }

const char* mfa_status_str(int s) {
  switch (s) {
    case MFA_OK: return "ok";
    case MFA_ERR_NULL: return "required pointer is NULL";
    case MFA_ERR_SHAPE: return "size out of range or inconsistent";
    case MFA_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case MFA_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MFA_ERR_UNSUPPORTED: return "the library has no kernel for this shape";
    case MFA_ERR_WORKSPACE: return "workspace missing or too small";
    case MFA_ERR_HIP: return "HIP runtime reported a launch failure";
    case MFA_ERR_TOO_LARGE: return "request needs more than the library's static scratch";
    default: return "unknown status";
  }
}

size_t mfa_qproj_workspace_bytes(int B, int hidden, int q_rank, int H, int d, int dtype) {
  if (check_qproj_shape(B, hidden, q_rank, H, d, dtype) != MFA_OK) return 0;
  return plan_qproj(B, hidden, q_rank, H * d, dtype, 2 * d).total;
}

// ---- attention output projection ----------------------------------------
namespace {
struct OutProjPlan {
  int rows;
  GemmPlan g;          // K-split kernel (passes of up to 64 rows, row-major weights)
  int rows_ks;         // row-split kernel's K slices for passes of 65 .. 128 rows (0: not used)
  size_t total;
};
OutProjPlan plan_out_proj(int B, int HD, int hidden) {
  OutProjPlan p{};
  p.rows = B < kOutProjRows ? B : kOutProjRows;
  p.g = plan_gemm(hidden, HD, p.rows);
  p.rows_ks = (B > 64 && hidden % 128 == 0) ? mfa::gemm_rows_splits(hidden, HD) : 0;
  const int ks = p.g.ks > p.rows_ks ? p.g.ks : p.rows_ks;
  p.total = round_up(static_cast<size_t>(ks) * p.rows * hidden * 4, 256);
  return p;
}
mfa_status check_out_proj_shape(int B, int HD, int hidden, int dtype) {
  if (dtype != MFA_BF16) return MFA_ERR_DTYPE;
  if (B < 1 || B > 256 || HD < 256 || hidden < 64) return MFA_ERR_SHAPE;
  if (HD % 256 || hidden % 64 || hidden > 8192) return MFA_ERR_SHAPE;
  return MFA_OK;
}
}  // namespace

size_t mfa_out_proj_workspace_bytes(int B, int HD, int hidden, int dtype) {
  if (check_out_proj_shape(B, HD, hidden, dtype) != MFA_OK) return 0;
  return plan_out_proj(B, HD, hidden).total;
}

mfa_status mfa_out_proj(const void* o, const void* w_o, int weight_layout, int B, int HD,
                        int hidden, int dtype, void* workspace, size_t workspace_bytes, void* y,
                        void* codes, float* scales, void* stream) {
  if (!o || !w_o) return MFA_ERR_NULL;
  if (!y && !codes) return MFA_ERR_NULL;                 // nothing to write
  if ((codes == nullptr) != (scales == nullptr)) return MFA_ERR_NULL;
  const mfa_status sh = check_out_proj_shape(B, HD, hidden, dtype);
  if (sh != MFA_OK) return sh;
  if (weight_layout != MFA_WEIGHTS_ROWMAJOR && weight_layout != MFA_WEIGHTS_PACKED)
    return MFA_ERR_SHAPE;
  if (!aligned16(o) || !aligned16(w_o) || (y && !aligned16(y)) || (codes && !aligned16(codes)) ||
      (scales && !aligned4(scales)) || (workspace && !aligned16(workspace)))
    return MFA_ERR_ALIGN;
  const OutProjPlan p = plan_out_proj(B, HD, hidden);
  if (!workspace || workspace_bytes < p.total) return MFA_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  float* part = static_cast<float*>(workspace);
  for (int r0 = 0; r0 < B; r0 += p.rows) {
    const int M = (B - r0) < p.rows ? (B - r0) : p.rows;
    const uint16_t* oa = static_cast<const uint16_t*>(o) + static_cast<size_t>(r0) * HD;
    // 65 .. 128 rows with packed weights: the row-split kernel
    const bool rows = M > 64 && p.rows_ks > 0 && weight_layout == MFA_WEIGHTS_PACKED;
    const int ks = rows ? p.rows_ks : p.g.ks;
    hipError_t e =
        rows ? mfa::launch_gemm_rows_bf16(oa, static_cast<const uint16_t*>(w_o), part, M, hidden,
                                          HD, ks, true, st)
             : mfa::launch_gemm_bf16(oa, static_cast<const uint16_t*>(w_o), part, nullptr, M,
                                     hidden, HD, ks, p.g.ntiles,
                                     weight_layout == MFA_WEIGHTS_PACKED, false, st, nullptr, 0,
                                     true);
    if (e != hipSuccess) return MFA_ERR_HIP;
    e = mfa::launch_outproj_pack(
        part, ks, M, hidden, y ? static_cast<uint16_t*>(y) + static_cast<size_t>(r0) * hidden : nullptr,
        codes ? static_cast<uint8_t*>(codes) + static_cast<size_t>(r0) * hidden : nullptr,
        scales ? scales + r0 : nullptr, st);
    if (e != hipSuccess) return MFA_ERR_HIP;
  }
  return MFA_OK;
}

mfa_status mfa_pack_weight(const void* w, void* packed, int N, int K, int dtype, void* stream) {
  if (!w || !packed) return MFA_ERR_NULL;
  if (dtype != MFA_BF16) return MFA_ERR_DTYPE;
  if (N < 16 || K < 32 || N % 16 || K % 32) return MFA_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(packed)) return MFA_ERR_ALIGN;
  return from_hip(mfa::launch_pack_weight(static_cast<const uint16_t*>(w),
                                          static_cast<uint16_t*>(packed), N, K, as_stream(stream)));
}

}  // extern "C"

namespace {

// A validated query-path call.
struct QprojCall {
  const void *x, *w_qdown, *w_qup;
  const float* q_norm_w;
  void* q_out;
  uint8_t* ws;
  int B, hidden, q_rank, HD, dtype;
  bool packed;
  float eps;
  QprojPlan p;
  const void* w_kv;  // K/V projection weights [kvc][hidden] or nullptr
  int kvc;           // 2d with w_kv, else 0
};

mfa_status prepare_qproj(const void* x, const void* w_qdown, const float* q_norm_w,
                         const void* w_qup, void* q_out, void* workspace, size_t workspace_bytes,
                         int B, int hidden, int q_rank, int H, int d, float eps, int dtype,
                         int weight_layout, QprojCall* c) {
  if (!x || !w_qdown || !q_norm_w || !w_qup || !q_out) return MFA_ERR_NULL;
  const mfa_status sh = check_qproj_shape(B, hidden, q_rank, H, d, dtype);
  if (sh != MFA_OK) return sh;
  if (weight_layout != MFA_WEIGHTS_ROWMAJOR && weight_layout != MFA_WEIGHTS_PACKED)
    return MFA_ERR_SHAPE;
  if (weight_layout == MFA_WEIGHTS_PACKED && dtype != MFA_BF16) return MFA_ERR_DTYPE;
  if (!aligned16(x) || !aligned16(w_qdown) || !aligned16(q_norm_w) || !aligned16(w_qup) ||
      !aligned16(q_out) || (workspace && !aligned16(workspace)))
    return MFA_ERR_ALIGN;
  if (!(eps >= 0.f)) return MFA_ERR_SHAPE;
  c->p = plan_qproj(B, hidden, q_rank, H * d, dtype, 2 * d);
  if (!workspace) return MFA_ERR_WORKSPACE;
  if (workspace_bytes < c->p.total) return MFA_ERR_WORKSPACE;
  c->x = x;
  c->w_qdown = w_qdown;
  c->w_qup = w_qup;
  c->q_norm_w = q_norm_w;
  c->q_out = q_out;
  c->ws = static_cast<uint8_t*>(workspace);
  c->B = B;
  c->hidden = hidden;
  c->q_rank = q_rank;
  c->HD = H * d;
  c->dtype = dtype;
  c->packed = weight_layout == MFA_WEIGHTS_PACKED;
  c->eps = eps;
  c->w_kv = nullptr;
  c->kvc = 0;
  return MFA_OK;
}

// Enqueues the query path; a single-token KV append (append != nullptr)
// rides in the first RMSNorm launch. With the K/V projection (c.w_kv), the
// K/V columns ride in each pass's down-projection and every pass appends
// its own rows from their partials.
mfa_status launch_qproj(const QprojCall& c, const mfa::AppendArgs* append, hipStream_t st) {
  const QprojPlan& p = c.p;
  const size_t esz = c.dtype == MFA_BF16 ? 2 : 4;
  const bool proj = c.w_kv != nullptr;
  for (int r0 = 0; r0 < c.B; r0 += p.rows) {
    const int M = (c.B - r0) < p.rows ? (c.B - r0) : p.rows;
    const uint8_t* xa = static_cast<const uint8_t*>(c.x) + static_cast<size_t>(r0) * c.hidden * esz;
    uint8_t* qo = static_cast<uint8_t*>(c.q_out) + static_cast<size_t>(r0) * c.HD * esz;
    hipError_t e;
    mfa::AppendArgs ap{};
    const mfa::AppendArgs* app = r0 == 0 ? append : nullptr;
    if (proj) {
      ap = *append;
      ap.kv_rows = M;
      ap.kv_row0 = r0;
      ap.kv_round_bf16 = c.dtype == MFA_BF16;
      app = &ap;
    }
    if (c.dtype == MFA_BF16) {
      float* pd = reinterpret_cast<float*>(c.ws + p.off_part_down);
      uint16_t* n = reinterpret_cast<uint16_t*>(c.ws + p.off_n);
      const GemmPlan& dp = proj ? p.down_kv : p.down;
      const int N = c.q_rank + c.kvc;
      e = mfa::launch_gemm_bf16(reinterpret_cast<const uint16_t*>(xa),
                                static_cast<const uint16_t*>(c.w_qdown), pd, nullptr, M, N,
                                c.hidden, dp.ks, dp.ntiles, c.packed, false, st,
                                static_cast<const uint16_t*>(c.w_kv), c.q_rank, true);
      if (e != hipSuccess) return MFA_ERR_HIP;
      if (proj) {
        ap.kv_part = pd;
        ap.kv_ks = dp.ks;
        ap.kv_stride = N;
        ap.kv_col0 = c.q_rank;
      }
      e = mfa::launch_rmsnorm_reduce(pd, dp.ks, c.q_norm_w, M, c.q_rank, c.eps, n, 0,
                                     mfa::gemm_row_tiles(M), app, st, N);
      if (e != hipSuccess) return MFA_ERR_HIP;
      if (p.up.ks == 1) {
        e = mfa::launch_gemm_bf16(n, static_cast<const uint16_t*>(c.w_qup), nullptr,
                                  reinterpret_cast<uint16_t*>(qo), M, c.HD, c.q_rank, 1,
                                  p.up.ntiles, c.packed, true, st);
      } else {
        float* pu = reinterpret_cast<float*>(c.ws + p.off_part_up);
        e = mfa::launch_gemm_bf16(n, static_cast<const uint16_t*>(c.w_qup), pu, nullptr, M, c.HD,
                                  c.q_rank, p.up.ks, p.up.ntiles, c.packed, true, st);
        if (e != hipSuccess) return MFA_ERR_HIP;
        e = mfa::launch_reduce_cast(pu, p.up.ks, M, c.HD, qo, 0, st);
      }
      if (e != hipSuccess) return MFA_ERR_HIP;
    } else {
      float* cc = reinterpret_cast<float*>(c.ws + p.off_part_down);
      float* n = reinterpret_cast<float*>(c.ws + p.off_n);
      e = mfa::launch_gemv_f32(reinterpret_cast<const float*>(xa),
                               static_cast<const float*>(c.w_qdown), cc, M, c.q_rank, c.hidden, st);
      if (e != hipSuccess) return MFA_ERR_HIP;
      if (proj) {
        float* kv = reinterpret_cast<float*>(c.ws + p.off_kv);
        e = mfa::launch_gemv_f32(reinterpret_cast<const float*>(xa),
                                 static_cast<const float*>(c.w_kv), kv, M, c.kvc, c.hidden, st);
        if (e != hipSuccess) return MFA_ERR_HIP;
        ap.kv_part = kv;
        ap.kv_ks = 1;
        ap.kv_stride = c.kvc;
        ap.kv_col0 = 0;
      }
      e = mfa::launch_rmsnorm_reduce(cc, 1, c.q_norm_w, M, c.q_rank, c.eps, n, 1, 0, app, st);
      if (e != hipSuccess) return MFA_ERR_HIP;
      e = mfa::launch_gemv_f32(n, static_cast<const float*>(c.w_qup), reinterpret_cast<float*>(qo),
                               M, c.HD, c.q_rank, st);
      if (e != hipSuccess) return MFA_ERR_HIP;
    }
  }
  return MFA_OK;
}

// projected: the token comes from the K/V projection (k_new, v_new are then
// optional outputs).
mfa_status prepare_append(const void* k_new, const void* v_new, int in_dtype, const int32_t* pos,
                          int n_new, int B, const mfa_kv_cache* cache, mfa::AppendArgs* a,
                          bool projected = false) {
  if (!pos) return MFA_ERR_NULL;
  if (!projected && (!k_new || !v_new)) return MFA_ERR_NULL;
  const mfa_status cs = check_cache(cache);
  if (cs != MFA_OK) return cs;
  if ((k_new && !aligned16(k_new)) || (v_new && !aligned16(v_new)) || !aligned4(pos))
    return MFA_ERR_ALIGN;
  if (B < 1 || n_new < 1) return MFA_ERR_SHAPE;
  if (static_cast<long long>(n_new) > static_cast<long long>(cache->max_blocks_per_seq) * kBlock)
    return MFA_ERR_SHAPE;
  if (in_dtype != MFA_F32 && in_dtype != MFA_BF16) return MFA_ERR_DTYPE;
  if (cache->dtype != MFA_FP8_E4M3 && cache->dtype != in_dtype) return MFA_ERR_DTYPE;
  if (!cache->block_table &&
      static_cast<long long>(B) * cache->max_blocks_per_seq > cache->num_blocks)
    return MFA_ERR_SHAPE;
  *a = mfa::AppendArgs{};
  a->k_new = k_new;
  a->v_new = v_new;
  a->in_f32 = in_dtype == MFA_F32;
  a->pos = pos;
  a->n_new = n_new;
  a->B = B;
  a->k = static_cast<uint8_t*>(cache->k);
  a->v = static_cast<uint8_t*>(cache->v);
  a->k_scale = cache->k_scale;
  a->v_scale = cache->v_scale;
  a->block_table = cache->block_table;
  a->num_blocks = cache->num_blocks;
  a->max_blocks_per_seq = cache->max_blocks_per_seq;
  a->d = cache->head_dim;
  a->cache_dtype = cache->dtype == MFA_F32 ? 0 : (cache->dtype == MFA_BF16 ? 1 : 2);
  if (projected) {
    a->k_new = a->v_new = nullptr;
    a->k_out = const_cast<void*>(k_new);
    a->v_out = const_cast<void*>(v_new);
  }
  return MFA_OK;
}

}  // namespace

extern "C" {

mfa_status mfa_qproj(const void* x, const void* w_qdown, const float* q_norm_w, const void* w_qup,
                     void* q_out, void* workspace, size_t workspace_bytes, int B, int hidden,
                     int q_rank, int H, int d, float eps, int dtype, int weight_layout,
                     void* stream) {
  QprojCall c{};
  const mfa_status st = prepare_qproj(x, w_qdown, q_norm_w, w_qup, q_out, workspace,
                                      workspace_bytes, B, hidden, q_rank, H, d, eps, dtype,
                                      weight_layout, &c);
  if (st != MFA_OK) return st;
  return launch_qproj(c, nullptr, as_stream(stream));
}

mfa_status mfa_kv_append(const void* k_new, const void* v_new, int in_dtype, const int32_t* pos,
                         int n_new, int B, const mfa_kv_cache* cache, void* stream) {
  mfa::AppendArgs a;
  const mfa_status st = prepare_append(k_new, v_new, in_dtype, pos, n_new, B, cache, &a);
  if (st != MFA_OK) return st;
  return from_hip(mfa::launch_kv_append(a, as_stream(stream)));
}

mfa_status mfa_decode_plan(int B, int H, int d, int max_seq_len, int kv_dtype, int* num_splits,
                           int* chunk_tokens) {
  if (!num_splits || !chunk_tokens) return MFA_ERR_NULL;
  if (B < 1 || H < 1 || d < 1 || max_seq_len < 0) return MFA_ERR_SHAPE;
  const int blocks = (max_seq_len + kBlock - 1) / kBlock;
  // One 8-wave attention workgroup per compute unit of an MI355X (256 CUs):
  // split each sequence so that the grid covers the chip once, with splits
  // of whole 128-token tiles (two cache blocks) for the matrix-core kernel
  // and of single blocks for the vector kernel (whose workgroups walk their
  // tokens 16 or 32 at a time: a short sequence is better spread out).
  const int gran = mfma_shape(H, d, kv_dtype) ? 2 : 1;
  constexpr int kTargetWorkgroups = 256;
  int splits = kTargetWorkgroups / B;
  if (splits < 1) splits = 1;
  if (splits > blocks / gran) splits = blocks / gran > 0 ? blocks / gran : 1;
  int per = blocks > 0 ? (blocks + splits - 1) / splits : gran;
  per = (per + gran - 1) / gran * gran;
  splits = blocks > 0 ? (blocks + per - 1) / per : 1;
  *num_splits = splits;
  *chunk_tokens = per * kBlock;
  return MFA_OK;
}

mfa_status mfa_decode_plan_lens(int B, int H, int d, const int32_t* seq_lens, int kv_dtype,
                                int* num_splits, int* chunk_tokens) {
  if (!num_splits || !chunk_tokens || !seq_lens) return MFA_ERR_NULL;
  if (B < 1 || H < 1 || d < 1) return MFA_ERR_SHAPE;
  int max_len = 0;
  long long total = 0;
  for (int b = 0; b < B; ++b) {
    if (seq_lens[b] < 0) return MFA_ERR_SHAPE;
    max_len = seq_lens[b] > max_len ? seq_lens[b] : max_len;
    total += (seq_lens[b] + kBlock - 1) / kBlock;
  }
  const mfa_status st = mfa_decode_plan(B, H, d, max_len, kv_dtype, num_splits, chunk_tokens);
  if (st != MFA_OK) return st;
  if (!mfma_shape(H, d, kv_dtype) || B > mfa::kBalancedMaxRows || total == 0 ||
      static_cast<long long>(B) * ((max_len + kBlock - 1) / kBlock) > (1ll << 21))
    return MFA_OK;
  // longest split workgroup of the plan (in blocks); with more workgroups
  // than compute units, at least the chip's share
  const int per = *chunk_tokens / kBlock;
  long long longest = 0;
  for (int b = 0; b < B; ++b) {
    const long long nb = (seq_lens[b] + kBlock - 1) / kBlock;
    longest = nb < per ? (nb > longest ? nb : longest) : (per > longest ? per : longest);
  }
  constexpr int kUnits = mfa::kBalancedWorkgroups;
  const long long wgs = static_cast<long long>(B) * *num_splits;
  const double split_ms = wgs <= kUnits ? static_cast<double>(longest)
                                        : static_cast<double>((total + kUnits - 1) / kUnits) + 0.5 * longest;
  const double bal_ms = static_cast<double>((total + kUnits - 1) / kUnits);
  const double margin = kv_dtype == MFA_FP8_E4M3 ? 1.15 : 1.05;
  if (split_ms > margin * bal_ms + 1.0) {
    *num_splits = MFA_SPLITS_BALANCED;
    *chunk_tokens = 0;
  }
  return MFA_OK;
}

size_t mfa_decode_workspace_bytes(int B, int H, int d, int num_splits) {
  if (B < 1 || H < 1 || d < 1 || num_splits == 1 || num_splits < 0) return 0;
  if (num_splits == 0 && B > mfa::kBalancedMaxRows) return 0;
  return workspace_layout(B, H, d, num_splits).total;
}

size_t mfa_split_workspace_bytes(int B, int H, int d, int num_splits) {
  return mfa_decode_workspace_bytes(B, H, d, num_splits);
}

}  // extern "C"

namespace {

struct AttnCall {
  mfa::AttnArgs a;
  bool mfma, fp8;
  int B, H, d, num_splits;
  void* out;
};

// q_len query tokens per sequence: the rows of q, the partials and out are
// the B * q_len virtual rows (sequence, query token).
mfa_status prepare_attn(const void* q, int q_dtype, int B, int H, const mfa_kv_cache* cache,
                        const int32_t* seq_lens, int max_seq_len, float sm_scale, int num_splits,
                        int chunk_tokens, void* workspace, size_t workspace_bytes, void* out,
                        int out_dtype, AttnCall* c, int q_len = 1, bool fp8_queries = false) {
  if (!q || !seq_lens) return MFA_ERR_NULL;
  const mfa_status cs = check_cache(cache);
  if (cs != MFA_OK) return cs;
  if (!aligned16(q) || !aligned4(seq_lens) || (out && !aligned16(out)) ||
      (workspace && !aligned16(workspace)))
    return MFA_ERR_ALIGN;
  const int d = cache->head_dim;
  if (B < 1 || H < 1 || max_seq_len < 0) return MFA_ERR_SHAPE;
  if (q_len < 1 || q_len > kMaxQueryTokens) return MFA_ERR_SHAPE;
  if (static_cast<long long>(B) * q_len > 0x7fffffffll / 64) return MFA_ERR_SHAPE;
  const int Bv = B * q_len;                       // virtual rows
  if (static_cast<long long>(max_seq_len) > static_cast<long long>(cache->max_blocks_per_seq) * kBlock)
    return MFA_ERR_SHAPE;
  if (!cache->block_table &&
      static_cast<long long>(B) * cache->max_blocks_per_seq > cache->num_blocks)
    return MFA_ERR_SHAPE;
  const bool balanced = num_splits == 0;
  if (balanced) {
    if (Bv > mfa::kBalancedMaxRows) return MFA_ERR_SHAPE;
    // the partition's cost arithmetic is 32-bit: at most 2^21 blocks in all
    if (static_cast<long long>(Bv) * ((max_seq_len + kBlock - 1) / kBlock) > (1ll << 21))
      return MFA_ERR_SHAPE;
  } else {
    if (num_splits < 1 || chunk_tokens < kBlock || chunk_tokens % kBlock) return MFA_ERR_SHAPE;
    if (static_cast<long long>(num_splits) * chunk_tokens < max_seq_len) return MFA_ERR_SHAPE;
  }
  if (static_cast<long long>(Bv) * num_splits > 0x7fffffffll / 64) return MFA_ERR_SHAPE;
  if (out_dtype != MFA_BF16 && out_dtype != MFA_F32) return MFA_ERR_DTYPE;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return MFA_ERR_SHAPE;
  c->mfma = mfma_shape(H, d, cache->dtype);
  if (fp8_queries && !(c->mfma && cache->dtype == MFA_FP8_E4M3)) return MFA_ERR_UNSUPPORTED;
  if (balanced && (!c->mfma || fp8_queries)) return MFA_ERR_UNSUPPORTED;
  if (c->mfma) {
    if (q_dtype != MFA_BF16) return MFA_ERR_DTYPE;
  } else if (valu_shape(H, d, cache->dtype)) {
    if (q_dtype != MFA_BF16 && q_dtype != MFA_F32) return MFA_ERR_DTYPE;
  } else {
    return MFA_ERR_UNSUPPORTED;
  }
  if (num_splits == 1) {
    if (!out) return MFA_ERR_NULL;
  } else {
    if (!workspace) return MFA_ERR_WORKSPACE;
    if (workspace_bytes < mfa_decode_workspace_bytes(Bv, H, d, num_splits)) return MFA_ERR_WORKSPACE;
  }

  mfa::AttnArgs& a = c->a;
  a = mfa::AttnArgs{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint8_t*>(cache->k);
  a.v = static_cast<const uint8_t*>(cache->v);
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.block_table = cache->block_table;
  a.seq_lens = seq_lens;
  a.max_blocks_per_seq = cache->max_blocks_per_seq;
  a.num_blocks = cache->num_blocks;
  a.max_seq_len = max_seq_len;
  a.chunk_tokens = chunk_tokens;
  a.num_splits = num_splits;
  if (halves(Bv, num_splits)) {      // two half-splits per split, 64 heads each
    a.num_splits = 2 * num_splits;
    a.chunk_tokens = (chunk_tokens / kBlock + 1) / 2 * kBlock;
  }
  a.heads = H;
  a.head_dim = d;
  a.q_f32 = q_dtype == MFA_F32;
  a.kv_f32 = cache->dtype == MFA_F32;
  a.sm_scale = sm_scale;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.q_len = q_len;
  a.fp8_queries = fp8_queries ? 1 : 0;
  if (num_splits != 1) {
    const SplitLayout l = workspace_layout(Bv, H, d, num_splits);
    a.part_o = static_cast<float*>(workspace);
    a.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + l.off_ml);
    if (balanced) a.bal_meta = reinterpret_cast<int*>(static_cast<uint8_t*>(workspace) + l.off_meta);
  }
  a.bal_rows = Bv;
  a.out = out;
  a.out_f32 = out_dtype == MFA_F32;
  c->fp8 = cache->dtype == MFA_FP8_E4M3;
  c->B = Bv;
  c->H = H;
  c->d = d;
  c->num_splits = a.num_splits;
  c->out = out;
  return MFA_OK;
}

// app (nullable, matrix-core kernel only): the decode step's KV append,
// done inside the attention launch.
mfa_status launch_attn(const AttnCall& c, hipStream_t st, const mfa::AppendArgs* app = nullptr) {
  const mfa::AttnArgs& a = c.a;
  hipError_t e = c.mfma ? mfa::launch_decode_mfma(a, c.fp8, c.B, st, app) : mfa::launch_decode_valu(a, c.B, st);
  if (e != hipSuccess) return MFA_ERR_HIP;
  if (c.num_splits != 1 && c.out) {
    e = mfa::launch_combine(a.part_o, a.part_ml, a.bal_meta, c.B, c.H, c.d, c.num_splits, c.out,
                            a.out_f32, st);
    if (e != hipSuccess) return MFA_ERR_HIP;
  }
  return MFA_OK;
}

}  // namespace

extern "C" {

mfa_status mfa_decode_attn(const void* q, int q_dtype, int B, int H, const mfa_kv_cache* cache,
                           const int32_t* seq_lens, int max_seq_len, float sm_scale,
                           int num_splits, int chunk_tokens, void* workspace,
                           size_t workspace_bytes, void* out, int out_dtype, void* stream) {
  AttnCall c;
  const mfa_status st = prepare_attn(q, q_dtype, B, H, cache, seq_lens, max_seq_len, sm_scale,
                                     num_splits, chunk_tokens, workspace, workspace_bytes, out,
                                     out_dtype, &c);
  if (st != MFA_OK) return st;
  return launch_attn(c, as_stream(stream));
}

}  // extern "C"

namespace {

// The split partials of mfa_decode_attn_static. In host code `scratch` only
// names the symbol; its device address (one per GPU) comes from
// hipGetSymbolAddress and is what the kernels are given.
static __device__ __align__(256) unsigned char scratch[MFA_STATIC_SCRATCH];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up once per device).
mfa_status scratch_for_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MFA_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MFA_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return MFA_OK;
}

}  // namespace

extern "C" {

mfa_status mfa_decode_attn_static(const void* q, int q_dtype, int B, int H,
                                  const mfa_kv_cache* cache, const int32_t* seq_lens,
                                  int max_seq_len, float sm_scale, int num_splits,
                                  int chunk_tokens, void* out, int out_dtype, void* stream) {
  if (!out) return MFA_ERR_NULL;
  if (cache && (num_splits == 0 || num_splits > 1) && B > 0 && H > 0 &&
      mfa_decode_workspace_bytes(B, H, cache->head_dim, num_splits) > MFA_STATIC_SCRATCH)
    return MFA_ERR_TOO_LARGE;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (num_splits == 0 || num_splits > 1) {
    const mfa_status ss = scratch_for_current_device(&ws);
    if (ss != MFA_OK) return ss;
    ws_bytes = MFA_STATIC_SCRATCH;
  }
  AttnCall c;
  const mfa_status st = prepare_attn(q, q_dtype, B, H, cache, seq_lens, max_seq_len, sm_scale,
                                     num_splits, chunk_tokens, ws, ws_bytes, out, out_dtype, &c);
  if (st != MFA_OK) return st;
  return launch_attn(c, as_stream(stream));
}

mfa_status mfa_decode_attn_multi(const void* q, int q_dtype, int B, int q_len, int H,
                                 const mfa_kv_cache* cache, const int32_t* seq_lens,
                                 int max_seq_len, float sm_scale, int num_splits, int chunk_tokens,
                                 void* workspace, size_t workspace_bytes, void* out, int out_dtype,
                                 void* stream) {
  AttnCall c;
  const mfa_status st = prepare_attn(q, q_dtype, B, H, cache, seq_lens, max_seq_len, sm_scale,
                                     num_splits, chunk_tokens, workspace, workspace_bytes, out,
                                     out_dtype, &c, q_len);
  if (st != MFA_OK) return st;
  return launch_attn(c, as_stream(stream));
}

mfa_status mfa_decode_attn_q8(const void* q, int q_dtype, int B, int q_len, int H,
                              const mfa_kv_cache* cache, const int32_t* seq_lens, int max_seq_len,
                              float sm_scale, int num_splits, int chunk_tokens, void* workspace,
                              size_t workspace_bytes, void* out, int out_dtype, void* stream) {
  AttnCall c;
  const mfa_status st = prepare_attn(q, q_dtype, B, H, cache, seq_lens, max_seq_len, sm_scale,
                                     num_splits, chunk_tokens, workspace, workspace_bytes, out,
                                     out_dtype, &c, q_len, true);
  if (st != MFA_OK) return st;
  return launch_attn(c, as_stream(stream));
}

mfa_status mfa_decode_step(const mfa_step_args* s, void* stream) {
  if (!s) return MFA_ERR_NULL;
  const bool has_qproj = s->x != nullptr;
  QprojCall qc{};
  if (has_qproj) {
    const mfa_status st = prepare_qproj(s->x, s->w_qdown, s->q_norm_w, s->w_qup, s->q,
                                        s->qproj_workspace, s->qproj_workspace_bytes, s->B,
                                        s->hidden, s->q_rank, s->H, s->d, s->eps, s->dtype,
                                        s->weight_layout, &qc);
    if (st != MFA_OK) return st;
  }
  const bool proj = s->w_kv != nullptr;
  if (proj) {
    if (!has_qproj) return MFA_ERR_NULL;                 // the projection needs x
    if (!aligned16(s->w_kv)) return MFA_ERR_ALIGN;
    if (s->kv_in_dtype != s->dtype) return MFA_ERR_DTYPE;
    if (s->cache && s->cache->head_dim != s->d) return MFA_ERR_SHAPE;
    qc.w_kv = s->w_kv;
    qc.kvc = 2 * s->d;
  }
  mfa::AppendArgs ap;
  mfa_status st = prepare_append(s->k_new, s->v_new, s->kv_in_dtype, s->pos, 1, s->B, s->cache, &ap,
                                 proj);
  if (st != MFA_OK) return st;
  AttnCall ac;
  st = prepare_attn(s->q, s->dtype, s->B, s->H, s->cache, s->seq_lens, s->max_seq_len, s->sm_scale,
                    s->num_splits, s->chunk_tokens, s->split_workspace, s->split_workspace_bytes,
                    s->out, s->out_dtype, &ac);
  if (st != MFA_OK) return st;
  if (s->cache->head_dim != s->d) return MFA_ERR_SHAPE;
  hipStream_t hs = as_stream(stream);
  if (has_qproj) {
    st = launch_qproj(qc, &ap, hs);            // the append rides in the RMSNorm launch
    if (st != MFA_OK) return st;
  } else if (ac.mfma && !ap.in_f32 && ac.a.num_splits != 0) {
    return launch_attn(ac, hs, &ap);           // split walk: the append rides in the attention launch
  } else if (mfa::launch_kv_append(ap, hs) != hipSuccess) {
    return MFA_ERR_HIP;
  }
  return launch_attn(ac, hs);
}

mfa_status mfa_combine(const void* workspace, size_t workspace_bytes, int B, int H, int d,
                       int num_splits, void* out, int out_dtype, void* stream) {
  if (!workspace || !out) return MFA_ERR_NULL;
  if (!aligned16(workspace) || !aligned16(out)) return MFA_ERR_ALIGN;
  if (B < 1 || H < 1 || num_splits == 1 || num_splits < 0) return MFA_ERR_SHAPE;
  if (num_splits == 0 && B > mfa::kBalancedMaxRows) return MFA_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return MFA_ERR_SHAPE;
  if (out_dtype != MFA_BF16 && out_dtype != MFA_F32) return MFA_ERR_DTYPE;
  if (workspace_bytes < mfa_decode_workspace_bytes(B, H, d, num_splits)) return MFA_ERR_WORKSPACE;
  const SplitLayout l = workspace_layout(B, H, d, num_splits);
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  const int* meta = num_splits == 0 ? reinterpret_cast<const int*>(ws + l.off_meta) : nullptr;
  return from_hip(mfa::launch_combine(reinterpret_cast<const float*>(ws),
                                      reinterpret_cast<const float*>(ws + l.off_ml), meta, B, H, d,
                                      effective_splits(B, num_splits), out, out_dtype == MFA_F32,
                                      as_stream(stream)));
}

}  // extern "C"
