/*
 * mfa.h -- C ABI of libmfa: the decode step of Multi-Matrix Factorization
 * Attention (MFA) on one AMD Instinct MI355X (gfx950).
 *
 * Source of the method: "Step-3 is Large yet Affordable: Model-system
 * Co-design for Cost-effective Decoding" (paperlayer.ai summary of arXiv
 * 2507.19427v1). §2 Step-3 Model Card: MFA applies a low-rank factorisation
 * in the QK circuit so that many attention heads share a small KV cache.
 * §5 Model-System Co-design: one KV head of an 8-bit cache shared by all
 * query heads gives arithmetic intensity 128 and effective rank 16,384
 * (64 heads x 256); KV quantisation raises the intensity. §6 Non-Flagship
 * Hardware Support: the attention stays memory-bandwidth bound. §7
 * Implementation and Results: attention instances own the KV caches.
 *
 * The pages print no equations. The readings this library implements:
 *   q    = RMSNorm(x W_qdown^T; g, eps) W_qup^T, split into H heads of width d
 *          (head h = output columns h*d .. h*d+d-1);
 *   o[h] = softmax_t(q[h] . k_t * sm_scale) . V over every cached token t of
 *          the sequence, all H heads against the same single K/V head.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Pointers are DEVICE pointers unless marked "host". The caller allocates
 *   and owns all memory, including scratch ("workspace") buffers; the
 *   library keeps no state between calls and never allocates, frees or
 *   synchronises.
 * - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *   void*; NULL means the null stream).
 * - Arguments are checked on the host before anything is launched; a check
 *   that fails returns a nonzero mfa_status and enqueues nothing. A launch
 *   failure reported by the HIP runtime returns MFA_ERR_HIP.
 * - Device-side data (sequence lengths, positions, block ids) is clamped to
 *   its documented range by the kernels, so malformed values give
 *   meaningless results but no out-of-bounds access.
 * - Every call is reentrant. Calls that write the same memory race unless
 *   the caller orders them on one stream.
 * - Tensors are dense and row-major in the order written, with the last
 *   index fastest. Device pointers must be 16-byte aligned, except the int32
 *   arrays (block table, positions, lengths), which need 4.
 *
 * KV cache layout (owned by the caller, written only by mfa_kv_append)
 * ---------------------------------------------------------------------
 * The cache of one layer holds one K head and one V head of width d. It is
 * stored in blocks of MFA_BLOCK_TOKENS = 64 consecutive logical tokens of
 * one sequence; every block of k and of v is 64*d elements:
 *   k       [num_blocks][64*d]    elements of dtype, order below
 *   v       [num_blocks][64*d]    elements of dtype, order below
 *   k_scale [num_blocks][64]      fp32, FP8 caches only (else NULL)
 *   v_scale [num_blocks][64]      fp32, FP8 caches only (else NULL)
 * Logical token t of sequence b is in logical block t/64 at offset t%64. The
 * block table [B][max_blocks_per_seq] (int32, device) maps logical block j of
 * sequence b to a physical block id. Without a block table (NULL) the cache
 * is contiguous: logical block j of sequence b is physical block
 * b*max_blocks_per_seq + j.
 *
 * Element order inside a block (t = token in block, f = feature < d). BF16
 * and FP8 blocks are stored in the order the matrix-core operands consume
 * them, as units of 64 lanes x 16 bytes (1 KB), so that every wave-wide
 * 16-byte load of the attention kernel reads contiguous memory:
 *   BF16 K: unit u = (t/16)*(d/32) + f/32; lane = 16*((f%32)/8) + t%16;
 *           element (t, f) at ((u*64 + lane)*8 + f%8)
 *   BF16 V: unit u = (f/16)*2 + t/32; lane = 16*((t%32)/8) + f%16;
 *           element (t, f) at ((u*64 + lane)*8 + t%8)
 *   FP8 K:  unit u = (t/16)*(d/64) + f/64; lane = 16*((f%64)/16) + t%16;
 *           element (t, f) at ((u*64 + lane)*16 + f%16)
 *   FP8 V:  unit u = f/16; lane = 16*(t/16) + f%16;
 *           element (t, f) at ((u*64 + lane)*16 + t%16)
 *   F32 K:  element (t, f) at (t*d + f)      (token-major rows)
 *   F32 V:  element (t, f) at (f*64 + t)     (feature-major rows)
 * (positions in elements from the start of the block).
 *
 * FP8 caches hold OCP e4m3 codes (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits, max 448, no infinities) with one fp32 scale per token for K
 * and one for V: scale = amax/448 over the token's d values (one correctly
 * rounded fp32 division; 1 when amax = 0), code = round-to-nearest-even of
 * the correctly rounded fp32 quotient x/scale. The stored value is
 * code * scale.
 */
#ifndef MFA_H
#define MFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MFA_ABI_VERSION 3
#define MFA_BLOCK_TOKENS 64
/* Most query tokens per sequence in mfa_decode_attn_multi. */
#define MFA_MAX_QUERY_TOKENS 16

typedef enum {
  MFA_OK = 0,
  MFA_ERR_NULL = 1,         /* a required pointer is NULL                    */
  MFA_ERR_SHAPE = 2,        /* a size is out of range or inconsistent        */
  MFA_ERR_DTYPE = 3,        /* unsupported dtype or dtype combination        */
  MFA_ERR_ALIGN = 4,        /* a device pointer is not 16-byte aligned       */
  MFA_ERR_UNSUPPORTED = 5,  /* valid request the library has no kernel for  */
  MFA_ERR_WORKSPACE = 6,    /* workspace missing or smaller than required    */
  MFA_ERR_HIP = 7,          /* the HIP runtime reported a launch failure     */
  MFA_ERR_TOO_LARGE = 8     /* needs more than the library's static scratch  */
} mfa_status;

typedef enum {
  MFA_WEIGHTS_ROWMAJOR = 0, /* [out][in] row-major (torch Linear)            */
  MFA_WEIGHTS_PACKED = 1    /* operand order, made by mfa_pack_weight        */
} mfa_weight_layout;

typedef enum {
  MFA_F32 = 0,              /* IEEE binary32                                 */
  MFA_BF16 = 1,             /* bfloat16                                      */
  MFA_FP8_E4M3 = 2          /* OCP e4m3 ("e4m3fn"), KV caches only           */
} mfa_dtype;

/* Description of one layer's KV cache (host struct, read during the call). */
typedef struct {
  void *k;                      /* device: [num_blocks][64][d] of dtype      */
  void *v;                      /* device: [num_blocks][d][64] of dtype      */
  float *k_scale;               /* device: [num_blocks][64], FP8 only        */
  float *v_scale;               /* device: [num_blocks][64], FP8 only        */
  const int32_t *block_table;   /* device: [B][max_blocks_per_seq] or NULL   */
  int32_t num_blocks;           /* physical blocks in k / v                  */
  int32_t max_blocks_per_seq;   /* table row length; capacity = 64x this     */
  int32_t head_dim;             /* d: 64, 128 or 256                         */
  int32_t dtype;                /* mfa_dtype of k and v                      */
} mfa_kv_cache;

/* Version of this ABI (MFA_ABI_VERSION of the built library). */
int mfa_abi_version(void);

/* Static, host-owned text for a status code. Never NULL. */
const char *mfa_status_str(int status);

/*
 * Query path (§2 Step-3 Model Card: low-rank factorisation in the QK
 * circuit; reading: down-projection, RMSNorm with gain, up-projection):
 *   c = x W_qdown^T            (fp32 accumulation)
 *   n = c / sqrt(mean(c^2) + eps) * g
 *   q = n W_qup^T -> q_out[B][H][d]
 * x        [B][hidden]          dtype
 * w_qdown  [q_rank][hidden]     dtype (torch Linear [out][in]), or packed
 * q_norm_w [q_rank]             fp32 gain g
 * w_qup    [H*d][q_rank]        dtype, or packed
 * weight_layout: MFA_WEIGHTS_ROWMAJOR, or MFA_WEIGHTS_PACKED (bf16 only: both
 *          weights packed by mfa_pack_weight)
 * q_out    [B][H][d]            dtype
 * workspace: >= mfa_qproj_workspace_bytes(B, hidden, q_rank, H, d, dtype) bytes
 *          (fp32 split-K partials and the normalised latent n). The size also
 *          covers mfa_decode_step with the K/V projection (w_kv set) for the
 *          same arguments, d being the KV head dim.
 * dtype: MFA_BF16 (c kept in fp32; n and q rounded to bf16) or MFA_F32 (all
 * fp32). Limits: 1 <= B <= 256, q_rank <= 8192; bf16: hidden and q_rank
 * multiples of 256, H*d a multiple of 64; fp32: hidden and H*d multiples of 4,
 * q_rank a multiple of 8.
 */
size_t mfa_qproj_workspace_bytes(int B, int hidden, int q_rank, int H, int d, int dtype);
mfa_status mfa_qproj(const void *x, const void *w_qdown, const float *q_norm_w,
                     const void *w_qup, void *q_out, void *workspace,
                     size_t workspace_bytes, int B, int hidden, int q_rank,
                     int H, int d, float eps, int dtype, int weight_layout,
                     void *stream);

/*
 * Weight packing for mfa_qproj (bf16): rewrites a row-major weight w [N][K]
 * (torch Linear [out][in]) into packed [N*K] in the order the matrix-core
 * operands read it, so that the query path streams weights in 1 KB
 * contiguous pieces. The packed weight is cut into 1 KB units of 64 lanes x
 * 16 bytes; unit (nt = n/16, kt = k/32) is unit number nt*(K/32) + kt, and
 * in it lane 16*((k%32)/8) + n%16 holds w[n][8*(k/8) .. 8*(k/8)+7].
 * Pack once (weights are static) and pass MFA_WEIGHTS_PACKED to mfa_qproj.
 * N % 16 == 0, K % 32 == 0, dtype MFA_BF16. packed must not alias w.
 */
mfa_status mfa_pack_weight(const void *w, void *packed, int N, int K, int dtype,
                           void *stream);

/*
 * KV append (§7 Implementation and Results: attention instances own the KV
 * caches): writes n_new consecutive tokens of every sequence b, logical
 * positions pos[b] .. pos[b]+n_new-1, into the cache. The decode step uses
 * n_new = 1; a larger n_new fills a cache from a prompt.
 * k_new, v_new [B][n_new][d] of in_dtype (MFA_F32 or MFA_BF16).
 * pos [B] int32 device. Positions must lie below 64*max_blocks_per_seq and
 * their blocks must be mapped by the block table.
 * Caches of dtype F32 or BF16 take inputs of the same dtype and store them
 * bit for bit. FP8 caches quantise each token as documented above and
 * store codes and scales.
 * Sequence lengths are the caller's: after appending, the caller sets
 * seq_lens[b] = pos[b] + n_new.
 */
mfa_status mfa_kv_append(const void *k_new, const void *v_new, int in_dtype,
                         const int32_t *pos, int n_new, int B,
                         const mfa_kv_cache *cache, void *stream);

/*
 * Split plan for mfa_decode_attn: the number of KV splits and tokens per
 * split (a multiple of 64) this library would use for B sequences of at
 * most max_seq_len tokens with H heads of width d. Host-only, no launch.
 * Returns MFA_OK and writes *num_splits, *chunk_tokens (host pointers).
 */
mfa_status mfa_decode_plan(int B, int H, int d, int max_seq_len, int kv_dtype,
                           int *num_splits, int *chunk_tokens);

/*
 * Split plan from the batch's lengths (host array seq_lens[B], the values the
 * call will attend, 0 .. capacity): as mfa_decode_plan for the longest row,
 * or the balanced partition (*num_splits = MFA_SPLITS_BALANCED,
 * *chunk_tokens = 0) when the lengths are mixed enough that the split plan's
 * longest workgroup would walk clearly more blocks (5% plus one block; 15%
 * for FP8 caches, whose split kernel takes two blocks per iteration) than
 * the balanced partition gives each workgroup. The balanced partition is
 * offered only for the matrix-core shapes, up to MFA_BALANCED_MAX_ROWS rows
 * and 2^21 blocks in all. Host-only, no launch. For multi-token decode
 * (mfa_decode_attn_multi) prefer mfa_decode_plan over the B*q_len rows: its
 * splits keep the query rows of a sequence side by side on one XCD, where
 * they share the KV blocks through L2, while the balanced partition walks
 * each query row's blocks separately (measured 218 against 212 us at 128
 * mixed-length sequences with 2 query tokens, 434 against 365 us with 4).
 */
#define MFA_SPLITS_BALANCED 0
#define MFA_BALANCED_MAX_ROWS 1024
mfa_status mfa_decode_plan_lens(int B, int H, int d, const int32_t *seq_lens, int kv_dtype,
                                int *num_splits, int *chunk_tokens);

/* Bytes of split workspace for mfa_decode_attn / mfa_combine (the split
 * partials of the long-context case, "Step-3 is Large yet Affordable"
 * summary page, §4 Cost Analysis for LLM Decoding: attention cost grows with
 * context and dominates from 8K on). Short plans walk every split as two
 * halves with a partial each: with S = 2*num_splits when B*num_splits*2 <=
 * 256 and B*num_splits is a multiple of 8, else S = num_splits, and
 * R = B*S*H rows:
 *   part_o  fp32 [B][S][H][d] unnormalised partial outputs at offset 0
 *           (with halves, partial k covers tokens [k*h, (k+1)*h) with
 *           h = 64*ceil(chunk_tokens/128))
 *   part_ml fp32 [B][S][H][2] at offset round_up(R*d*4, 256): the
 *           running max m in natural-log units of the scaled logits, then
 *           l = sum_t exp(s_t - m)
 * Total round_up(R*d*4, 256) + R*8 bytes; 0 when num_splits == 1. The
 * partials are fp32 whatever the output type, so mfa_combine may write
 * either output type. The caller owns the workspace; the library keeps
 * nothing in it between calls.
 * For the balanced partition (num_splits == MFA_SPLITS_BALANCED, B <=
 * MFA_BALANCED_MAX_ROWS, else 0 bytes) there are 256 + B partial slots:
 * R = (256 + B)*H rows of part_o and part_ml as above (slot w + b holds the
 * piece of row b that workgroup w walked), then int32 [B][2] at offset
 * round_up(off_ml + R*8, 16): row b's first slot and its number of slots. */
size_t mfa_decode_workspace_bytes(int B, int H, int d, int num_splits);
/* The same function under its earlier name. */
size_t mfa_split_workspace_bytes(int B, int H, int d, int num_splits);

/*
 * Decode attention (§2/§5: all H query heads against one shared K/V head).
 * q          [B][H][d] of q_dtype (MFA_BF16 with BF16/FP8 caches, MFA_F32 with
 *            F32 caches)
 * seq_lens   [B] int32 device: tokens of sequence b to attend (0..max_seq_len;
 *            0 gives zeros)
 * max_seq_len host upper bound of seq_lens (sizes the launch)
 * sm_scale   logit scale, positive and finite (1/sqrt(d) for scaled dot
 *            products); anything else is MFA_ERR_SHAPE
 * num_splits >= 1 KV splits per sequence; split j covers tokens
 *            [j*chunk_tokens, min((j+1)*chunk_tokens, seq_len)). Requires
 *            chunk_tokens % 64 == 0 and num_splits*chunk_tokens >= max_seq_len.
 *            MFA_SPLITS_BALANCED (0) instead runs the balanced partition
 *            (matrix-core shapes, B <= MFA_BALANCED_MAX_ROWS, at most 2^21
 *            blocks of 64 tokens in all; chunk_tokens is ignored): the
 *            batch's blocks, concatenated row after row, are cut evenly over
 *            the chip's 256 compute units, so rows of mixed lengths cost one
 *            equal share each instead of the longest split. A row start that
 *            falls inside a share is charged 1.5 blocks of work (the piece
 *            that ends there costs its workgroup that much). The same
 *            softmax is computed: results equal the split plan's up to
 *            rounding.
 * workspace  mfa_decode_workspace_bytes(...) bytes when num_splits != 1
 *            (receives the partials), else may be NULL.
 * out        [B][H][d] of out_dtype (MFA_BF16 or MFA_F32). With
 *            num_splits != 1, out may be NULL: only the partials are
 *            written and the caller runs mfa_combine; otherwise the library
 *            merges the partials into out on the same stream.
 * Supported: H in 1..64 and d in {64,128,256} with F32 caches (VALU kernel);
 * H == 64 and d == 256 with BF16 or FP8 caches (matrix-core kernel).
 */
mfa_status mfa_decode_attn(const void *q, int q_dtype, int B, int H,
                           const mfa_kv_cache *cache, const int32_t *seq_lens,
                           int max_seq_len, float sm_scale, int num_splits,
                           int chunk_tokens, void *workspace,
                           size_t workspace_bytes, void *out, int out_dtype,
                           void *stream);

/*
 * Decode attention that allocates nothing, for callers that cannot allocate
 * or pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): mfa_decode_attn with its split partials
 * in a scratch array the library holds in device memory, MFA_STATIC_SCRATCH
 * bytes on every GPU it runs on, until the process ends. Arguments as in
 * mfa_decode_attn, less the workspace; out is required (the library merges
 * the splits into it). A call whose partials need more than
 * MFA_STATIC_SCRATCH bytes (mfa_decode_workspace_bytes(B, H, d, num_splits))
 * returns MFA_ERR_TOO_LARGE and enqueues nothing. All calls on one GPU share
 * that GPU's scratch: calls that can overlap on one GPU (other streams,
 * other host threads without ordering) race and give wrong results; calls
 * ordered on one stream do not. Nothing in the scratch needs clearing
 * between calls (every split writes its own partials). The first call on a
 * device looks up that device's scratch address (MFA_ERR_HIP if that
 * fails).
 */
#define MFA_STATIC_SCRATCH (32u << 20)
mfa_status mfa_decode_attn_static(const void *q, int q_dtype, int B, int H,
                                  const mfa_kv_cache *cache, const int32_t *seq_lens,
                                  int max_seq_len, float sm_scale, int num_splits,
                                  int chunk_tokens, void *out, int out_dtype,
                                  void *stream);

/*
 * Multi-token decode attention: q_len new tokens per sequence (several
 * tokens decoded in one step, as in multi-token prediction: "Step-3 is Large
 * yet Affordable" summary page, §5, where more query tokens per KV read
 * raise the attention's arithmetic intensity). The q_len new tokens are the
 * last q_len of each sequence (appended before the call, e.g. by
 * mfa_kv_append with n_new = q_len); query token j (0-based) of sequence b
 * attends to the sequence's first seq_lens[b] - (q_len - 1 - j) tokens, so
 * the new tokens see each other causally.
 *   q        [B][q_len][H][d] of q_dtype
 *   out      [B][q_len][H][d] of out_dtype
 *   q_len    1 .. MFA_MAX_QUERY_TOKENS; q_len == 1 is mfa_decode_attn
 * Every other argument is as in mfa_decode_attn, with the split partials and
 * the combine over the B * q_len rows (sequence, query token): the workspace
 * is mfa_decode_workspace_bytes(B * q_len, H, d, num_splits) bytes and a
 * separate mfa_combine takes B * q_len as its batch. The query tokens of a
 * sequence run on one XCD side by side, so its KV blocks are read from HBM
 * about once and from that XCD's L2 q_len times.
 */
mfa_status mfa_decode_attn_multi(const void *q, int q_dtype, int B, int q_len, int H,
                                 const mfa_kv_cache *cache, const int32_t *seq_lens,
                                 int max_seq_len, float sm_scale, int num_splits,
                                 int chunk_tokens, void *workspace,
                                 size_t workspace_bytes, void *out, int out_dtype,
                                 void *stream);

/*
 * FP8-query decode attention (FP8 caches, H = 64, d = 256): as
 * mfa_decode_attn_multi (q_len = 1 is single-token decode), with Q.K^T on
 * the FP8 matrix cores. The page runs attention in FP8 ("Step-3 is Large yet
 * Affordable" summary page, §7; §5: an 8-bit KV cache). Each (row, head)
 * of the bf16 q is quantized inside the call with the cache's own codec:
 *   s = max_i |q_i| / 448 (1 when 0; one correctly rounded fp32 division),
 *   code_i = RNE e4m3(q_i / s),
 * and the logits are (codes . K codes) * s * k_scale * sm_scale. Softmax,
 * P.V (bf16 P, V widened to bf16), the split partials and the combine are
 * those of mfa_decode_attn. The result therefore equals attention with q
 * replaced by its e4m3 dequantisation, up to fp32 rounding.
 * Errors: MFA_ERR_UNSUPPORTED unless the cache is MFA_FP8_E4M3 and H = 64,
 * d = 256; q_dtype must be MFA_BF16; everything else as mfa_decode_attn_multi.
 */
mfa_status mfa_decode_attn_q8(const void *q, int q_dtype, int B, int q_len, int H,
                              const mfa_kv_cache *cache, const int32_t *seq_lens,
                              int max_seq_len, float sm_scale, int num_splits,
                              int chunk_tokens, void *workspace, size_t workspace_bytes,
                              void *out, int out_dtype, void *stream);

/*
 * Split combine ("Step-3 is Large yet Affordable" summary page, §4 Cost
 * Analysis for LLM Decoding: attention cost grows with context and
 * dominates the FFN from 8K on, so one sequence's context is spread over
 * many workgroups and their partial softmax sums are merged here): merges
 * the num_splits partials (layout as in mfa_decode_workspace_bytes) of
 * every (sequence, head) by log-sum-exp:
 *   m* = max_j m_j,  w_j = exp(m_j - m*),  out = sum_j w_j o_j / sum_j w_j l_j.
 * Splits with l_j == 0 (empty) get weight 0; a head whose splits are all
 * empty gives zeros. out [B][H][d] of out_dtype (MFA_BF16 or MFA_F32; the
 * partials are fp32 either way). num_splits >= 2, or MFA_SPLITS_BALANCED
 * for the balanced partition's workspace (each row's own slots, as the
 * attention call listed them); d in {64, 128, 256}.
 * Host checks as for every call;
 * MFA_ERR_WORKSPACE when workspace_bytes is below the required size.
 */
mfa_status mfa_combine(const void *workspace, size_t workspace_bytes, int B,
                       int H, int d, int num_splits, void *out, int out_dtype,
                       void *stream);

/*
 * Attention output projection and the FP8 hand-off to the FFN side
 * ("Step-3 is Large yet Affordable" summary page, §7: attention instances
 * send FP8 tokens with their scales to the FFN instances; 128 tokens of
 * hidden 7168 are 896 KiB of codes):
 *   y = o W_o^T                 (fp32 accumulation, rounded to bf16)
 *   scales[b] = max_j |y[b][j]| / 448  (1 when the row is zero; one correctly
 *               rounded fp32 division),  codes[b][j] = RNE e4m3(y[b][j] / scales[b])
 * o        [B][HD] bf16 (the attention output, heads concatenated)
 * w_o      [hidden][HD] bf16 (torch Linear [out][in]), or packed by
 *          mfa_pack_weight when weight_layout is MFA_WEIGHTS_PACKED
 * y        [B][hidden] bf16, or NULL (not written)
 * codes    [B][hidden] OCP e4m3 bytes and scales [B] fp32: both or neither
 *          (at least one of y and codes must be given)
 * workspace >= mfa_out_proj_workspace_bytes(B, HD, hidden, dtype) bytes
 *          (fp32 split-K partials)
 * dtype    MFA_BF16. Limits: 1 <= B <= 256; HD a multiple of 256; hidden a
 *          multiple of 64, at most 8192.
 */
size_t mfa_out_proj_workspace_bytes(int B, int HD, int hidden, int dtype);
mfa_status mfa_out_proj(const void *o, const void *w_o, int weight_layout, int B, int HD,
                        int hidden, int dtype, void *workspace, size_t workspace_bytes,
                        void *y, void *codes, float *scales, void *stream);

/*
 * One whole decode step on one stream, equal to
 *   mfa_qproj (when x != NULL) -> mfa_kv_append (one token per sequence)
 *   -> mfa_decode_attn (with out: attention and split combine)
 * with the same arguments, in that order, and with the same results.
 * It exists so the stages can share launches: with a query path, the KV
 * append runs inside the query path's normalisation launch instead of on
 * its own; without one, with bf16 k_new / v_new and a split plan
 * (num_splits >= 1) on the matrix-core kernel (H = 64, d = 256), inside
 * the attention launch (the workgroup that reads the token's block writes
 * the token first). The balanced plan keeps its own append launch.
 * Every stage's arguments are checked (as by the separate calls) before
 * anything is launched.
 *   B, H, d      batch, query heads, head dim (d must equal cache->head_dim)
 *   dtype        MFA_BF16 or MFA_F32: x, weights and q (as in mfa_qproj and
 *                the q_dtype of mfa_decode_attn)
 *   x ... q_rank, eps, weight_layout, qproj_workspace(_bytes): as in
 *                mfa_qproj; x == NULL skips the query path and q is an input
 *   q            [B][H][d] device: written by the query path, read by the
 *                attention
 *   k_new, v_new [B][d] of kv_in_dtype; pos [B] int32: as in mfa_kv_append
 *                with n_new == 1
 *   cache ... out_dtype: as in mfa_decode_attn
 *   w_kv         optional K/V projection of the new token (the input side
 *                of the attention instance's KV cache: "Step-3 is Large yet
 *                Affordable" summary page, §7, attention instances own their
 *                KV caches). NULL: k_new, v_new are inputs. Otherwise (x must
 *                be set) w_kv is [2d][hidden] of dtype, W_k stacked over W_v
 *                (torch Linear [out][in]; packed by mfa_pack_weight as one
 *                2d x hidden matrix when weight_layout is packed), and
 *                  k = x W_k^T,  v = x W_v^T   (fp32 accumulation)
 *                rounded to dtype are appended at pos instead; k_new, v_new
 *                are then optional outputs ([B][d] of dtype; NULL: not
 *                written) and kv_in_dtype must equal dtype. The product
 *                shares the down-projection's launch (x is read once).
 */
typedef struct {
  int B, H, d, dtype;
  const void *x, *w_qdown, *w_qup;
  const float *q_norm_w;
  int hidden, q_rank, weight_layout;
  float eps;
  void *qproj_workspace;
  size_t qproj_workspace_bytes;
  void *q;
  const void *k_new, *v_new;
  int kv_in_dtype;
  const int32_t *pos;
  const mfa_kv_cache *cache;
  const int32_t *seq_lens;
  int max_seq_len;
  float sm_scale;
  int num_splits, chunk_tokens;
  void *split_workspace;
  size_t split_workspace_bytes;
  void *out;
  int out_dtype;
  const void *w_kv;
} mfa_step_args;

mfa_status mfa_decode_step(const mfa_step_args *args, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MFA_H */
