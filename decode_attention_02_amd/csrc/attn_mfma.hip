// MFA decode attention on the matrix cores: 64 query heads of width 256
// against one shared K/V head, bf16 or OCP-e4m3 KV cache.
//
// The method: "Step-3 is Large yet Affordable" (summary page), §2 Step-3
// Model Card (many query heads share a small KV cache through MFA's
// low-rank QK circuit) and §5 Model-System Co-design (one KV head read once
// for all 64 heads: 128 flop per byte of an 8-bit cache, 64 per byte of a
// bf16 cache). §6 states the attention stays memory-bandwidth bound, so the
// kernel is built around keeping HBM busy: every K and V byte is read once,
// with several cache blocks in flight per compute unit at all times.
//
// One workgroup (8 waves, 2 per SIMD) owns one (sequence, split) pair and
// walks it one 64-token cache block at a time. The waves split by role, and
// each role runs its own loop (the role index is a scalar, so the branch is
// uniform and each wave passes only its own role's barriers; both loops pass
// the same number):
//   * QK waves 0..3: wave w holds K rows 16w..16w+15 of each block and
//     computes S^T[token][head] = K . Q^T on the 16x16x32 matrix cores (the
//     16 tokens are the row side, the 64 heads sharing the KV head four
//     16-column tiles of Q, staged once in LDS in operand order), writes the
//     logits to LDS and its per-head maximum over its 16 tokens;
//   * PV waves 4..7: wave 4+j runs the online softmax for the 16 tokens QK
//     wave j scored (block max from the four per-wave maxima, p = exp2(s * c
//     - m) as one fma and one exp2, lane-partial row sums, P^T (bf16) into
//     LDS), and holds the V^T rows (features) 64j..64j+63 of each block to
//     accumulate O^T[feature][head] += V^T . P^T.
// Each wave holds only its own role's operands in a register ring of RK
// (QK) or RV (PV) blocks, filled with buffer loads. The stages are skewed
// across iterations separated by one barrier each: iteration i computes S
// of unit i, the P.V product of unit i-2 and the softmax of unit i-1, where a
// unit is one cache block, or two consecutive blocks for FP8 caches (the same
// bytes between barriers as one bf16 block, twice the independent work).
// Every iteration issues the same number of loads (past the walk through
// empty buffer resources, which read nothing), so the compiler's wait before
// a ring slot is consumed leaves the younger slots in flight. The ring loads
// are non-temporal (each cache byte is read once). At the end the PV waves
// stage bf16 outputs in LDS and all eight waves store whole 512-byte head
// rows; fp32 results (split partials, fp32 outputs) are stored directly.
// The running max is updated lazily: only when a block's max exceeds it by
// more than 2^8 (log2 units) are O and the row sums rescaled, so p <= 256;
// the result is the same softmax, normalised by the same reference at the end.
// Cache blocks are stored in operand order (kv_layout.h): every wave-wide
// 16-byte load reads 1 KB of contiguous memory and lands in the operand
// registers as is. FP8 codes are widened to bf16 in registers (exact);
// per-token K scales multiply the logits, V scales multiply P before its
// bf16 rounding.
// Several query tokens per sequence (multi-token decode) are virtual rows:
// row r = sequence b, query token j walks b's cache up to its own position.
// FP8 queries (Q8, FP8 caches): the QK waves quantize each head's q row to
// e4m3 with one scale amax/448 (the cache's own per-token codec) while
// staging it, and multiply the raw K codes from the ring on the 16x16x128
// FP8 matrix cores (two products per 16x16 tile, no K conversion); the
// logits are scaled by the K and q scales. The PV side is unchanged.
#include <type_traits>

#include "append_one.h"
#include "device_common.h"
#include "kernels.h"

namespace mfa {

namespace {

constexpr int kH = 64;
constexpr int kD = 256;
constexpr float kLazy = 8.0f;           // rescale only when the max grows by > 2^8
// balanced partition: extra cost of a row start, in quarter blocks (a piece
// that ends inside a walk stalls its workgroup for about 1.5 blocks' time)
constexpr int kBalRowCost = 6;

template <bool FP8>
struct Cfg {
  static constexpr int kBlockBytes = kBlockTokens * kD * (FP8 ? 1 : 2);
  static constexpr int kLoads = FP8 ? 4 : 8;     // 16-byte loads per lane per block (K or V)
  static constexpr int kSlot = kLoads + (FP8 ? 2 : 0);   // + K and V scales (QK waves, FP8)
};

// Unroll of a loop over blocks that keeps ring slots (ring of R) and
// parities static: a multiple of R and of 2.
constexpr int unroll_for(int r) { return r % 2 ? 2 * r : r; }

// d offset of operand k-step s for lane group g (the K and Q sides agree).
template <bool FP8>
__device__ __forceinline__ int qk_dim(int s, int g) {
  return FP8 ? ((s >> 1) * 64 + g * 16 + (s & 1) * 8) : (s * 32 + g * 8);
}

// Calls f(std::integral_constant<int, I>) for I = I0 .. I1-1 (a compile-time
// unrolled loop: register arrays indexed by I stay in registers).
template <int I0, int I1, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < I1) {
    f(std::integral_constant<int, I0>{});
    static_for<I0 + 1, I1>(f);
  }
}

__device__ __forceinline__ uint32_t keep_bf16(uint32_t word, bool lo_ok, bool hi_ok) {
  return (lo_ok ? (word & 0xffffu) : 0u) | (hi_ok ? (word & 0xffff0000u) : 0u);
}

// Buffer-resource word 3 for untyped dword loads (32-bit data format).
constexpr int kRsrcFlags = 0x00020000;

// 16-byte load through a buffer resource; a resource with zero records makes
// it a load that returns zeros and touches no memory. The loads are marked
// non-temporal: every cache byte is read once per launch, and streaming it
// past the caches raised the plain stream rate from 5.96 to 6.62 TB/s.
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

}  // namespace

// RK, RV: ring depth (blocks of registers) of the QK and of the PV waves.
// BAL: the balanced partition (num_splits == 0). The rows' 64-token blocks,
// concatenated in row order, are cut into gridDim.x equal ranges, one per
// workgroup (fewer when there are fewer blocks than workgroups). A workgroup
// walks its range across row boundaries: each row it touches is a "piece"
// with its own partial (o, m, l) in slot (workgroup + row). At the first
// block of a new piece the QK waves switch Q (loaded into registers one
// piece ahead) behind one extra barrier that both roles pass, and the PV
// waves put the finished piece's o into LDS (the workgroup's first piece,
// stored by the QK waves at the end: partials written during the walk slow
// the reads of every workgroup) or store it (later pieces, rare), then its
// (m, l) one iteration later, once the four PV waves' row sums have met.
// APP (split walk): the decode step's KV append (one new token per row,
// bf16 input) in the same launch. The workgroup whose split walks the
// token's block writes the token before its waves read the block: the QK
// wave that loads the token's K rows reads the token together with Q,
// stores K (and the FP8 scales) before it issues the ring unit holding the
// block, and passes V (with its slot and scale) through LDS to the PV
// waves, which store their features of it after the Q barrier, before their
// first V loads. A wave's memory operations take effect in its program
// order, so its later loads of the block see its own stores. A token in a
// block past the row's length has no reader in the launch; the row's first
// split writes it whole. (The balanced walk keeps the separate append: there
// the extra work at the start of the owning workgroups cost more than the
// launch it saves.)
template <bool FP8, int RK, int RV, bool Q8 = false, int BPI = 1, bool BAL = false,
          bool APP = false>
__global__ __launch_bounds__(512) void mfa_decode_mfma_kernel(
    std::conditional_t<APP, AttnAppArgs, AttnArgs> a) {
  constexpr int HT = 4;                 // 16-head tiles: every workgroup holds all 64 heads
  static_assert(!Q8 || FP8, "FP8 queries run against FP8 caches");
  static_assert(!APP || (!Q8 && !BAL), "in-launch append: split walk, bf16 queries");
  static_assert(BPI == 1 || (BPI == 2 && !Q8), "two blocks per iteration: plain FP8 and bf16 only");
  static_assert(!BAL || (BPI == 1 && !Q8), "balanced walk: one block per unit");
  using C = Cfg<FP8>;
  constexpr int kHW = 16 * HT;                                          // heads of this workgroup
  // Q in operand order: bf16 HT x 8 KB; Q8 codes HT x 4 KB, block (ht, k2),
  // lane (gg, cc), two uint4: codes of q[h0+16ht+cc][128k2 + 16gg .. +16]
  // and [128k2 + 64 + 16gg .. +16] (the K ring's unit pair for k2)
  __shared__ __attribute__((aligned(16))) uint4 q_lds[HT * (Q8 ? 4 : 8) * 64];
  __shared__ float qs_lds[Q8 ? kHW : 1];                                 // Q8: q scale per head
  // per parity, per block of the iteration unit (bb < BPI)
  __shared__ __attribute__((aligned(16))) uint4 p_lds[2][BPI * HT * 2 * 64];  // HT x 2 KB per block, operand order
  __shared__ __attribute__((aligned(16))) f32x4_t s_lds[2][BPI * 4 * HT * 64]; // logits by (block, QK wave, tile, lane)
  __shared__ __attribute__((aligned(16))) float red[2][kHW * 4];        // block max [head][QK wave]
  __shared__ __attribute__((aligned(16))) uint4 vs_lds[2][BPI * 16];    // FP8 V scales by (block, QK wave, row)
  __shared__ __attribute__((aligned(16))) float lred[kHW * 4];          // row sums [head][PV wave]
  // balanced walk: prefix sums of the rows' block counts, row lengths, the
  // scan's per-wave sums (+ the first row), and the row sums of pieces
  // finished inside the walk, by piece parity
  __shared__ int bal_pfx[BAL ? kBalancedMaxRows + 1 : 1];
  __shared__ int bal_len[BAL ? kBalancedMaxRows : 1];
  // balanced walk: o of the first piece that ends inside the walk, held here
  // until the end ([head][64 chunks of 4 features], rows padded to 65 chunks
  // so that the 16 heads of a write fall in different banks); before the
  // walk its first 8 KB hold the setup's cost prefix sums and row-start costs
  __shared__ __attribute__((aligned(16))) float4 bal_hold[BAL ? kHW * 65 : 1];
  int* const bal_cpfx = reinterpret_cast<int*>(bal_hold);
  int* const bal_rc = bal_cpfx + kBalancedMaxRows + 4;
  // APP: the V hand-off slot (QK wave -> PV waves): the token's block id,
  // offset and FP8 V scale, then its 256 bf16 V values
  __shared__ __attribute__((aligned(16))) uint32_t app_lds[APP ? 4 + kD / 2 : 1];
  __shared__ int bal_wsum[20];
  __shared__ __attribute__((aligned(16))) float lred2[2][BAL ? kHW * 4 : 4];

  const int tid = threadIdx.x;
  // wave index as a scalar: the role branches below are uniform per wave
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int ww = w & 3;                 // QK: token group; PV: feature group of 64

  // Workgroups are dispatched round-robin over the 8 XCDs (id % 8). Remap so
  // that each XCD runs a contiguous range of (sequence, split) pairs (of the
  // balanced walk's ranges): the splits of a sequence then share that XCD's
  // L2 for their query reads.
  int id = blockIdx.x;
  if ((gridDim.x & 7) == 0) id = (id & 7) * (gridDim.x >> 3) + (id >> 3);
  const int ql = a.q_len > 0 ? a.q_len : 1;
  int split = 0, b = 0, bs = 0, t1 = 0, blk0 = 0, N = 0;
  int nbl = 0, app_p = -1;              // APP: the row's blocks, its new token's position
  int lo = 0, hi = 0;                   // balanced walk: the workgroup's global block range
  bool hold_first = false;              // balanced walk: its first piece ends inside the walk
  if constexpr (BAL) {
    // rows 2 tid, 2 tid + 1: lengths (clamped like the split path), block
    // counts and costs; exclusive scans of both over all rows.
    // The partition cuts the rows' concatenated cost evenly: a block costs
    // U units and an interior row start kBalRowCost more (the price of a
    // piece that ends inside a walk: its partial stores and the Q switch),
    // so a workgroup that crosses row starts gets fewer blocks. With fewer
    // than 4 blocks per workgroup the cost is the block count alone (U = 1,
    // no row-start charge) and only min(blocks, workgroups) workgroups run.
    const int rows = a.bal_rows;
    // both lengths are read before either is stored: a store to LDS between
    // them kept the second read waiting for the first (a generic pointer
    // may alias LDS), two memory latencies instead of one
    int sl[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 2 * tid + e;
      sl[e] = r < rows ? a.seq_lens[r / ql] : 0;
    }
    int nb2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 2 * tid + e;
      int Lr = 0;
      if (r < rows) {
        const int sq = r / ql;
        Lr = sl[e] - (ql - 1 - (r - sq * ql));
        Lr = Lr < 0 ? 0 : (Lr > a.max_seq_len ? a.max_seq_len : Lr);
        bal_len[r] = Lr;
      }
      nb2[e] = (Lr + kBlockTokens - 1) >> 6;
    }
    // block counts: wave-inclusive scan; wave totals in bal_wsum[0..7]
    const int s2 = nb2[0] + nb2[1];
    int inc = s2;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(inc, off);
      if (lane >= off) inc += t;
    }
    if (lane == 63) bal_wsum[w] = inc;
    __syncthreads();
    int wpre = 0, NB = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int v = bal_wsum[k];
      wpre += k < w ? v : 0;
      NB += v;
    }
    NB = __builtin_amdgcn_readfirstlane(NB);
    const int G = static_cast<int>(gridDim.x);
    const bool weighted = NB >= 4 * G;
    const int U = weighted ? 4 : 1;                  // cost of a block
    const int RC = weighted ? kBalRowCost : 0;       // extra cost of an interior row start
    const int Geff = NB < G ? NB : G;                // every workgroup below Geff gets >= 1 block
    // A row start is interior when it is not one of the plain partition's
    // cuts floor(v NB / Geff): only there does a piece end inside a walk
    // (uniform rows that line up with the cuts are not charged).
    const int ex = wpre + inc - s2;                  // first block of row 2 tid
    auto interior = [&](int st) {
      const unsigned v = (static_cast<unsigned>(st) * Geff + NB - 1) / NB;
      return !(v < static_cast<unsigned>(Geff) && v * NB / Geff == static_cast<unsigned>(st));
    };
    const int ch0 = nb2[0] > 0 && interior(ex), ch1 = nb2[1] > 0 && interior(ex + nb2[0]);
    const int c2 = ch0 + ch1;
    int inc_c = c2;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(inc_c, off);
      if (lane >= off) inc_c += t;
    }
    if (lane == 63) bal_wsum[8 + w] = inc_c;
    __syncthreads();
    int wpre_c = 0, NC = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int v = bal_wsum[8 + k];
      wpre_c += k < w ? v : 0;
      NC += v;
    }
    NC = __builtin_amdgcn_readfirstlane(NC);
    const int TC = U * NB + RC * NC;                 // total cost
    {
      const int ex_c = wpre_c + inc_c - c2;
      const int r0 = 2 * tid, r1 = r0 + 1;
      if (r0 < rows) {
        bal_pfx[r0] = ex;
        bal_cpfx[r0] = U * ex + RC * ex_c;
        bal_rc[r0] = RC * ch0;
      }
      if (r1 < rows) {
        bal_pfx[r1] = ex + nb2[0];
        bal_cpfx[r1] = U * (ex + nb2[0]) + RC * (ex_c + ch0);
        bal_rc[r1] = RC * ch1;
      }
      if (tid == 0) {
        bal_pfx[rows] = NB;
        bal_cpfx[rows] = TC;
      }
    }
    __syncthreads();   // prefix sums complete
    // the workgroup whose cost range [floor(w TC / Geff), floor((w+1) TC / Geff))
    // holds cost position x (32-bit products: the host bounds NB by 2^21)
    auto wg_of = [&](int x) {
      int v = static_cast<int>(static_cast<unsigned>(x) * Geff / TC);
      if (static_cast<unsigned>(v + 1) * TC / Geff <= static_cast<unsigned>(x)) ++v;
      return v;
    };
    // block j of a nonempty row r starts at cost position cpfx[r] + rc[r] + U j;
    // the workgroup's blocks are those starting inside its cost range
    // (first slot, slot count) of this workgroup's share of the rows
    {
      const int r = id * rows / G + tid;
      const int rend = (id + 1) * rows / G;
      if (r < rend) {
        const int nb = bal_pfx[r + 1] - bal_pfx[r];
        int2 m = make_int2(0, 0);
        if (nb > 0) {
          const int c0 = bal_cpfx[r] + bal_rc[r];
          const int wf = wg_of(c0), wl = wg_of(c0 + U * (nb - 1));
          m = make_int2(wf + r, wl - wf + 1);
        }
        reinterpret_cast<int2*>(a.bal_meta)[r] = m;
      }
    }
    if (id >= Geff) return;              // no blocks for this workgroup
    // first block at or after cost position cut: in the nonempty row r with
    // cpfx[r] - U < cut <= its last block start, block max(0, ceil((cut -
    // cpfx[r] - rc[r]) / U))
    const int lo_c = static_cast<int>(static_cast<unsigned>(id) * TC / Geff);
    const int hi_c = static_cast<int>(static_cast<unsigned>(id + 1) * TC / Geff);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 2 * tid + e;
      if (r < rows) {
        const int nb = bal_pfx[r + 1] - bal_pfx[r];
        const int c = bal_cpfx[r], rc = bal_rc[r];
        const int last = c + rc + U * (nb - 1);
        if (nb > 0 && c - U < lo_c && lo_c <= last) {
          const int j = lo_c <= c + rc ? 0 : (lo_c - c - rc + U - 1) / U;
          bal_wsum[16] = r;
          bal_wsum[17] = bal_pfx[r] + j;
        }
        if (nb > 0 && id + 1 < Geff && c - U < hi_c && hi_c <= last) {
          const int j = hi_c <= c + rc ? 0 : (hi_c - c - rc + U - 1) / U;
          bal_wsum[18] = bal_pfx[r] + j;
        }
      }
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(bal_wsum[16]);
    lo = __builtin_amdgcn_readfirstlane(bal_wsum[17]);
    hi = id + 1 < Geff ? __builtin_amdgcn_readfirstlane(bal_wsum[18]) : NB;
    N = hi - lo;
    hold_first = __builtin_amdgcn_readfirstlane(bal_pfx[b + 1]) < hi;
  } else {
    split = id % a.num_splits;
    b = id / a.num_splits;                                              // virtual row (q, partials, out)
    bs = b / ql;                                                        // its sequence (cache, lengths)
    const int jq = b - bs * ql;                                         // its query token
    // query token jq sees the sequence up to and including itself
    int L = ((const __attribute__((address_space(4))) int*)a.seq_lens)[bs] - (ql - 1 - jq);
    L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
    const int t0 = split * a.chunk_tokens;
    t1 = min(t0 + a.chunk_tokens, L);
    blk0 = t0 >> 6;
    N = t0 < t1 ? ((t1 + kBlockTokens - 1) >> 6) - blk0 : 0;            // blocks to walk
    nbl = (L + kBlockTokens - 1) >> 6;
    if constexpr (APP) app_p = ((const __attribute__((address_space(4))) int*)a.app.pos)[bs];
  }
  constexpr int h0 = 0;                                                 // first head
  // iterations walk units of BPI consecutive blocks (a unit's second block
  // past the walk reads nothing and is masked out)
  const int NU = (N + BPI - 1) / BPI;

  // Q rows of the workgroup's heads -> LDS in operand order: block (ht, s),
  // lane (gg, cc) holds Q[h0+ht*16+cc][qk_dim(s, gg) .. +8]. The QK waves
  // load all of it, ahead of their first K blocks, and stage it before the
  // first barrier; the PV waves issue their first V blocks only after that
  // barrier. The first requests of every compute unit are then the ones the
  // first iteration waits for (Q and K block 0), not V blocks needed two
  // iterations later.
  constexpr int kQLoads = 2 * HT;                                       // 16-byte loads per QK thread (8)
  // Q8 staging: kTPH adjacent threads share a head, each with kDPT
  // consecutive dims (so a head's amax is a reduction over kTPH lanes)
  constexpr int kTPH = 256 / kHW;
  constexpr int kDPT = kD / kTPH;
  static_assert(kDPT == 8 * kQLoads, "Q8 staging: one 16-byte load per 8 dims");
  auto q_src = [&](int row, int r) __attribute__((always_inline)) -> const uint4* {
    if constexpr (Q8) {
      return reinterpret_cast<const uint4*>(a.q + static_cast<size_t>(row) * kH * kD +
                                            (h0 + tid / kTPH) * kD + (tid % kTPH) * kDPT + 8 * r);
    }
    const int idx = tid + 256 * r;
    const int ln = idx & 63, blk = idx >> 6;
    const int ht = blk >> 3, s = blk & 7;
    const int gg = ln >> 4, cc = ln & 15;
    return reinterpret_cast<const uint4*>(a.q + static_cast<size_t>(row) * kH * kD +
                                          (h0 + ht * 16 + cc) * kD + qk_dim<FP8>(s, gg));
  };
  // Q8: this thread's kDPT bf16 values of head h0 + tid/kTPH -> e4m3 codes
  // in operand order, scale = amax/448 of the head's row (1 when 0), code =
  // RNE e4m3 of the correctly rounded quotient
  auto stage_q8 = [&](const uint4 (&qv)[8]) __attribute__((always_inline)) {
    const int hl = tid / kTPH, j = tid % kTPH;
    float x[kDPT];
#pragma unroll
    for (int r = 0; r < kQLoads; ++r) {
      const uint32_t u[4] = {qv[r].x, qv[r].y, qv[r].z, qv[r].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * r + 2 * e] = __uint_as_float(u[e] << 16);
        x[8 * r + 2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < kDPT; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
    for (int off = 1; off < kTPH; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int p = 0; p < kDPT / 16; ++p) {        // pieces of 16 codes
      uint32_t wd[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint32_t v = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) v |= encode_e4m3_rne(x[16 * p + 4 * q4 + e] / sc) << (8 * e);
        wd[q4] = v;
      }
      const int d0 = j * kDPT + 16 * p;
      const int k2 = d0 >> 7, half = (d0 >> 6) & 1, gp = (d0 >> 4) & 3;
      q_lds[((((hl >> 4) * 2 + k2) * 64) + gp * 16 + (hl & 15)) * 2 + half] =
          make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
    if (j == 0) qs_lds[hl] = sc;
  };
  // prologue of either role: the QK waves load Q, then ring blocks 0 .. R-1,
  // then stage Q; the PV waves fill their ring after the Q barrier
  auto prologue_qk = [&](auto r_c, auto&& issue, auto&& pre, auto&& mid) __attribute__((always_inline)) {
    constexpr int RR = decltype(r_c)::value;
    if (N > 0) {
      // named registers, not an array: an array held across the scheduling
      // barriers below would be left in scratch memory
      uint4 q0, q1, q2, q3, q4, q5, q6, q7;
      q0 = *q_src(b, 0); q1 = *q_src(b, 1); q2 = *q_src(b, 2); q3 = *q_src(b, 3);
      q4 = *q_src(b, 4); q5 = *q_src(b, 5); q6 = *q_src(b, 6); q7 = *q_src(b, 7);
      pre();
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, RR>([&](auto rc) {
        mid(decltype(rc)::value);
        issue(rc, decltype(rc)::value);
      });
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (Q8) {
        const uint4 qv[8] = {q0, q1, q2, q3, q4, q5, q6, q7};
        stage_q8(qv);
      } else {
        q_lds[tid] = q0; q_lds[tid + 256] = q1; q_lds[tid + 512] = q2; q_lds[tid + 768] = q3;
        q_lds[tid + 1024] = q4; q_lds[tid + 1280] = q5; q_lds[tid + 1536] = q6; q_lds[tid + 1792] = q7;
      }
    }
  };
  auto prologue_pv = [&](auto r_c, auto&& issue) __attribute__((always_inline)) {
    constexpr int RR = decltype(r_c)::value;
    if (N > 0) static_for<0, RR>([&](auto rc) { issue(rc, decltype(rc)::value); });
  };

  // Block-table reads go through the constant address space: the table is
  // read-only here, so a uniform index becomes a scalar load that does not
  // join the vector-memory counter the K/V ring waits on.
  using cint = const __attribute__((address_space(4))) int;
  cint* bt_row = a.block_table
                     ? (cint*)a.block_table + static_cast<size_t>(bs) * a.max_blocks_per_seq
                     : nullptr;
  auto phys = [&](int n) __attribute__((always_inline)) -> size_t {   // physical id of the workgroup's n-th block
    const int j = blk0 + n;
    int pid = bt_row ? bt_row[j] : bs * a.max_blocks_per_seq + j;
    pid = pid < 0 ? 0 : (pid >= a.num_blocks ? a.num_blocks - 1 : pid);
    return static_cast<size_t>(pid);
  };
  auto tokens_in = [&](int n) __attribute__((always_inline)) { return t1 - (blk0 + n) * kBlockTokens; };   // valid tokens of block n (>= 1)

  // Balanced walk: a cursor over the rows of the workgroup's range. For the
  // row r holding global block x: rb = its first global block, gs / ge = the
  // part of its blocks inside [lo, hi), L = its length, sq = its sequence.
  struct Cur {
    int r, rb, gs, ge, L, sq;
  };
  auto cur_set = [&](Cur& cu, int r) __attribute__((always_inline)) {
    cu.r = r;
    cu.rb = __builtin_amdgcn_readfirstlane(bal_pfx[r]);
    cu.ge = min(__builtin_amdgcn_readfirstlane(bal_pfx[r + 1]), hi);
    cu.gs = max(cu.rb, lo);
    cu.L = __builtin_amdgcn_readfirstlane(bal_len[r]);
    cu.sq = r / ql;
  };
  // moves the cursor forward to the row holding global block x (< hi)
  auto cur_at = [&](Cur& cu, int x) __attribute__((always_inline)) {
    while (x >= cu.ge) cur_set(cu, cu.r + 1);
  };
  auto phys_bal = [&](const Cur& cu, int x) __attribute__((always_inline)) -> size_t {
    const int j = x - cu.rb;
    int pid = a.block_table ? ((cint*)a.block_table)[static_cast<size_t>(cu.sq) * a.max_blocks_per_seq + j]
                            : cu.sq * a.max_blocks_per_seq + j;
    pid = pid < 0 ? 0 : (pid >= a.num_blocks ? a.num_blocks - 1 : pid);
    return static_cast<size_t>(pid);
  };
  auto lim_bal = [&](const Cur& cu, int x) __attribute__((always_inline)) {
    return min(kBlockTokens, cu.L - (x - cu.rb) * kBlockTokens);
  };
  auto cur_init = [&](Cur& cu) __attribute__((always_inline)) {
    if constexpr (BAL) cur_set(cu, b);
  };
  // Paged caches: physical ids of walk blocks base .. base + 63, one per lane,
  // fetched by one gather; issuing a block then takes its id with readlane
  // instead of waiting on a scalar load of the table in every iteration.
  auto bt_window = [&](int base) __attribute__((always_inline)) -> int {
    const int n = base + lane;
    int pid = 0;
    if (n < N) {
      int sq, j;
      if constexpr (BAL) {
        const int x = lo + n;
        int r = b;
        while (x >= bal_pfx[r + 1]) ++r;
        j = x - bal_pfx[r];
        sq = r / ql;
      } else {
        sq = bs;
        j = blk0 + n;
      }
      pid = a.block_table[static_cast<size_t>(sq) * a.max_blocks_per_seq + j];
      pid = pid < 0 ? 0 : (pid >= a.num_blocks ? a.num_blocks - 1 : pid);
    }
    return pid;
  };
  const bool paged = a.block_table != nullptr;

  // partial results (split or balanced) or the final output
  const bool partial = BAL || a.num_splits > 1;
  // bf16 outputs leave through LDS as whole 512-byte head rows (end of the
  // kernel); fp32 outputs and the fp32 split partials are stored directly
  const bool stage_out = !partial && !a.out_f32;

  // In-launch append (APP): f(r, p, n) for the workgroup's row when its new
  // token (position p) lies in block n of this split's walk; g(r) for the
  // row in the row's first split when the token lies in no walked block.
  constexpr int kCache = FP8 ? 2 : 1;
  auto for_owned = [&](auto&& f) __attribute__((always_inline)) {
    const int j = app_p >> 6;
    if (app_p >= 0 && j >= blk0 && j < blk0 + N) f(b, app_p, j - blk0);
  };
  auto for_orphans = [&](auto&& g) __attribute__((always_inline)) {
    if (split == 0 && app_p >= 0 && (app_p >> 6) >= nbl) g(b);
  };

  // Every wave passes the same barriers: one after staging Q, one per
  // iteration i = 0 .. NU+1 (NU units of BPI blocks), one before the epilogue (and one more before the
  // staged stores).
  if (w < 4) {
    // ================= QK waves: S = K.Q^T -> LDS, per-wave block max
    constexpr int R = RK;
    constexpr int U = unroll_for(RK);
    uint4 ring[R][BPI][C::kSlot];        // K units of 16 tokens (+ FP8 K, V scales) per block
    Cur kc, sc;                          // balanced walk: K issue and scores cursors
    cur_init(kc);
    cur_init(sc);
    int wbase = 0;                       // paged: the block-id window of the K issue
    int win = paged ? bt_window(0) : 0;
    // Loads iteration unit u (blocks BPI*u ..) into a ring slot; blocks past
    // the walk issue the same number of loads through empty resources, which
    // return zeros and read nothing, so the loop's load count is the same on
    // every path.
    auto issue = [&](auto slot_c, int u) __attribute__((always_inline)) {
      constexpr int slot = decltype(slot_c)::value;
#pragma unroll
      for (int bb = 0; bb < BPI; ++bb) {
      const int n = u * BPI + bb;
      const bool real = n < N;
      size_t pb = 0;
      if (paged) {
        if (real) {
          if (n - wbase >= kWave) {
            wbase += kWave;
            win = bt_window(wbase);
          }
          pb = static_cast<size_t>(__builtin_amdgcn_readlane(win, n - wbase));
        }
      } else if constexpr (BAL) {
        if (real) {
          cur_at(kc, lo + n);
          pb = phys_bal(kc, lo + n);
        }
      } else {
        pb = phys(real ? n : 0);
      }
      // units (tg = ww, s): K[16ww + c][..], 1 KB contiguous per load
      const auto rk = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(a.k) + pb * C::kBlockBytes, 0, real ? C::kBlockBytes : 0, kRsrcFlags);
      const int vo = (ww * C::kLoads) * 1024 + lane * 16;
      static_for<0, C::kLoads>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        ring[slot][bb][s] = buf_load16(rk, vo + s * 1024);
      });
      if constexpr (FP8) {
        const int so = (16 * ww + 4 * g) * 4;
        const int nr = real ? kBlockTokens * 4 : 0;
        const auto rks = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(a.k_scale) + pb * kBlockTokens, 0, nr, kRsrcFlags);
        const auto rvs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(a.v_scale) + pb * kBlockTokens, 0, nr, kRsrcFlags);
        ring[slot][bb][4] = buf_load16(rks, so);
        ring[slot][bb][5] = buf_load16(rvs, so);
      }
      }
    };
    // Q8: the query codes and scales of the workgroup's heads stay in
    // registers once staged (64 + HT registers), not re-read from LDS per block
    i32x8_t qreg[Q8 ? 2 * HT : 1];
    float qsr[Q8 ? HT : 1];
    // S^T of the blocks of unit u (16 tokens x kHW heads of this wave per
    // block) -> s_lds[par], the wave's per-head max over the unit -> red[par]
    // (FP8: V scales -> vs_lds[par])
    auto scores = [&](auto slot_c, auto par_c, int u) __attribute__((always_inline)) {
      constexpr int slot = decltype(slot_c)::value;
      constexpr int par = decltype(par_c)::value;
      f32x4_t s_acc[BPI][HT];
#pragma unroll
      for (int bb = 0; bb < BPI; ++bb)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) s_acc[bb][ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (Q8) {
        // two 128-deep k-steps: the K unit pair (2k2, 2k2+1) as codes
        static_for<0, 2>([&](auto kc) {
          constexpr int k2 = decltype(kc)::value;
          const uint4 u0 = ring[slot][0][2 * k2], u1 = ring[slot][0][2 * k2 + 1];
          const i32x8_t kop = {static_cast<int>(u0.x), static_cast<int>(u0.y),
                               static_cast<int>(u0.z), static_cast<int>(u0.w),
                               static_cast<int>(u1.x), static_cast<int>(u1.y),
                               static_cast<int>(u1.z), static_cast<int>(u1.w)};
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
            s_acc[0][ht] = mfma_16x16x128_e4m3(kop, qreg[Q8 ? ht * 2 + k2 : 0], s_acc[0][ht]);
        });
      }
      // bf16: the Q operands of k-step s+1 are read from LDS while step s
      // multiplies (FP8: its operand conversions fill the gaps instead)
      constexpr bool kQdb = !FP8;
      bf16x8_t qop[2][HT];
      if constexpr (kQdb) {
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) qop[0][ht] = as_bf16x8(q_lds[(ht * 8) * 64 + lane]);
      }
      if constexpr (!Q8) static_for<0, 8>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        if constexpr (kQdb && s + 1 < 8) {
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
            qop[(s + 1) & 1][ht] = as_bf16x8(q_lds[(ht * 8 + s + 1) * 64 + lane]);
          __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of this step's products
        }
        bf16x8_t kop[BPI];
#pragma unroll
        for (int bb = 0; bb < BPI; ++bb) {
          if constexpr (FP8) {
            const uint4 kw = ring[slot][bb][s >> 1];
            kop[bb] = (s & 1) ? e4m3x8_to_bf16x8(kw.z, kw.w) : e4m3x8_to_bf16x8(kw.x, kw.y);
          } else {
            kop[bb] = as_bf16x8(ring[slot][bb][s]);
          }
        }
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          // one Q operand serves every block of the unit
          const bf16x8_t qv = kQdb ? qop[s & 1][ht] : as_bf16x8(q_lds[(ht * 8 + s) * 64 + lane]);
#pragma unroll
          for (int bb = 0; bb < BPI; ++bb) s_acc[bb][ht] = mfma_16x16x32(kop[bb], qv, s_acc[bb][ht]);
        }
      });
#pragma unroll
      for (int bb = 0; bb < BPI; ++bb) {
        int lim;
        if constexpr (BAL) lim = lim_bal(sc, lo + u);
        else lim = tokens_in(u * BPI + bb);
        const int tt0 = 16 * ww + 4 * g;         // this lane's first token of the block
        if constexpr (FP8) {
          const uint4 k4 = ring[slot][bb][4];
          const float ks[4] = {__uint_as_float(k4.x), __uint_as_float(k4.y), __uint_as_float(k4.z),
                               __uint_as_float(k4.w)};
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) {
            // Q8: and the q scale of head h0 + 16ht + c
            const float qsc = Q8 ? qsr[Q8 ? ht : 0] : 1.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) s_acc[bb][ht][e] *= Q8 ? ks[e] * qsc : ks[e];
          }
          // V scales (same value from the 16 lanes of a row); the scale slots
          // of tokens past the end were never written and may hold anything
          // (a NaN would survive p = 0 in p * scale), so they become 0
          uint4 v4 = ring[slot][bb][5];
          if (lim < kBlockTokens) {
            v4.x = tt0 + 0 < lim ? v4.x : 0u;
            v4.y = tt0 + 1 < lim ? v4.y : 0u;
            v4.z = tt0 + 2 < lim ? v4.z : 0u;
            v4.w = tt0 + 3 < lim ? v4.w : 0u;
          }
          vs_lds[par][bb * 16 + ww * 4 + g] = v4;
        }
        if (lim < kBlockTokens) {        // tail block (uniform): tokens past the end -> -inf
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int e = 0; e < 4; ++e) s_acc[bb][ht][e] = (tt0 + e < lim) ? s_acc[bb][ht][e] : -INFINITY;
        }
      }
      // per-head max over the wave's 16 tokens of each block; lane row g
      // ends with the max of tile g, so one store per
      // lane covers them all
      float mt[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        mt[ht] = max_nonan(max3_nonan(s_acc[0][ht][0], s_acc[0][ht][1], s_acc[0][ht][2]), s_acc[0][ht][3]);
#pragma unroll
        for (int bb = 1; bb < BPI; ++bb)
          mt[ht] = max_nonan(mt[ht], max_nonan(max3_nonan(s_acc[bb][ht][0], s_acc[bb][ht][1],
                                                          s_acc[bb][ht][2]), s_acc[bb][ht][3]));
#pragma unroll
        for (int bb = 0; bb < BPI; ++bb) s_lds[par][((bb * 4 + ww) * HT + ht) * 64 + lane] = s_acc[bb][ht];
      }
      red[par][(g * 16 + c) * 4 + ww] = rows4_max_t4(mt[0], mt[1], mt[2], mt[3]);
    };

    // APP: the new token, when this wave loads its K row (token rows 16ww ..
    // 16ww+15 of the block). Its K, V and table entry are read together
    // with Q, as raw words (any use of them before the ring loads would hold
    // those behind their latency); the table entry by a scalar load (a
    // vector one would be waited for at once to move the uniform value into
    // a scalar register). The wave stores K before it issues the ring unit
    // holding the token.
    auto own_k = [&](auto&& f) __attribute__((always_inline)) {
      for_owned([&](int r, int p, int n) {
        if (((p & 63) >> 4) == ww) f(r, p, n);
      });
    };
    uint2 akw = make_uint2(0u, 0u), avw = make_uint2(0u, 0u);
    int a_r = -1, a_u = 0, a_p = 0, a_tab = 0;
    bool a_done = true;
    auto app_pre = [&]() __attribute__((always_inline)) {
      if constexpr (APP) {
        int n0 = 0;
        own_k([&](int r, int p, int n) {
          a_r = r;
          a_p = p;
          n0 = n;
        });
        // issued whether or not the wave owns a token (row 0 then): no branch
        a_done = a_r < 0;
        a_u = n0 / BPI;
        const int rr = a_r >= 0 ? a_r : 0;
        const size_t i = static_cast<size_t>(rr) * kD + 4 * lane;
        akw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.app.k_new) + i);
        avw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.app.v_new) + i);
        // an owner walks the token's block, so (a_p >> 6) is a block of the
        // table row; a contiguous cache needs no entry (pos[0] is read instead)
        const int* tp = a.app.block_table
                            ? a.app.block_table + static_cast<size_t>(rr) * a.app.max_blocks_per_seq +
                                  (a_r >= 0 ? (a_p >> 6) : 0)
                            : a.app.pos;
        a_tab = *(const __attribute__((address_space(4))) int*)tp;
      }
    };
    // the token: K (FP8: codes and both scales) to the cache; V, its slot
    // and its FP8 scale to the hand-off slot (the PV waves store V)
    auto app_store = [&]() __attribute__((always_inline)) {
      if constexpr (APP) {
        {
          const int r = a_r, p = a_p;
          RowPiece<4, false> rk, rv;
          rk.w[0] = akw.x; rk.w[1] = akw.y;
          rv.w[0] = avw.x; rv.w[1] = avw.y;
          const TokenSlot ts =
              token_slot_of(a.app, a.app.block_table ? a_tab : r * a.app.max_blocks_per_seq + (p >> 6), p);
          float sv = 1.f;
          if (ts.id >= 0) {
            float xk[4];
            row_piece_f32(rk, xk);
            float sk = 1.f;
            if constexpr (FP8) {
              float xv[4];
              row_piece_f32(rv, xv);
              sk = token_scale(xk);
              sv = token_scale(xv);
              if (lane == 0) {
                a.app.k_scale[static_cast<size_t>(ts.id) * kBlockTokens + ts.off] = sk;
                a.app.v_scale[static_cast<size_t>(ts.id) * kBlockTokens + ts.off] = sv;
              }
            }
            store_token_k<kCache, 4>(a.app, ts, xk, sk, lane);
          }
          if (lane == 0) {
            app_lds[0] = static_cast<uint32_t>(ts.id);
            app_lds[1] = static_cast<uint32_t>(ts.off);
            app_lds[2] = __float_as_uint(sv);
          }
          app_lds[4 + 2 * lane] = rv.w[0];
          app_lds[5 + 2 * lane] = rv.w[1];
        }
        a_done = true;
      }
    };
    auto app_mid = [&](int u) __attribute__((always_inline)) {
      if constexpr (APP) {
        if (!a_done && u == a_u) app_store();
      }
    };

    // Every iteration issues the same loads (empty ones past the walk), so
    // every path into a consumer has the same loads in flight and the wait
    // before it leaves R-1 blocks outstanding.
    prologue_qk(std::integral_constant<int, R>{}, issue, app_pre, app_mid);
    if constexpr (APP) {
      if (!a_done) app_store();          // the token's unit is issued after the prologue
    }
    __syncthreads();   // Q staged
    if constexpr (Q8) {
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int qi = ((ht * 2 + k2) * 64 + lane) * 2;
          const uint4 qa = q_lds[qi], qb = q_lds[qi + 1];
          qreg[ht * 2 + k2] = i32x8_t{static_cast<int>(qa.x), static_cast<int>(qa.y),
                                      static_cast<int>(qa.z), static_cast<int>(qa.w),
                                      static_cast<int>(qb.x), static_cast<int>(qb.y),
                                      static_cast<int>(qb.z), static_cast<int>(qb.w)};
        }
        qsr[ht] = qs_lds[16 * ht + c];
      }
    }
    // balanced walk: Q of the next piece, in registers until its first block
    uint4 qn0, qn1, qn2, qn3, qn4, qn5, qn6, qn7;
    // before S of unit i: at the first block of a piece after the first, Q
    // of the piece goes to LDS (every QK wave has finished reading the old Q
    // at the previous barrier) behind the extra barrier both roles pass.
    // Returns whether unit i starts a piece.
    auto piece_start = [&](int i) __attribute__((always_inline)) -> bool {
      if constexpr (BAL) {
        cur_at(sc, lo + i);
        const bool first = lo + i == sc.gs;
        if (first && i > 0) {
          q_lds[tid] = qn0; q_lds[tid + 256] = qn1; q_lds[tid + 512] = qn2; q_lds[tid + 768] = qn3;
          q_lds[tid + 1024] = qn4; q_lds[tid + 1280] = qn5; q_lds[tid + 1536] = qn6;
          q_lds[tid + 1792] = qn7;
          __syncthreads();
        }
        return first;
      }
      return false;
    };
    // after S of the first unit of a piece, before the ring loads: Q of the
    // piece after it (if any) into registers
    auto prefetch_q = [&](bool first) __attribute__((always_inline)) {
      if constexpr (BAL) {
        if (first && sc.ge < hi) {
          Cur nc = sc;
          cur_at(nc, sc.ge);
          qn0 = *q_src(nc.r, 0); qn1 = *q_src(nc.r, 1); qn2 = *q_src(nc.r, 2); qn3 = *q_src(nc.r, 3);
          qn4 = *q_src(nc.r, 4); qn5 = *q_src(nc.r, 5); qn6 = *q_src(nc.r, 6); qn7 = *q_src(nc.r, 7);
        }
      }
    };
    // iterations i = 0 .. NU+1, S(unit i) for i < NU; groups of U keep ring slots
    // and parities static (i = base + r, base a multiple of U)
    int base = 0;
    for (; base + U <= NU; base += U) {
      static_for<0, U>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        constexpr int slot = r % R, par = r & 1;
        const int i = base + r;
        const bool first = piece_start(i);
        scores(std::integral_constant<int, slot>{}, std::integral_constant<int, par>{}, i);
        prefetch_q(first);
        issue(std::integral_constant<int, slot>{}, i + R);
        __syncthreads();
      });
    }
    // the rest: i = base .. NU+1 (at most U+1 iterations)
    static_for<0, U + 1>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      constexpr int slot = r % R, par = r & 1;
      const int i = base + r;
      if (i <= NU + 1) {
        if (i < NU) {
          const bool first = piece_start(i);
          scores(std::integral_constant<int, slot>{}, std::integral_constant<int, par>{}, i);
          prefetch_q(first);
          issue(std::integral_constant<int, slot>{}, i + R);
        }
        __syncthreads();
      }
    });
    __syncthreads();   // row sums staged (by the PV waves)
    // balanced walk: the held first piece leaves LDS as whole 1 KB head rows
    // while the PV waves store the last piece. Written out inside the walk,
    // these stores slowed every workgroup's reads.
    if (BAL && hold_first) {
      float* dst = a.part_o + static_cast<size_t>(id + b) * kH * kD;
#pragma unroll 4
      for (int k = 0; k < kHW / 4; ++k) {
        const int h = 4 * k + w;
        *reinterpret_cast<float4*>(dst + h * kD + 4 * lane) = bal_hold[h * 65 + lane];
      }
    }
  } else {
    // ================= PV waves: online softmax, O^T += V^T . P^T
    constexpr int R = RV;
    constexpr int U = unroll_for(RV);
    const float cl2 = a.scale_log2;      // > 0
    // acc[dt][ht]: lane holds O^T[64ww + 16dt + 4g + i][16ht + c]
    f32x4_t acc[4][HT];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc[dt][ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // running max per head h0 + 16ht + c (log2 units of scaled logits; the
    // same in every PV wave) and this wave's partial row sums over the
    // tokens of its softmax share
    float m_run[HT], l_run[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) { m_run[ht] = -INFINITY; l_run[ht] = 0.f; }
    uint4 ring[R][BPI][C::kLoads];
    Cur vc, bc, pc;        // balanced walk: V issue, piece-start and P.V cursors
    cur_init(vc);
    cur_init(bc);
    cur_init(pc);
    int wbase = 0;         // paged: the block-id window of the V issue
    int win = paged ? bt_window(0) : 0;
    auto issue = [&](auto slot_c, int u) __attribute__((always_inline)) {   // as for K
      constexpr int slot = decltype(slot_c)::value;
#pragma unroll
      for (int bb = 0; bb < BPI; ++bb) {
        const int n = u * BPI + bb;
        const bool real = n < N;
        size_t pb = 0;
        if (paged) {
          if (real) {
            if (n - wbase >= kWave) {
              wbase += kWave;
              win = bt_window(wbase);
            }
            pb = static_cast<size_t>(__builtin_amdgcn_readlane(win, n - wbase));
          }
        } else if constexpr (BAL) {
          if (real) {
            cur_at(vc, lo + n);
            pb = phys_bal(vc, lo + n);
          }
        } else {
          pb = phys(real ? n : 0);
        }
        // bf16 units (fg = 4ww + s/2, ks = s%2); FP8 units fg = 4ww + s
        const auto rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(a.v) + pb * C::kBlockBytes, 0, real ? C::kBlockBytes : 0, kRsrcFlags);
        const int vo = (ww * C::kLoads) * 1024 + lane * 16;
        static_for<0, C::kLoads>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          ring[slot][bb][s] = buf_load16(rv, vo + s * 1024);
        });
      }
    };
    auto pv = [&](auto slot_c, auto par_c, int u) __attribute__((always_inline)) {
      constexpr int slot = decltype(slot_c)::value;
      constexpr int par = decltype(par_c)::value;
#pragma unroll
      for (int bb = 0; bb < BPI; ++bb) {
      int lim;
      if constexpr (BAL) {
        cur_at(pc, lo + u);
        lim = lim_bal(pc, lo + u);
      } else {
        lim = tokens_in(u * BPI + bb);
      }
      if (lim < kBlockTokens) {
        // tokens past the end: zero their V so 0 * (stale data) cannot reach O
        static_for<0, C::kLoads>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          uint4 u = ring[slot][bb][s];
          if constexpr (FP8) {
            uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              uint32_t msk = 0;
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (g * 16 + q4 * 4 + e < lim) msk |= 0xffu << (8 * e);
              wd[q4] &= msk;
            }
            u = make_uint4(wd[0], wd[1], wd[2], wd[3]);
          } else {
            const int tb = (s & 1) * 32 + g * 8;      // unit (dt = s/2, ks = s%2)
            u.x = keep_bf16(u.x, tb + 0 < lim, tb + 1 < lim);
            u.y = keep_bf16(u.y, tb + 2 < lim, tb + 3 < lim);
            u.z = keep_bf16(u.z, tb + 4 < lim, tb + 5 < lim);
            u.w = keep_bf16(u.w, tb + 6 < lim, tb + 7 < lim);
          }
          ring[slot][bb][s] = u;
        });
      }
      static_for<0, 2>([&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        bf16x8_t pop[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          pop[ht] = as_bf16x8(p_lds[par][bb * HT * 2 * 64 + (ht * 2 + ks) * 64 + lane]);
        static_for<0, 4>([&](auto dtc) {
          constexpr int dt = decltype(dtc)::value;
          bf16x8_t vop;
          if constexpr (FP8) {
            const uint4 vw = ring[slot][bb][dt];
            vop = ks ? e4m3x8_to_bf16x8(vw.z, vw.w) : e4m3x8_to_bf16x8(vw.x, vw.y);
          } else {
            vop = as_bf16x8(ring[slot][bb][dt * 2 + ks]);
          }
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) acc[dt][ht] = mfma_16x16x32(vop, pop[ht], acc[dt][ht]);
        });
      });
      }
    };

    // softmax of one unit for this wave's 16 tokens per block (those QK wave
    // ww scored): unit max from all four QK waves, lazy update of the running
    // max (O rescaled here, so the next products add to a consistent sum),
    // P^T (bf16, FP8: times the V scales) -> p_lds[par]
    auto softmax = [&](auto par_c) __attribute__((always_inline)) {
      constexpr int par = decltype(par_c)::value;
      float4 r4[HT];
      f32x4_t sv[BPI][HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        r4[ht] = reinterpret_cast<const float4*>(red[par])[ht * 16 + c];
#pragma unroll
        for (int bb = 0; bb < BPI; ++bb) sv[bb][ht] = s_lds[par][((bb * 4 + ww) * HT + ht) * 64 + lane];
      }
      float vs[BPI][4];
#pragma unroll
      for (int bb = 0; bb < BPI; ++bb) {
        vs[bb][0] = vs[bb][1] = vs[bb][2] = vs[bb][3] = 1.f;
        if constexpr (FP8) {
          const uint4 v4 = vs_lds[par][bb * 16 + ww * 4 + g];
          vs[bb][0] = __uint_as_float(v4.x); vs[bb][1] = __uint_as_float(v4.y);
          vs[bb][2] = __uint_as_float(v4.z); vs[bb][3] = __uint_as_float(v4.w);
        }
      }
      bool rescale = false;
      float alpha[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        // max over the unit's tokens (finite: every walked unit has a valid token)
        const float tz = max_nonan(max3_nonan(r4[ht].x, r4[ht].y, r4[ht].z), r4[ht].w) * cl2;
        alpha[ht] = 1.0f;
        if (tz > m_run[ht] + kLazy) {          // also true for the first unit
          alpha[ht] = __builtin_amdgcn_exp2f(m_run[ht] - tz);
          m_run[ht] = tz;
          rescale = true;
        }
        const float nm = -m_run[ht];
        float lsum = 0.f;
#pragma unroll
        for (int bb = 0; bb < BPI; ++bb) {
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[bb][ht][e], cl2, nm));
          lsum += (p[0] + p[1]) + (p[2] + p[3]);
          if constexpr (FP8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) p[e] *= vs[bb][e];
          }
          // P^T into operand block (ht, ks) of block bb of buffer par
          int ks, gr;
          if constexpr (FP8) { ks = g >> 1; gr = ww; }
          else { ks = ww >> 1; gr = 2 * (ww & 1) + (g >> 1); }
          uint2 pk;
          pk.x = pack_bf16x2(p[0], p[1]);
          pk.y = pack_bf16x2(p[2], p[3]);
          uint8_t* dst = reinterpret_cast<uint8_t*>(p_lds[par] + bb * HT * 2 * 64) +
                         ((ht * 2 + ks) * 64 + gr * 16 + c) * 16 + (g & 1) * 8;
          *reinterpret_cast<uint2*>(dst) = pk;
        }
        l_run[ht] = l_run[ht] * alpha[ht] + lsum;
      }
      if (__ballot(rescale) != 0ull) {   // uniform: every PV wave takes the same branch
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) acc[dt][ht] *= alpha[ht];
      }
    };

    // balanced walk: a piece that ends inside the walk is written out after
    // its last P.V: o from the accumulators (fp32, unnormalised), this wave's
    // row-sum share to lred2[parity]; wave 4 writes (m, l) in the next
    // iteration, after the barrier, from the four shares and the saved max
    float m_done[HT];
    bool ml_pending = false;
    int ml_slot = 0, ml_par = 0, piece_par = 0;
    auto finish_piece = [&](int row) __attribute__((always_inline)) {
      const size_t slot = static_cast<size_t>(id + row);
      if (row == b) {                     // the first piece waits in LDS (QK waves store it)
        float4* hb = bal_hold + c * 65 + 16 * ww + g;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const f32x4_t v = acc[dt][ht];
            hb[16 * 65 * ht + 4 * dt] = make_float4(v[0], v[1], v[2], v[3]);
          }
      } else {
        float* pb = a.part_o + (slot * kH + c) * kD + 64 * ww + 4 * g;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const f32x4_t v = acc[dt][ht];
            *reinterpret_cast<float4*>(pb + 16 * ht * kD + 16 * dt) = make_float4(v[0], v[1], v[2], v[3]);
          }
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[dt][ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const float l = rows4_sum(l_run[ht]);
        if (g == 0) lred2[piece_par][(ht * 16 + c) * 4 + ww] = l;
        m_done[ht] = m_run[ht];
        m_run[ht] = -INFINITY;
        l_run[ht] = 0.f;
      }
      ml_pending = true;
      ml_slot = static_cast<int>(slot);
      ml_par = piece_par;
      piece_par ^= 1;
    };
    auto write_pending_ml = [&]() __attribute__((always_inline)) {
      if (ml_pending) {
        if (ww == 0 && g == 0) {
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) {
            const float4 r4 = reinterpret_cast<const float4*>(lred2[ml_par])[ht * 16 + c];
            float2 ml;
            ml.x = m_done[ht] * kLn2;
            ml.y = (r4.x + r4.y) + (r4.z + r4.w);
            store_nt(a.part_ml + (static_cast<size_t>(ml_slot) * kH + 16 * ht + c) * 2, ml);
          }
        }
        ml_pending = false;
      }
    };
    // the extra barrier of iteration i when unit i starts a piece (i > 0)
    auto piece_barrier = [&](int i) __attribute__((always_inline)) {
      if constexpr (BAL) {
        if (i < NU) {
          cur_at(bc, lo + i);
          if (lo + i == bc.gs) __syncthreads();
        }
      }
    };
    // P.V of unit n done: finish its piece if the walk goes on past it
    auto after_pv = [&](int n) __attribute__((always_inline)) {
      if constexpr (BAL) {
        if (n + 1 < NU && lo + n == pc.ge - 1) finish_piece(pc.r);
      }
    };

    __syncthreads();   // Q staged
    if constexpr (APP) {
      // V features 64ww .. 64ww+63 of the workgroup's new token (this
      // wave's own V columns), from the hand-off slot, stored before this
      // wave's first V loads. A token in no walked block is written whole by
      // wave 4 (nothing in the launch reads it).
      for_owned([&](int, int, int) {
        float xv[4];
        TokenSlot ts;
        ts.id = static_cast<int>(app_lds[0]);
        ts.off = static_cast<int>(app_lds[1]);
        const float sv = __uint_as_float(app_lds[2]);
        RowPiece<4, false> rv;
        rv.w[0] = app_lds[4 + 2 * lane];
        rv.w[1] = app_lds[5 + 2 * lane];
        row_piece_f32(rv, xv);
        if (ts.id >= 0 && (lane >> 4) == ww) store_token_v<kCache, 4>(a.app, ts, xv, sv, lane);
      });
      if (ww == 0) for_orphans([&](int r) { append_token_plain<kCache, 4, false>(a.app, r, lane); });
    }
    prologue_pv(std::integral_constant<int, R>{}, issue);
    __syncthreads();   // iteration 0 (S of unit 0 on the QK waves)
    piece_barrier(1);
    if (NU > 0) softmax(std::integral_constant<int, 0>{});
    __syncthreads();   // iteration 1
    // iteration n + 2: P.V of unit n, then the softmax of unit n + 1
    int nb = 0;
    for (; nb + U <= NU; nb += U) {
      static_for<0, U>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        constexpr int slot = r % R, par = r & 1;
        const int n = nb + r;
        if constexpr (BAL) {
          write_pending_ml();
          piece_barrier(n + 2);
        }
        pv(std::integral_constant<int, slot>{}, std::integral_constant<int, par>{}, n);
        issue(std::integral_constant<int, slot>{}, n + R);
        after_pv(n);
        if (n + 1 < NU) softmax(std::integral_constant<int, par ^ 1>{});
        __syncthreads();
      });
    }
    static_for<0, U>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      constexpr int slot = r % R, par = r & 1;
      const int n = nb + r;
      if (n < NU) {
        if constexpr (BAL) {
          write_pending_ml();
          piece_barrier(n + 2);
        }
        pv(std::integral_constant<int, slot>{}, std::integral_constant<int, par>{}, n);
        issue(std::integral_constant<int, slot>{}, n + R);
        after_pv(n);
        if (n + 1 < NU) softmax(std::integral_constant<int, par ^ 1>{});
        __syncthreads();
      }
    });

    // row sums: this wave's share -> LDS, then the total over the four
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const float l = rows4_sum(l_run[ht]);
      if (g == 0) lred[(ht * 16 + c) * 4 + ww] = l;
    }
    __syncthreads();   // row sums staged
    float lsum[HT], mh[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const float4 r4 = reinterpret_cast<const float4*>(lred)[ht * 16 + c];
      lsum[ht] = (r4.x + r4.y) + (r4.z + r4.w);
      mh[ht] = m_run[ht];
    }
    // O^T lane (g, c) of tile (dt, ht): head 16ht + c, features 64ww + 16dt +
    // 4g .. +3. bf16 results go to LDS (the logits buffer, free now) as head
    // rows of 32 16-byte chunks, chunk j of row hl at j ^ (hl & 31) (the 16
    // heads of a store land in 16 different bank groups); fp32 results are
    // stored directly and merge in L2.
    uint2* stage2 = reinterpret_cast<uint2*>(&s_lds[0][0]);
    const bool has_o = !partial || N > 0;   // an empty split writes only (m, l)
    // the partial slot: (row, split), or (workgroup + row of the last piece)
    const size_t row = BAL ? static_cast<size_t>(id + pc.r)
                           : static_cast<size_t>(b) * a.num_splits + split;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const float inv = !partial ? (lsum[ht] > 0.f ? 1.0f / lsum[ht] : 0.f) : 1.0f;
      const int hl = ht * 16 + c, head = h0 + hl;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        if (!has_o) break;
        const f32x4_t v = acc[dt][ht] * inv;
        if (stage_out) {
          const int j = 8 * ww + 2 * dt + (g >> 1);
          uint2 pk;
          pk.x = pack_bf16x2(v[0], v[1]);
          pk.y = pack_bf16x2(v[2], v[3]);
          stage2[(hl * 32 + (j ^ (hl & 31))) * 2 + (g & 1)] = pk;
        } else {
          const int f = 64 * ww + 16 * dt + 4 * g;
          float* dst = !partial
                           ? reinterpret_cast<float*>(a.out) + (static_cast<size_t>(b) * kH + head) * kD + f
                           : a.part_o + (row * kH + head) * kD + f;
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
      // (m, l) of every split, empty ones as (-inf, 0): the combine gives
      // those no weight and never uses their o
      if (partial && ww == 0 && g == 0) {
        float2 ml;
        ml.x = mh[ht] * kLn2;     // natural-log units of the scaled logits
        ml.y = lsum[ht];
        store_nt(a.part_ml + (row * kH + head) * 2, ml);
      }
    }
  }
  if (stage_out) {
    __syncthreads();   // head rows staged by the PV waves
    // the workgroup's kHW head rows are one contiguous range of the output:
    // 16 bytes per thread per pass
    uint16_t* dst = static_cast<uint16_t*>(a.out) + (static_cast<size_t>(b) * kH + h0) * kD;
    const uint4* stage4 = reinterpret_cast<const uint4*>(&s_lds[0][0]);
#pragma unroll
    for (int i = tid; i < kHW * 32; i += 512) {
      const int hl = i >> 5, j = i & 31;
      store_nt(dst + static_cast<size_t>(i) * 8, stage4[hl * 32 + (j ^ (hl & 31))]);
    }
  }
}

hipError_t launch_decode_mfma(const AttnArgs& a, bool fp8, int B, hipStream_t stream,
                              const AppendArgs* app) {
  if (app && (a.num_splits == 0 || a.q_len != 1 || a.fp8_queries || app->in_f32 || app->n_new != 1 ||
              app->kv_part || app->d != kD))
    return hipErrorInvalidValue;
  AttnAppArgs aa;
  static_cast<AttnArgs&>(aa) = a;
  if (app) aa.app = *app;
  if (a.num_splits == 0) {
    // balanced partition: one workgroup per compute unit
    const dim3 grid(kBalancedWorkgroups), block(512);
    if (fp8)
      hipLaunchKernelGGL((mfa_decode_mfma_kernel<true, 4, 4, false, 1, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((mfa_decode_mfma_kernel<false, 3, 2, false, 1, true>), grid, block, 0, stream, a);
    return hipGetLastError();
  }
  // one workgroup of 64 heads per (row, split); short plans already walk
  // each split as two halves (the host doubles the split count)
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(B) * a.num_splits)), block(512);
  if (fp8 && a.fp8_queries) {
    hipLaunchKernelGGL((mfa_decode_mfma_kernel<true, 4, 4, true>), grid, block, 0, stream, a);
  } else if (fp8) {
    // two 32 KB FP8 blocks per iteration: the same bytes between barriers as one bf16 block
    if (app)
      hipLaunchKernelGGL((mfa_decode_mfma_kernel<true, 2, 2, false, 2, false, true>), grid, block, 0, stream, aa);
    else
      hipLaunchKernelGGL((mfa_decode_mfma_kernel<true, 2, 2, false, 2>), grid, block, 0, stream, a);
  } else {
    // five K blocks in flight: 4K attention 28.0-28.3 -> 27.3-27.7 us (64K unchanged)
    if (app)
      hipLaunchKernelGGL((mfa_decode_mfma_kernel<false, 5, 2, false, 1, false, true>), grid, block, 0, stream, aa);
    else
      hipLaunchKernelGGL((mfa_decode_mfma_kernel<false, 5, 2>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mfa
