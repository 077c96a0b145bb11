// Exact tiled attention forward, bf16 storage, bf16 matrix cores with fp32
// accumulation (gfx950).
//
// Method ("LLM Architecture Refresh [3]: Flash Attention Is Exact", section 4
// "Tiled attention in 40 lines", with section 2's running statistics and
// section 7's causal tile skipping; "How FlashAttention Uses Tiling", update
// equations under "The Running Statistics"): for one query block, stream the
// key/value tiles through on-chip memory; per tile compute the scores, keep a
// running reference m per row, rebase the running sum l and the unnormalised
// output by exp(m_old - m_new) whenever m moves, add the tile's
// exp(s - m) and p.V, and divide by l once at the end.  Tiles whose first key
// lies after the block's last query are never loaded.  The N x N scores
// never leave registers.
//
// Mapping onto CDNA4:
//   * a workgroup of W waves owns W*32 query rows; each wave keeps its Q
//     fragments, fp32 output accumulators and m, l in VGPRs (at most 256 per
//     lane, so two waves share each SIMD and one wave's softmax and LDS waits
//     can overlap the other's matrix-core work).  The BLOCKS parameter also
//     builds 64-row waves (two 32-row blocks, one wave per SIMD), a shape that
//     measured slower and is not launched;
//   * 64-key tiles of K are copied global -> LDS by the buffer unit
//     (buffer_load_dwordx4 ... lds, 16 bytes per lane, no VGPR staging) into
//     rows padded by 16 bytes (the copy points pad slots past the end of the
//     buffer); V tiles are loaded into registers one tile ahead and stored
//     transposed.  Rows past N read as zero.  Tiles are double-buffered with
//     one barrier per tile;
//   * the scores are computed transposed, S^T = K Q^T, so each lane owns one
//     query row and the score accumulator becomes the P^T operand of
//     O^T += V^T P^T without leaving registers.  Every K and V^T operand is a
//     single conflict-free ds_read_b128 at a base register plus an immediate
//     (a transpose read would need two instructions per operand, which
//     measured slower);
//   * the running reference is raised lazily (see softmax_block), so the
//     common path has no cross-lane reduction and never touches O;
//   * exponentials are base 2 with scale*log2(e) folded into one FMA; the
//     scale is never applied to Q in bf16;
//   * heavy causal query blocks are dispatched first.
#include "common.hpp"
#include "launch.hpp"

namespace fattn {
namespace {

constexpr int kBN = 64;   // keys per tile

#ifdef FATTN_DEVICE_COUNTERS
// Debug build only: per-launch totals of the bf16 forward, summed over waves
// (a tile is one wave's 32 query rows against one 64-key tile):
//   [0] tiles computed, [1] tiles skipped (key tiles of the sequence a row
//   block never computes), [2] computed tiles that needed masking,
//   [3] reference raises (a row block's running max moved after its first
//   tile, rebasing l and O).
__device__ unsigned long long g_fwd_counters[4];
#endif
constexpr float kNegInf = -__builtin_inff();
// How far (log2 units) a row max may exceed the running reference before the
// accumulator is rebased.  Terms stay below 2^48, so sums over N <= 2^31 keys
// of p * v remain finite in fp32 for any |v| < 2^48; on inputs with rare,
// much larger keys (1% of rows x8) a rebase after the first tile is then
// almost never needed.
constexpr float kSlack = 48.f;
constexpr float kSlackSum = 281474976710656.f;   // 2^kSlack
static_assert(kSlackSum == static_cast<float>(1ull << static_cast<int>(kSlack)), "2^kSlack");

template <int D>
struct Tile {
  static constexpr int kRowBytes = 2 * D;                // one bf16 row in global memory
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
  // K rows in LDS are padded by one 16-byte slot, so 16 consecutive rows read
  // with ds_read_b128 start 4 banks apart and never collide.  V is stored
  // transposed (d-major, one row per column of V, keys permuted to match the
  // score layout) with rows of 64 keys padded by 16 bytes (36 banks apart).
  static constexpr int kKSlots = kChunks + 1;            // 16-byte slots per K row in LDS
  static constexpr int kKStride = 16 * kKSlots;          // bytes
  static constexpr int kVtStride = 2 * kBN + 16;         // bytes per V^T row
  static constexpr int kKTile = kBN * kKStride;
  static constexpr int kVTile = D * kVtStride;
  static constexpr int kKCopies = kBN * kKSlots / 64;    // wave-wide copy instructions per K tile
  static constexpr int kVBlocks = (kBN / 4) * (D / 8);   // 4-key x 8-column V blocks per tile
  static constexpr int kKSteps = D / 16;                 // contraction steps of S^T over d
  static constexpr int kDBlocks = D / 32;                // 32-row blocks of O^T
  static_assert((kBN * kKSlots) % 64 == 0, "whole copy instructions");
};

// Ask the scheduler to keep LDS operand reads kLead matrix-core steps ahead of
// their use in a region of n (read, MFMA) pairs: with two waves per SIMD the
// LDS latency is otherwise exposed on almost every step.
template <int n, int kLead = 4>
__device__ __forceinline__ void interleave_reads_and_mfma() {
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  __builtin_amdgcn_sched_group_barrier(kDsRead, kLead, 0);
#pragma unroll
  for (int i = 0; i < n - kLead; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMfma, kLead, 0);
}

// LOCAL (which implies CAUSAL): query i sees keys i - window + 1 .. i only;
// key tiles older than every row of the workgroup are never loaded.
// SPLIT > 1 (short sequences): the waves form SPLIT groups that take turns
// over the key tiles (group sp takes tiles sp, sp + SPLIT, ...), each with its
// own running statistics; the groups' partial results over disjoint key sets
// are merged at the end by the rebase identity.  The serial chain of key
// tiles per workgroup is SPLIT times shorter.
template <int D, bool CAUSAL, bool LOCAL, int WAVES, int BLOCKS, int SPLIT = 1>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int B, int H, int Hkv, int N, float c, int neg_q, int n_qblocks, int window, int hp) {
  static_assert(CAUSAL || !LOCAL, "local attention is causal");
  static_assert(SPLIT == 1 || (!LOCAL && BLOCKS == 1), "key split: plain attention, 32-row waves");
  using T = Tile<D>;
  constexpr int kRowsPerWave = 32 * BLOCKS;
  // [buffer][K tile | V tile]
  constexpr int kStage = T::kKTile + T::kVTile;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * SPLIT * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int kSplitWaves = WAVES / SPLIT;            // waves per key-split group
  const int sp = SPLIT > 1 ? wave / kSplitWaves : 0;    // this wave's group
  const int wl = SPLIT > 1 ? wave - sp * kSplitWaves : wave;   // wave within the group
  const int tid_l = SPLIT > 1 ? tid - 64 * kSplitWaves * sp : tid;
  const int col = lane & 31;
  const int grp = lane >> 5;

  // ---- work item: hp query heads that share one kv head, the same block of
  // rows_h query rows in each; heavy causal query blocks first.  All waves of
  // the workgroup then see the same causal extent, and one K/V tile serves
  // every head of the group.
  const int wph = kSplitWaves / hp;              // waves per query head
  const int rows_h = wph * kRowsPerWave;         // query rows per head
  const int rep = H / Hkv;
  const int n_groups = B * Hkv * (rep / hp);
  const int item_q = blockIdx.x / n_groups;
  const int grp_id = blockIdx.x - item_q * n_groups;
  const int qb = CAUSAL ? (n_qblocks - 1 - item_q) : item_q;
  const int bg = grp_id / (rep / hp);
  const int hs = grp_id - bg * (rep / hp);
  const int b = bg / Hkv;
  const int g = bg - b * Hkv;
  const int h = g * rep + hs * hp + wl / wph;    // this wave's query head
  const int q0 = qb * rows_h;

  const size_t head_q = ((size_t)b * H + h) * N;
  const size_t head_kv = ((size_t)b * Hkv + g) * N;
  const uint16_t* Qh = Q + head_q * D;
  const i32x4_t k_rsrc = make_buffer_rsrc(K + head_kv * D, (uint32_t)N * T::kRowBytes);
  const i32x4_t v_rsrc = make_buffer_rsrc(V + head_kv * D, (uint32_t)N * T::kRowBytes);

  const int wq_first = q0 + (wl % wph) * kRowsPerWave;   // this wave's first query row
  int qi[BLOCKS];
#pragma unroll
  for (int hf = 0; hf < BLOCKS; ++hf) qi[hf] = wq_first + 32 * hf + col;

  // ---- Q fragments (B operands of S^T), one set per 32-row block ------------
  u32x4_t qf[BLOCKS][T::kKSteps];
  {
    const uint32_t flip = neg_q ? 0x80008000u : 0u;   // exact sign flip for scale < 0
#pragma unroll
    for (int hf = 0; hf < BLOCKS; ++hf) {
      const bool ok = qi[hf] < N;
      const uint16_t* qrow = Qh + (size_t)(ok ? qi[hf] : 0) * D + 8 * grp;
#pragma unroll
      for (int s = 0; s < T::kKSteps; ++s) {
        u32x4_t x = ok ? *reinterpret_cast<const u32x4_t*>(qrow + 16 * s) : u32x4_t{0, 0, 0, 0};
        qf[hf][s] = x ^ flip;
      }
    }
  }

  const int q_hi = min(q0 + rows_h, N);
  int n_kt = (N + kBN - 1) / kBN;
  if (CAUSAL) n_kt = min(n_kt, (q_hi - 1) / kBN + 1);
  // first tile holding a key that the block's first query still sees
  const int kt_begin = LOCAL ? max(0, q0 - window + 1) / kBN : 0;

  // ---- tile copy: wave-wide instruction j fills LDS slots 64j .. 64j+63 ------
  // (lane order).  Slot -> (row, chunk) of the padded layout; pad slots and rows
  // past N are pointed past the end of the buffer and read as zero.
  const uint32_t kv_bytes = (uint32_t)N * T::kRowBytes;
  auto copy_offset = [&](int slot, int slots_per_row) {
    const int row = slot / slots_per_row;
    const int chunk = slot - row * slots_per_row;
    return chunk < T::kChunks ? row * T::kRowBytes + 16 * chunk : -1;
  };
  // Per-lane offsets of this wave's copy slots within a tile, fixed for the
  // whole loop; pad slots get 2^31, which with any tile base below 2^31 lands
  // past the buffer's range and reads as zero (no per-copy select).
  constexpr int kKCopiesPerWave = (T::kKCopies + kSplitWaves - 1) / kSplitWaves;
  uint32_t k_off[kKCopiesPerWave];
#pragma unroll
  for (int i = 0; i < kKCopiesPerWave; ++i) {
    const int off = copy_offset(64 * (kSplitWaves * i + wl) + lane, T::kKSlots);
    k_off[i] = off < 0 ? 0x80000000u : (uint32_t)off;
  }
  auto issue_k_tile = [&](int k0, int buf) {
    uint8_t* kdst = smem + buf * kStage;
    const uint32_t base = (uint32_t)k0 * T::kRowBytes;
#pragma unroll
    for (int i = 0; i < kKCopiesPerWave; ++i) {
      const int j = kSplitWaves * i + wl;
      if (j < T::kKCopies)
        buffer_load_lds16(k_rsrc, kdst + 1024 * j, (int)(base + k_off[i]));
    }
  };
  // V goes through registers so it can be stored transposed: thread = (4-key
  // group, 8-column chunk), key group fastest, so the 8-byte transposed stores
  // of one wave cover whole V^T rows without bank conflicts.
  const int v_kg4 = tid_l & 15;
  const int v_dc = tid_l >> 4;
  const bool v_loader = tid_l < T::kVBlocks;
  u32x4_t vreg[4];
  auto load_v_tile = [&](int k0) {
    if (v_loader) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vreg[r] = buffer_load_b128(v_rsrc, (k0 + 4 * v_kg4 + r) * T::kRowBytes + 16 * v_dc);
    }
  };
  auto store_v_tile = [&](int buf) {
    if (v_loader) {
      uint16_t* vt = reinterpret_cast<uint16_t*>(smem + buf * kStage + T::kKTile);
      store_block_transposed(vt, T::kVtStride / 2, 8 * v_dc, 4 * v_kg4, vreg);
    }
  };

  // ---- running state (log2 units), per 32-row block -------------------------
  // l: the fp32 weights (for the LSE); lr: the same weights as rounded to
  // bf16 for the P.V product, so O is normalised by exactly the weights it
  // accumulated (without it, a row dominated by one key whose weight rounds
  // by 2^-9 carries that error into O).  Both cover this lane's keys only;
  // lane pairs are summed at the end.
  float m2[BLOCKS], l[BLOCKS], lr[BLOCKS];
  f32x16_t oacc[BLOCKS][T::kDBlocks];
#pragma unroll
  for (int hf = 0; hf < BLOCKS; ++hf) {
    m2[hf] = kNegInf;
    l[hf] = 0.f;
    lr[hf] = 0.f;
#pragma unroll
    for (int cb = 0; cb < T::kDBlocks; ++cb) oacc[hf][cb] = f32x16_t{};
  }

#ifdef FATTN_DEVICE_COUNTERS
  unsigned n_computed = 0, n_masked = 0, n_raised = 0;
#endif

  // S^T = K Q^T for one block (32 keys x 32 queries per accumulator, two key blocks)
  auto scores = [&](const uint8_t* kt_lds, int hf, f32x16_t (&sacc)[2]) {
    sacc[0] = f32x16_t{};
    sacc[1] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < T::kKSteps; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
            kt_lds + (32 * kb + col) * T::kKStride + 32 * s + 16 * grp);
        sacc[kb] = mfma_32x32x16_bf16(a, qf[hf][s], sacc[kb]);
      }
    }
    interleave_reads_and_mfma<2 * T::kKSteps>();
  };

  // softmax of one block's 32 x 64 score tile -> bf16 P^T operands; updates l.
  // The running reference m (log2 units) is set to the row max on the first
  // tile (key tile 0, which holds key 0, visible to every row) and afterwards
  // raised only when needed: exp2(s*c - m) may exceed 1, and the tile is
  // accepted as long as this lane's terms sum to at most 2^kSlack (so no term
  // is larger).  Otherwise the reference is raised to the row max, l and O are
  // rebased by exp2(m_old - m_new) and the tile's terms are recomputed.  O and
  // l always share m, so the result is the same; fp32 holds the larger terms.
  // l sums the fp32 weights (the saved LSE must not carry the bf16 rounding
  // of the weights that multiply V).  c > 0 always (the host clamps it), so
  // masked scores of -inf give exp2(-inf) = 0 without a select.
  auto softmax_block = [&](f32x16_t (&sacc)[2], int hf, int k0, bool need_mask, bool first,
                           u32x4_t (&pf)[2][2]) {
    if (need_mask) {
      asm volatile("" ::: "memory");   // a real branch: unmasked tiles pay nothing
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = k0 + 32 * kb + 8 * (r >> 2) + 4 * grp + (r & 3);
          const bool dead =
              (kj >= N) || (CAUSAL && kj > qi[hf]) || (LOCAL && qi[hf] - kj >= window);
          if (dead) sacc[kb][r] = kNegInf;
        }
      }
    }
    auto row_max = [&]() {
      float smax = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sacc[kb][r]);
      return pair_max(smax) * c;
    };
    if (LOCAL || SPLIT > 1) {
      // a row's first visible key may lie in any tile: take the row max on
      // the first tile that shows the row a key (m2 stays -inf until then)
      if (__any(m2[hf] == kNegInf)) {
        const float mx = row_max();
        if (m2[hf] == kNegInf) m2[hf] = mx;
      }
    } else if (first) {
      m2[hf] = row_max();
    }
    float rsum = 0.f;   // the tile's weights as rounded to bf16
    auto weights = [&]() {
      // a row that has seen no key yet has only -inf scores here: reference 0
      const float m = ((LOCAL || SPLIT > 1) && m2[hf] == kNegInf) ? 0.f : m2[hf];
      float sa = 0.f, sb = 0.f, ra = 0.f, rb = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(fmaf(sacc[kb][r], c, -m));
          if (r & 1) sb += p[r]; else sa += p[r];
        }
        pf[kb][0] = pack_bf16x8(&p[0]);
        pf[kb][1] = pack_bf16x8(&p[8]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          ra = add_bf16_pair(pf[kb][t][0], ra);
          rb = add_bf16_pair(pf[kb][t][1], rb);
          ra = add_bf16_pair(pf[kb][t][2], ra);
          rb = add_bf16_pair(pf[kb][t][3], rb);
        }
      }
      rsum = ra + rb;
      return sa + sb;
    };
    float psum = weights();
    if (__builtin_expect(__any(psum > kSlackSum), 0)) {
#ifdef FATTN_DEVICE_COUNTERS
      if (!first) ++n_raised;
#endif
      asm volatile("" ::: "memory");
      const float m_new = fmaxf(m2[hf], row_max());
      // 1 for a row that has still seen no key (l and O are 0 there)
      const float corr = (m_new == kNegInf) ? 1.f : fast_exp2(m2[hf] - m_new);
      l[hf] *= corr;
      lr[hf] *= corr;
#pragma unroll
      for (int cb = 0; cb < T::kDBlocks; ++cb) oacc[hf][cb] *= corr;
      m2[hf] = m_new;
      psum = weights();
    }
    l[hf] += psum;
    lr[hf] += rsum;
  };

  // V^T operand (32 d x 16 keys) for d-block cb, key block kb, step t: one
  // 16-byte read of the transposed tile (keys 16t + 8*grp + 0..7 in the
  // permuted order that matches registers 8t..8t+7 of the score accumulator).
  const int vt_base = col * T::kVtStride + 16 * grp;
  auto v_operand = [&](const uint8_t* vt_lds, int cb, int kb, int t) {
    return *reinterpret_cast<const u32x4_t*>(vt_lds + vt_base + 32 * cb * T::kVtStride +
                                             2 * (32 * kb + 16 * t));
  };

  // ---- main loop: one barrier per step, LDS double-buffered; a step covers
  // SPLIT consecutive tiles, of which group sp takes the sp-th --------------
  const int t0 = kt_begin + sp;   // this group's first tile
  if (SPLIT == 1 || t0 < n_kt) {
    load_v_tile(t0 * kBN);
    issue_k_tile(t0 * kBN, sp);
  }
  wait_vmem_all();
  if (SPLIT == 1 || t0 < n_kt) store_v_tile(sp);
  if (t0 + SPLIT < n_kt) issue_k_tile((t0 + SPLIT) * kBN, SPLIT + sp);
  __syncthreads();

  for (int kt = kt_begin; kt < n_kt; kt += SPLIT) {
    const int my = kt + sp;   // this group's tile in this step
    const int buf = ((kt - kt_begin) / SPLIT) & 1;
    const int k0 = my * kBN;
    const uint8_t* kt_lds = smem + (buf * SPLIT + sp) * kStage;
    const uint8_t* vt_lds = kt_lds + T::kKTile;
    if (my + SPLIT < n_kt) load_v_tile(k0 + SPLIT * kBN);   // lands during this step

    bool act[BLOCKS], msk[BLOCKS];
    bool any_act = false;
#pragma unroll
    for (int hf = 0; hf < BLOCKS; ++hf) {
      const int first = wq_first + 32 * hf;
      act[hf] = (SPLIT == 1 || my < n_kt) && (first < N) && !(CAUSAL && k0 > first + 31) &&
                !(LOCAL && first - (k0 + kBN - 1) >= window);
      msk[hf] = (k0 + kBN > N) || (CAUSAL && k0 + kBN - 1 > first) ||
                (LOCAL && first + 31 - k0 >= window);
      any_act |= act[hf];
    }
    if (any_act) {
      f32x16_t sacc[BLOCKS][2];
      u32x4_t pf[BLOCKS][2][2];
      // block 0's softmax can run while block 1's scores are on the matrix cores
#pragma unroll
      for (int hf = 0; hf < BLOCKS; ++hf)
        if (act[hf]) scores(kt_lds, hf, sacc[hf]);
#pragma unroll
      for (int hf = 0; hf < BLOCKS; ++hf)
        if (act[hf]) softmax_block(sacc[hf], hf, k0, msk[hf], my == 0, pf[hf]);
#ifdef FATTN_DEVICE_COUNTERS
#pragma unroll
      for (int hf = 0; hf < BLOCKS; ++hf) {
        n_computed += act[hf] ? 1 : 0;
        n_masked += (act[hf] && msk[hf]) ? 1 : 0;
      }
#endif
      // O^T += V^T P^T; each V operand is read once and used by every block.
      // The d-block loop is innermost so consecutive matrix-core operations
      // accumulate into different registers (no back-to-back dependency).
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int cb = 0; cb < T::kDBlocks; ++cb) {
            const u32x4_t a = v_operand(vt_lds, cb, kb, t);
#pragma unroll
            for (int hf = 0; hf < BLOCKS; ++hf)
              if (act[hf]) oacc[hf][cb] = mfma_32x32x16_bf16(a, pf[hf][kb][t], oacc[hf][cb]);
          }
      if (BLOCKS == 1) interleave_reads_and_mfma<4 * T::kDBlocks>();
    }

    // tile kt+1 (K copy, V registers) must have landed; V^T goes into the
    // other buffer, which nobody has read since the previous barrier; then every
    // wave must be done with buffer `buf` before its K is overwritten
    wait_vmem_all();
    if (my + SPLIT < n_kt) store_v_tile((buf ^ 1) * SPLIT + sp);
    __syncthreads();
    if (my + 2 * SPLIT < n_kt) issue_k_tile(k0 + 2 * SPLIT * kBN, buf * SPLIT + sp);
  }

  if constexpr (SPLIT > 1) {
    // Groups sp > 0 hand their (m, l, lr, O) to group 0 through LDS (every
    // tile read ended before the loop's last barrier); group 0 brings both
    // partial results to their common reference and adds them ("How
    // FlashAttention Uses Tiling", "Why the Correction Factor Works").
    constexpr int kVals = 3 + 16 * T::kDBlocks;
    float* xch = reinterpret_cast<float*>(smem);
    static_assert((SPLIT - 1) * kSplitWaves * kVals * 64 * 4 <= 2 * SPLIT * kStage, "exchange");
    if (sp > 0) {
      float* mine = xch + ((sp - 1) * kSplitWaves + wl) * kVals * 64 + lane;
      mine[0] = m2[0];
      mine[64] = l[0];
      mine[128] = lr[0];
#pragma unroll
      for (int cb = 0; cb < T::kDBlocks; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[(3 + 16 * cb + r) * 64] = oacc[0][cb][r];
    }
    __syncthreads();
    if (sp == 0) {
#pragma unroll
      for (int o = 1; o < SPLIT; ++o) {
        const float* th = xch + ((o - 1) * kSplitWaves + wl) * kVals * 64 + lane;
        const float m1 = th[0];
        const float mm = fmaxf(m2[0], m1);
        const float f0 = m2[0] == kNegInf ? 0.f : fast_exp2(m2[0] - mm);
        const float f1 = m1 == kNegInf ? 0.f : fast_exp2(m1 - mm);
        l[0] = l[0] * f0 + th[64] * f1;
        lr[0] = lr[0] * f0 + th[128] * f1;
#pragma unroll
        for (int cb = 0; cb < T::kDBlocks; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            oacc[0][cb][r] = oacc[0][cb][r] * f0 + th[(3 + 16 * cb + r) * 64] * f1;
        m2[0] = mm;
      }
    }
  }

#ifdef FATTN_DEVICE_COUNTERS
  {
    // row blocks that hold rows of the sequence; each could have computed
    // every key tile of it
    unsigned blocks = 0;
#pragma unroll
    for (int hf = 0; hf < BLOCKS; ++hf) blocks += (wq_first + 32 * hf < N) ? 1 : 0;
    // (with a key split, group 0 accounts for the whole row block: the
    // additions below are modulo 2^64, so the sum over the groups is exact)
    const unsigned long long all_tiles =
        sp == 0 ? (unsigned long long)blocks * (unsigned long long)((N + kBN - 1) / kBN) : 0ull;
    if (lane == 0) {   // one vector atomic per counter and wave
      atomicAdd(&g_fwd_counters[0], (unsigned long long)n_computed);
      atomicAdd(&g_fwd_counters[1], all_tiles - (unsigned long long)n_computed);
      atomicAdd(&g_fwd_counters[2], (unsigned long long)n_masked);
      atomicAdd(&g_fwd_counters[3], (unsigned long long)n_raised);
    }
  }
#endif

  // ---- epilogue: O = acc / lr, LSE = (m + log2 l) ln 2 ---------------------
  if (SPLIT > 1 && sp != 0) return;
#pragma unroll
  for (int hf = 0; hf < BLOCKS; ++hf) {
    const float lt = pair_sum(l[hf]);
    const float lrt = pair_sum(lr[hf]);
    if (qi[hf] < N) {
      const float inv = 1.f / lrt;
      uint16_t* orow = O + (head_q + qi[hf]) * D;
#pragma unroll
      for (int cb = 0; cb < T::kDBlocks; ++cb) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = 32 * cb + 8 * r4 + 4 * grp;
          u32x2_t w;
          w.x = pack_bf16x2(oacc[hf][cb][4 * r4 + 0] * inv, oacc[hf][cb][4 * r4 + 1] * inv);
          w.y = pack_bf16x2(oacc[hf][cb][4 * r4 + 2] * inv, oacc[hf][cb][4 * r4 + 3] * inv);
          *reinterpret_cast<u32x2_t*>(orow + d0) = w;
        }
      }
      if (grp == 0) LSE[head_q + qi[hf]] = (m2[hf] + fast_log2(lt)) * kLn2;
    }
  }
}

// Workgroup shape: 8 waves (two per SIMD) of one 32-row block each.  Short
// sequences, whose 8-wave grid would leave CUs idle, use the 4-wave shape's
// grid (twice the workgroups, half the rows on each one's serial chain of key
// tiles): as 4-wave workgroups (two per CU), or, for causal rows of at least
// kSplitMinN keys, as 8-wave workgroups whose two wave groups take alternate
// key tiles and merge their partial results.
constexpr int kBlocks = 1;

template <int WAVES>
long long grid_items(const FwdArgs& a, int* hp_out, int* n_qblocks_out) {
  // query heads per workgroup: as many of a kv head's query heads as divide
  // both the group size and the wave count (at most 4)
  const int rep = a.H / a.Hkv;
  const int hp = (rep % 4 == 0 && WAVES % 4 == 0) ? 4 : (rep % 2 == 0 && WAVES % 2 == 0) ? 2 : 1;
  const int rows_h = (WAVES / hp) * 32 * kBlocks;
  const int n_qblocks = (a.N + rows_h - 1) / rows_h;
  *hp_out = hp;
  *n_qblocks_out = n_qblocks;
  return (long long)n_qblocks * a.B * a.H / hp;
}

template <int D, bool CAUSAL, bool LOCAL, int WAVES>
hipError_t launch_shape(const FwdArgs& a) {
  int hp = 1, n_qblocks = 0;
  const long long items = grid_items<WAVES>(a, &hp, &n_qblocks);
  // c > 0 lets masked scores (-inf) give exp2(-inf) = 0 directly; for scale 0
  // a c of 1e-30 changes no weight (|s| c stays far below fp32 resolution).
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  const int neg_q = a.scale < 0.f ? 1 : 0;
  return launch_kernel(fwd_bf16_kernel<D, CAUSAL, LOCAL, WAVES, kBlocks>,
                       dim3((unsigned)items), dim3(64 * WAVES), 0, a.stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                       a.B, a.H, a.Hkv, a.N, c, neg_q, n_qblocks, a.window, hp);
}

// Short sequences: 8-wave workgroups over the 4-wave shape's grid, the waves
// in two groups that take alternate key tiles (half the serial chain).
template <int D, bool CAUSAL>
hipError_t launch_split(const FwdArgs& a) {
  int hp = 1, n_qblocks = 0;
  const long long items = grid_items<4>(a, &hp, &n_qblocks);
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  const int neg_q = a.scale < 0.f ? 1 : 0;
  return launch_kernel(fwd_bf16_kernel<D, CAUSAL, false, 8, kBlocks, 2>, dim3((unsigned)items),
                       dim3(512), 0, a.stream, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                       static_cast<uint16_t*>(a.o), a.lse, a.B, a.H, a.Hkv, a.N, c, neg_q,
                       n_qblocks, a.window, hp);
}

constexpr long long kSmallGrid = 2 * 256;   // 8-wave workgroups: fewer than two per CU
constexpr int kSplitMinN = 512;
// Local attention with a window up to this many keys gives each workgroup a
// short chain of key tiles; two 4-wave workgroups per CU then overlap one's
// start-up with the other's tiles (measured on the 8192-row GQA shape: 11%
// faster at window 256, 3% at 512, even at 1024-2048; the 8-wave shape wins
// by 8% at full causal length).
constexpr int kLocalShortWindow = 2048;

template <int D, bool CAUSAL, bool LOCAL>
hipError_t launch_one(const FwdArgs& a) {
  int hp = 1, n_qblocks = 0;
  if (LOCAL && a.window <= kLocalShortWindow) return launch_shape<D, CAUSAL, LOCAL, 4>(a);
  if (grid_items<8>(a, &hp, &n_qblocks) < kSmallGrid) {
    // the key split pays where the causal chain is long enough (measured on
    // B=1 H=32 Hkv=8 d=128: N=512 -4%, 1024 -14%, 2048 -10%; N=128/256 and
    // non-causal rows, whose tiles all carry the same work, did not gain)
    if constexpr (CAUSAL && !LOCAL)
      if (a.N >= kSplitMinN) return launch_split<D, CAUSAL>(a);
    return launch_shape<D, CAUSAL, LOCAL, 4>(a);
  }
  return launch_shape<D, CAUSAL, LOCAL, 8>(a);
}

}  // namespace

hipError_t fwd_counters(unsigned long long* out, bool reset) {
#ifdef FATTN_DEVICE_COUNTERS
  hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_fwd_counters), sizeof(g_fwd_counters));
  if (e == hipSuccess && reset) {
    const unsigned long long zero[4] = {0, 0, 0, 0};
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_fwd_counters), zero, sizeof(zero));
  }
  return e;
#else
  (void)out;
  (void)reset;
  return hipErrorNotSupported;
#endif
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  // a window covering the whole sequence is plain causal attention
  const bool local = a.causal && a.window > 0 && a.window < a.N;
  if (a.d == 128) {
    if (local) return launch_one<128, true, true>(a);
    return a.causal ? launch_one<128, true, false>(a) : launch_one<128, false, false>(a);
  }
  if (local) return launch_one<64, true, true>(a);
  return a.causal ? launch_one<64, true, false>(a) : launch_one<64, false, false>(a);
}

}  // namespace fattn
