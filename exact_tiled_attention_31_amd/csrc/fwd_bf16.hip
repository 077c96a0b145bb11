// Exact tiled attention forward, bf16 storage, bf16 matrix cores with fp32
// accumulation (gfx950).
//
// Method ("LLM Architecture Refresh [3]: Flash Attention Is Exact", section 4
// "Tiled attention in 40 lines", with section 2's running statistics and
// section 7's causal tile skipping; "How FlashAttention Uses Tiling", update
// equations under "The Running Statistics"): for one query block, stream the
// key/value tiles through on-chip memory; per tile compute the scores, raise
// the running max m, rebase the running sum l and the unnormalised output by
// exp(m_old - m_new), add the tile's exp(s - m_new) and p.V, and divide by l
// once at the end.  Tiles whose first key lies after the block's last query
// are never loaded.  The N x N scores never leave registers.
//
// Mapping onto CDNA4:
//   * one workgroup = 4 waves = 256 query rows; each wave owns 64 rows as two
//     32-row halves and keeps their Q fragments, fp32 output accumulators and
//     m, l in registers;
//   * 64-key tiles of K and V are copied global -> LDS by the buffer unit
//     (buffer_load_dwordx4 ... lds, 16 bytes per lane, no VGPR staging);
//     rows past N read as zero.  Tiles are double-buffered with one barrier
//     per tile; the copy of tile j+2 is in flight while tile j+1 waits;
//   * LDS rows are unpadded; each 16-byte chunk is XOR-swizzled by its row so
//     that the K reads (ds_read_b128, 16 consecutive rows) and the V
//     transpose reads (ds_read_b64_tr_b16, 8 rows x 64 bytes) are free of
//     bank conflicts;
//   * the scores are computed transposed, S^T = K Q^T, so each lane owns one
//     query row: the row max needs one exchange with the other half-wave
//     (v_permlane32_swap) and the score accumulator becomes the P^T operand of
//     O^T += V^T P^T without leaving registers.  V^T operands come straight
//     from row-major V through the transpose read;
//   * the halves are staggered: S of half 1 runs on the matrix cores while
//     half 0 does its softmax, and half 1's softmax overlaps half 0's P.V;
//     V fragments are read once per tile and reused by both halves;
//   * exponentials are base 2 with scale*log2(e) folded into one FMA; the
//     scale is never applied to Q in bf16;
//   * heavy causal query blocks are dispatched first.
#include "common.hpp"
#include "launch.hpp"

namespace fattn {
namespace {

constexpr int kWaves = 4;
constexpr int kQW = 64;               // query rows per wave (two 32-row halves)
constexpr int kBM = kWaves * kQW;     // query rows per workgroup
constexpr int kBN = 64;               // keys per tile
constexpr int kThreads = 64 * kWaves;
constexpr float kNegInf = -__builtin_inff();

template <int D>
struct Tile {
  static constexpr int kRowBytes = 2 * D;                // unpadded bf16 row
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
  static constexpr int kRowsPer256 = 256 / kRowBytes;    // rows sharing one 256-byte bank span
  static constexpr int kTileBytes = kBN * kRowBytes;
  static constexpr int kSlots = kTileBytes / 16;         // 16-byte copy slots per tile
  static constexpr int kCopiesPerThread = kSlots / kThreads;
  static constexpr int kKSteps = D / 16;                 // contraction steps of S^T over d
  static constexpr int kDBlocks = D / 32;                // 32-row blocks of O^T
  static_assert(kSlots % kThreads == 0, "tile copy split");
};

// XOR swizzle of the 16-byte chunk index within an LDS row.
template <int D>
__device__ __forceinline__ int swz(int row) {
  using T = Tile<D>;
  constexpr int kQ = T::kChunks / 4;
  const int m = row / T::kRowsPer256;
  return 4 * (m % kQ) + (m / kQ) % 4;
}

// Byte offset in a tile of element (row, col) (col a multiple of 4).
template <int D>
__device__ __forceinline__ int lds_off(int row, int col) {
  using T = Tile<D>;
  return row * T::kRowBytes + 16 * ((col >> 3) ^ swz<D>(row)) + 2 * (col & 7);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int B, int H, int Hkv, int N, float c, int neg_q, int n_qblocks) {
  using T = Tile<D>;
  // [buffer][K | V] tiles
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * 2 * T::kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int grp = lane >> 5;

  // ---- work item: heavy causal query blocks first --------------------------
  const int BH = B * H;
  const int item_q = blockIdx.x / BH;
  const int bh = blockIdx.x - item_q * BH;
  const int qb = CAUSAL ? (n_qblocks - 1 - item_q) : item_q;
  const int b = bh / H;
  const int h = bh - b * H;
  const int g = h / (H / Hkv);
  const int q0 = qb * kBM;

  const size_t head_q = (size_t)bh * N;
  const size_t head_kv = ((size_t)b * Hkv + g) * N;
  const uint16_t* Qh = Q + head_q * D;
  const i32x4_t k_rsrc = make_buffer_rsrc(K + head_kv * D, (uint32_t)N * T::kRowBytes);
  const i32x4_t v_rsrc = make_buffer_rsrc(V + head_kv * D, (uint32_t)N * T::kRowBytes);

  const int wq_first = q0 + wave * kQW;   // this wave's first query row
  int qi[2];
  qi[0] = wq_first + col;
  qi[1] = wq_first + 32 + col;

  // ---- Q fragments (B operands of S^T), one set per half --------------------
  u32x4_t qf[2][T::kKSteps];
  {
    const uint32_t flip = neg_q ? 0x80008000u : 0u;   // exact sign flip for scale < 0
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const bool ok = qi[hf] < N;
      const uint16_t* qrow = Qh + (size_t)(ok ? qi[hf] : 0) * D + 8 * grp;
#pragma unroll
      for (int s = 0; s < T::kKSteps; ++s) {
        u32x4_t x = ok ? *reinterpret_cast<const u32x4_t*>(qrow + 16 * s) : u32x4_t{0, 0, 0, 0};
        qf[hf][s] = x ^ flip;
      }
    }
  }

  const int q_hi = min(q0 + kBM, N);
  int n_kt = (N + kBN - 1) / kBN;
  if (CAUSAL) n_kt = min(n_kt, (q_hi - 1) / kBN + 1);

  // ---- tile copy: slot = (instruction, wave, lane) -> (row, swizzled chunk) --
  int copy_src[T::kCopiesPerThread];   // byte offset of this lane's chunk within a tile's rows
#pragma unroll
  for (int i = 0; i < T::kCopiesPerThread; ++i) {
    const int slot = (i * kWaves + wave) * 64 + lane;
    const int row = slot / T::kChunks;
    const int pchunk = slot % T::kChunks;
    copy_src[i] = row * T::kRowBytes + 16 * (pchunk ^ swz<D>(row));
  }
  auto issue_tile = [&](int k0, int buf) {
    uint8_t* kdst = smem + (2 * buf) * T::kTileBytes;
    uint8_t* vdst = kdst + T::kTileBytes;
    const int base = k0 * T::kRowBytes;
#pragma unroll
    for (int i = 0; i < T::kCopiesPerThread; ++i) {
      const int wslot = (i * kWaves + wave) * 64 * 16;   // this wave's 1 KB destination
      buffer_load_lds16(k_rsrc, kdst + wslot, base + copy_src[i]);
      buffer_load_lds16(v_rsrc, vdst + wslot, base + copy_src[i]);
    }
  };

  // ---- running state (log2 units), per half ---------------------------------
  float m2[2] = {kNegInf, kNegInf};
  float l[2] = {0.f, 0.f};   // partial: this lane's keys only; lane pairs are summed at the end
  f32x16_t oacc[2][T::kDBlocks];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int cb = 0; cb < T::kDBlocks; ++cb) oacc[hf][cb] = f32x16_t{};

  // S^T = K Q^T for one half (32 keys x 32 queries per block, two key blocks)
  auto scores = [&](const uint8_t* kt_lds, int hf, f32x16_t (&sacc)[2]) {
    sacc[0] = f32x16_t{};
    sacc[1] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < T::kKSteps; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
            kt_lds + lds_off<D>(32 * kb + col, 16 * s + 8 * grp));
        sacc[kb] = mfma_32x32x16_bf16(a, qf[hf][s], sacc[kb]);
      }
    }
  };

  // softmax of one half's 32 x 64 score tile -> bf16 P^T operands; updates m, l, O
  auto softmax_half = [&](f32x16_t (&sacc)[2], int hf, int k0, bool need_mask,
                          u32x4_t (&pf)[2][2]) {
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = k0 + 32 * kb + 8 * (r >> 2) + 4 * grp + (r & 3);
          const bool dead = (kj >= N) || (CAUSAL && kj > qi[hf]);
          if (dead) sacc[kb][r] = kNegInf;
        }
      }
    }
    float smax = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sacc[kb][r]);
    smax = pair_max(smax);
    const float mx = (smax == kNegInf) ? kNegInf : smax * c;
    const float m_new = fmaxf(m2[hf], mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float corr = fast_exp2(m2[hf] - m_use);   // 0 while nothing was seen
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = fast_exp2(fmaf(sacc[kb][r], c, -m_use));
        if (need_mask && sacc[kb][r] == kNegInf) e = 0.f;   // exact zero even if c == 0
        p[r] = e;
        psum += e;
      }
      pf[kb][0] = pack_bf16x8(&p[0]);
      pf[kb][1] = pack_bf16x8(&p[8]);
    }
    l[hf] = l[hf] * corr + psum;
    if (__any(corr != 1.f)) {
#pragma unroll
      for (int cb = 0; cb < T::kDBlocks; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[hf][cb][r] *= corr;
    }
    m2[hf] = m_new;
  };

  // V^T operand (32 d x 16 keys) for d-block cb, key block kb, step t:
  // two transpose reads of 4 keys each (keys 16t + 4*grp + 0..3 and +8).
  const int tr_j = (lane & 15) >> 2;                 // row within the 4-row group
  const int tr_col = 4 * (lane & 3) + 16 * ((lane >> 4) & 1);
  auto v_operand = [&](const uint8_t* vt_lds, int cb, int kb, int t) {
    const int key = 32 * kb + 16 * t + 4 * grp + tr_j;
    const int dcol = 32 * cb + tr_col;
    const u32x2_t lo = ds_read_tr16_b64(vt_lds + lds_off<D>(key, dcol));
    const u32x2_t hi = ds_read_tr16_b64(vt_lds + lds_off<D>(key + 8, dcol));
    return u32x4_t{lo.x, lo.y, hi.x, hi.y};
  };

  // ---- main loop: one barrier per tile, LDS double-buffered ----------------
  issue_tile(0, 0);
  if (n_kt > 1) issue_tile(kBN, 1);
  wait_vmem_at_most_one_tile<2 * T::kCopiesPerThread>(n_kt > 1);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    const int k0 = kt * kBN;
    const uint8_t* kt_lds = smem + (2 * buf) * T::kTileBytes;
    const uint8_t* vt_lds = kt_lds + T::kTileBytes;

    const bool act0 = (wq_first < N) && !(CAUSAL && k0 > wq_first + 31);
    const bool act1 = (wq_first + 32 < N) && !(CAUSAL && k0 > wq_first + 63);
    if (act1) {   // act0 implies act1 unless the second half is past N
      f32x16_t s0[2], s1[2];
      u32x4_t pf0[2][2], pf1[2][2];
      u32x4_t vf[T::kDBlocks][2][2];
      const bool mask0 = (k0 + kBN > N) || (CAUSAL && k0 + kBN - 1 > wq_first);
      const bool mask1 = (k0 + kBN > N) || (CAUSAL && k0 + kBN - 1 > wq_first + 32);
      if (act0) scores(kt_lds, 0, s0);
      scores(kt_lds, 1, s1);
      if (act0) softmax_half(s0, 0, k0, mask0, pf0);
#pragma unroll
      for (int cb = 0; cb < T::kDBlocks; ++cb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) vf[cb][kb][t] = v_operand(vt_lds, cb, kb, t);
      if (act0) {
#pragma unroll
        for (int cb = 0; cb < T::kDBlocks; ++cb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
              oacc[0][cb] = mfma_32x32x16_bf16(vf[cb][kb][t], pf0[kb][t], oacc[0][cb]);
      }
      softmax_half(s1, 1, k0, mask1, pf1);
#pragma unroll
      for (int cb = 0; cb < T::kDBlocks; ++cb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            oacc[1][cb] = mfma_32x32x16_bf16(vf[cb][kb][t], pf1[kb][t], oacc[1][cb]);
    } else if (act0) {   // only the first half is below N
      f32x16_t s0[2];
      u32x4_t pf0[2][2];
      const bool mask0 = (k0 + kBN > N) || (CAUSAL && k0 + kBN - 1 > wq_first);
      scores(kt_lds, 0, s0);
      softmax_half(s0, 0, k0, mask0, pf0);
#pragma unroll
      for (int cb = 0; cb < T::kDBlocks; ++cb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            oacc[0][cb] = mfma_32x32x16_bf16(v_operand(vt_lds, cb, kb, t), pf0[kb][t], oacc[0][cb]);
    }

    // tile kt+1 must have landed and every wave must be done with buffer `buf`
    wait_vmem_all();
    __syncthreads();
    if (kt + 2 < n_kt) issue_tile(k0 + 2 * kBN, buf);
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----------------------
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const float lt = pair_sum(l[hf]);
    if (qi[hf] < N) {
      const float inv = 1.f / lt;
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

template <int D, bool CAUSAL>
hipError_t launch_one(const FwdArgs& a) {
  const int n_qblocks = (a.N + kBM - 1) / kBM;
  const long long items = (long long)n_qblocks * a.B * a.H;
  const float c = fabsf(a.scale) * kLog2e;
  const int neg_q = a.scale < 0.f ? 1 : 0;
  return launch_kernel(fwd_bf16_kernel<D, CAUSAL>, dim3((unsigned)items), dim3(kThreads), 0,
                       a.stream, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                       static_cast<uint16_t*>(a.o), a.lse, a.B, a.H, a.Hkv, a.N, c, neg_q,
                       n_qblocks);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch_one<128, true>(a) : launch_one<128, false>(a);
  return a.causal ? launch_one<64, true>(a) : launch_one<64, false>(a);
}

}  // namespace fattn
