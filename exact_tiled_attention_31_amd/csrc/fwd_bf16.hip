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
//   * one workgroup = 4 waves = 128 query rows; each wave owns 32 rows and
//     keeps its Q fragment, the fp32 output accumulator and m, l in VGPRs;
//   * per 64-key tile the workgroup stages K (row-major) and V transposed
//     (d-major, keys permuted to match the score layout) in LDS; global
//     loads for tile j+1 are issued before tile j is computed;
//   * the scores are computed transposed, S^T = K Q^T, so each lane owns one
//     query row: the row max needs one exchange with the other half-wave and
//     the score accumulator becomes the P^T operand of O^T += V^T P^T
//     without leaving registers;
//   * exponentials are base 2 with scale*log2(e) folded into one FMA; the
//     scale is never applied to Q in bf16;
//   * heavy causal query blocks are dispatched first.
#include "common.hpp"
#include "launch.hpp"

namespace fattn {
namespace {

constexpr int kBM = 128;   // query rows per workgroup
constexpr int kBN = 64;    // keys per tile
constexpr int kThreads = 256;
constexpr float kNegInf = -__builtin_inff();

template <int D>
struct Tile {
  static constexpr int kKStride = D + 8;      // bf16 elements per K row in LDS (16-byte pad)
  static constexpr int kVStride = kBN + 8;    // bf16 elements per V^T row in LDS
  static constexpr int kKSteps = D / 16;      // contraction steps of S^T over d
  static constexpr int kDBlocks = D / 32;     // 32-row blocks of O^T
  static constexpr int kKChunks = kBN * D / 8 / kThreads;   // 16-byte K chunks per thread
  static constexpr int kVBlocks = (kBN / 4) * (D / 8);      // 4-key x 8-d V blocks per tile
  static_assert(kKChunks * kThreads * 8 == kBN * D, "K tile split");
  static_assert(kVBlocks <= kThreads, "one V block per thread at most");
};

// Position of key kk (0..kBN-1) inside a V^T row in LDS: bits 2 and 3 swapped.
// Register r of an S^T accumulator holds key 8*(r/4) + 4*grp + r%4 of its
// 32-key block; with the swap, the 8 keys one lane feeds to one P^T operand
// are 8 consecutive LDS positions, so the matching V^T operand is one
// 16-byte read.
__device__ __forceinline__ int vt_pos(int kk) {
  return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int B, int H, int Hkv, int N, float c, int neg_q, int n_qblocks) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBN * T::kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * T::kVStride];

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
  const uint16_t* Kh = K + head_kv * D;
  const uint16_t* Vh = V + head_kv * D;

  // ---- Q fragment (B operand of S^T): this lane's query row ----------------
  const int qi = q0 + wave * 32 + col;
  u32x4_t qf[T::kKSteps];
  {
    const uint32_t flip = neg_q ? 0x80008000u : 0u;   // exact sign flip for scale < 0
    const bool ok = qi < N;
    const uint16_t* qrow = Qh + (size_t)(ok ? qi : 0) * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < T::kKSteps; ++s) {
      u32x4_t x = ok ? *reinterpret_cast<const u32x4_t*>(qrow + 16 * s) : u32x4_t{0, 0, 0, 0};
      qf[s] = x ^ flip;
    }
  }

  const int q_hi = min(q0 + kBM, N);
  int n_kt = (N + kBN - 1) / kBN;
  if (CAUSAL) n_kt = min(n_kt, (q_hi - 1) / kBN + 1);
  const int wq_first = q0 + wave * 32;
  const int wq_last = wq_first + 31;

  // ---- tile loaders --------------------------------------------------------
  u32x4_t kreg[T::kKChunks];
  u32x4_t vreg[4];
  const int vblk = tid;                         // V block owned by this thread
  const int v_kg4 = vblk / (D / 8);             // which 4-key group
  const int v_dc = vblk - v_kg4 * (D / 8);      // which 8-column chunk

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < T::kKChunks; ++i) {
      const int ch = tid + kThreads * i;
      const int row = ch / (D / 8);
      const int c8 = ch - row * (D / 8);
      const int kr = k0 + row;
      kreg[i] = kr < N ? *reinterpret_cast<const u32x4_t*>(Kh + (size_t)kr * D + 8 * c8)
                       : u32x4_t{0, 0, 0, 0};
    }
    if (vblk < T::kVBlocks) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kr = k0 + 4 * v_kg4 + r;
        vreg[r] = kr < N ? *reinterpret_cast<const u32x4_t*>(Vh + (size_t)kr * D + 8 * v_dc)
                         : u32x4_t{0, 0, 0, 0};
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < T::kKChunks; ++i) {
      const int ch = tid + kThreads * i;
      const int row = ch / (D / 8);
      const int c8 = ch - row * (D / 8);
      *reinterpret_cast<u32x4_t*>(&sK[row * T::kKStride + 8 * c8]) = kreg[i];
    }
    if (vblk < T::kVBlocks) {
      const int pos0 = vt_pos(4 * v_kg4);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int w = i >> 1;
        u32x2_t pair;
        if ((i & 1) == 0) {
          pair.x = pack_lo_halves(vreg[0][w], vreg[1][w]);
          pair.y = pack_lo_halves(vreg[2][w], vreg[3][w]);
        } else {
          pair.x = pack_hi_halves(vreg[0][w], vreg[1][w]);
          pair.y = pack_hi_halves(vreg[2][w], vreg[3][w]);
        }
        *reinterpret_cast<u32x2_t*>(&sVt[(8 * v_dc + i) * T::kVStride + pos0]) = pair;
      }
    }
  };

  // ---- running state (log2 units) -----------------------------------------
  float m2 = kNegInf;
  float l = 0.f;   // partial: this lane's keys only; halves are summed at the end
  f32x16_t oacc[T::kDBlocks];
#pragma unroll
  for (int cb = 0; cb < T::kDBlocks; ++cb) oacc[cb] = f32x16_t{};

  load_tile(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * kBN;
    if (kt > 0) __syncthreads();   // every wave has finished reading the previous tile
    store_tile();
    __syncthreads();
    if (kt + 1 < n_kt) load_tile(k0 + kBN);

    const bool active = (wq_first < N) && !(CAUSAL && k0 > wq_last);
    if (!active) continue;

    // S^T = K Q^T for two 32-key blocks
    f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int s = 0; s < T::kKSteps; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4_t a =
            *reinterpret_cast<const u32x4_t*>(&sK[(32 * kb + col) * T::kKStride + 16 * s + 8 * grp]);
        sacc[kb] = mfma_32x32x16_bf16(a, qf[s], sacc[kb]);
      }
    }

    const bool need_mask = (k0 + kBN > N) || (CAUSAL && k0 + kBN - 1 > wq_first);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = k0 + 32 * kb + 8 * (r >> 2) + 4 * grp + (r & 3);
          const bool dead = (kj >= N) || (CAUSAL && kj > qi);
          if (dead) sacc[kb][r] = kNegInf;
        }
      }
    }

    float smax = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sacc[kb][r]);
    smax = fmaxf(smax, swap_half(smax));
    const float mx = (smax == kNegInf) ? kNegInf : smax * c;
    const float m_new = fmaxf(m2, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float corr = fast_exp2(m2 - m_use);   // 0 while nothing was seen

    float psum = 0.f;
    u32x4_t pf[2][2];
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
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        pf[kb][t] = u32x4_t{pack_bf16x2(p[8 * t + 0], p[8 * t + 1]),
                            pack_bf16x2(p[8 * t + 2], p[8 * t + 3]),
                            pack_bf16x2(p[8 * t + 4], p[8 * t + 5]),
                            pack_bf16x2(p[8 * t + 6], p[8 * t + 7])};
      }
    }
    l = l * corr + psum;
    if (__any(corr != 1.f)) {
#pragma unroll
      for (int cb = 0; cb < T::kDBlocks; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] *= corr;
    }
    m2 = m_new;

    // O^T += V^T P^T
#pragma unroll
    for (int cb = 0; cb < T::kDBlocks; ++cb) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
              &sVt[(32 * cb + col) * T::kVStride + 32 * kb + 16 * t + 8 * grp]);
          oacc[cb] = mfma_32x32x16_bf16(a, pf[kb][t], oacc[cb]);
        }
      }
    }
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----------------------
  const float lt = l + swap_half(l);
  if (qi < N) {
    const float inv = 1.f / lt;
    uint16_t* orow = O + (head_q + qi) * D;
#pragma unroll
    for (int cb = 0; cb < T::kDBlocks; ++cb) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * cb + 8 * r4 + 4 * grp;
        u32x2_t w;
        w.x = pack_bf16x2(oacc[cb][4 * r4 + 0] * inv, oacc[cb][4 * r4 + 1] * inv);
        w.y = pack_bf16x2(oacc[cb][4 * r4 + 2] * inv, oacc[cb][4 * r4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(orow + d0) = w;
      }
    }
    if (grp == 0) LSE[head_q + qi] = (m2 + fast_log2(lt)) * kLn2;
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
