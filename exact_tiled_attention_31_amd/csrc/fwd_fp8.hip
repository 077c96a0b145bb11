// Exact tiled attention forward on FP8 (OCP e4m3) inputs with per-tensor
// scales, fp8 matrix cores with fp32 accumulation, bf16 output (gfx950).
//
// Method: the same tiled loop as the bf16 forward ("LLM Architecture Refresh
// [3]: Flash Attention Is Exact", section 4, with section 2's running
// statistics and section 7's causal tile skipping; "How FlashAttention Uses
// Tiling", "The Running Statistics"), on the low-precision matrix cores that
// section 8 of the same page credits to FlashAttention-3.  The inputs hold
// the values x = descale_x * e4m3(code); both products run on
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales):
//   * S^T = K Q^T from the fp8 codes; the matrix core sums each 64-term step
//     with less than fp32 precision (measured on random codes: within
//     2^-12.4 of the sum of |terms|), the steps add in fp32; the scale and
//     both descales are folded into c = scale * dq * dk * log2(e);
//   * the weights p = exp2(s*c - m) are rounded to e4m3 (round to nearest
//     even) for O^T += V^T P^T.  The running reference m is raised whenever a
//     tile's row max exceeds it by more than 2 (log2 units), and the weights
//     are formed relative to m - 6, so they lie in (0, 256] (e4m3 holds up to
//     448) and keep e4m3's 3-bit precision down to 2^-12 of the row max;
//   * l sums the unrounded fp32 weights, so the saved LSE carries no fp8
//     rounding; O = acc * dv / l is rounded to bf16 once.
// Against the definition evaluated on the same fp8 inputs, with e_i the
// largest score error of row i (at most 2^-11 |scale| max_j sum_c |q_ic k_jc|
// by the accumulation above), the error is bounded elementwise by
// (2^-4 + 2 e_i) (P|V|)_ic + 2^-16 sum_j |v_jc| (e4m3 rounding of each weight:
// half an ulp is 2^-4 relative in the normal range and 2^-10 absolute below
// it, against l >= 2^6) plus the bf16 rounding of O; the LSE error by e_i.
//
// Mapping onto CDNA4 (as the bf16 forward, with 1-byte elements):
//   * a workgroup of 12 waves owns 384 query rows; each wave keeps 32 rows'
//     Q fragments, fp32 output accumulators and m, l in registers.  The
//     kernel fits 168 registers per lane, so three waves share each SIMD and
//     a third wave's matrix-core steps fill the softmax of the other two
//     (measured 5% faster than 8-wave workgroups at two waves per SIMD);
//   * a 32x32x64 fp8 operand is 32 bytes per lane: lane = row (A) or column
//     (B), bytes j = k index 32*(lane/32) + j;
//   * 64-key tiles: K copied global -> LDS by the buffer unit into rows padded
//     by 16 bytes; V loaded into registers one tile ahead and stored
//     transposed (d-major) with the keys permuted so that one lane's 32
//     bytes are the keys whose weights it holds, i.e. the P^T operand is the
//     score accumulator converted in place;
//   * heavy causal query blocks are dispatched first; tiles after the block's
//     last query are never loaded.
#include "common.hpp"
#include "launch.hpp"

namespace fattn {
namespace {

constexpr int kBN = 64;   // keys per tile
constexpr int kWaves = 12;
constexpr int kBM = kWaves * 32;
constexpr float kNegInf = -__builtin_inff();
constexpr float kSlack = 2.f;     // log2 units a row max may exceed m by
constexpr float kPShift = 6.f;    // weights are exp2(s*c - (m - kPShift)) <= 2^8

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

template <int D>
struct Tile8 {
  static constexpr int kRowBytes = D;                  // one fp8 row in global memory
  static constexpr int kChunks = D / 16;               // 16-byte chunks per row
  static constexpr int kKSlots = kChunks + 1;          // K rows padded by one 16-byte slot
  static constexpr int kKStride = 16 * kKSlots;        // 144 (D = 128) or 80 bytes
  static constexpr int kVtStride = kBN + 16;           // one V^T row: 64 keys + 16 pad
  static constexpr int kKTile = kBN * kKStride;
  // every 16-row group of V^T starts 64 bytes further on, so the transposed
  // 4-byte stores of one wave (rows 8 apart) never share a bank
  static constexpr int kVTile = D * kVtStride + 64 * (D / 16 - 1);
  static constexpr int kKCopies = kBN * kKSlots / 64;  // wave-wide copy instructions per K tile
  static constexpr int kKSteps = D / 64;               // contraction steps of S^T over d
  static constexpr int kDBlocks = D / 32;              // 32-row blocks of O^T
  static constexpr int kVPieces = (kBN / 4) * (D / 8); // 4-key x 8-column V pieces per tile
  static constexpr int kStage = ((kKTile + kVTile + 15) / 16) * 16;
  static_assert((kBN * kKSlots) % 64 == 0, "whole copy instructions");
  static_assert(kVPieces <= 64 * kWaves, "one V piece per thread at most");
};

// n matrix-core steps with two 16-byte operand reads each: the reads of the
// first two steps first, then each step followed by the reads of the step
// two ahead.
template <int n>
__device__ __forceinline__ void reads_ahead_fp8() {
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  constexpr int lead = n < 2 ? n : 2;
  __builtin_amdgcn_sched_group_barrier(kDsRead, 2 * lead, 0);
#pragma unroll
  for (int i = 0; i < n - lead; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMfma, lead, 0);
}

__device__ __forceinline__ f32x16_t mfma_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
  // formats 0/0 = e4m3 for A and B; block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Byte position of key kk (0..63) inside a V^T row: lane group g = (kk/4)%2
// holds bytes 32g .. 32g+31, in the order of the score accumulator registers
// (key block kk/32, register 4*((kk%32)/8) + kk%4).
__device__ __forceinline__ int vt_pos(int kk) {
  return 32 * ((kk >> 2) & 1) + 16 * (kk >> 5) + 4 * ((kk & 31) >> 3) + (kk & 3);
}
// Byte offset of V^T row c (d index) inside the tile.
__device__ __forceinline__ int vt_row(int c, int stride) { return c * stride + 64 * (c >> 4); }

extern "C" __device__ u32x2_t fattn_llvm_raw_buffer_load_v2i32(i32x4_t rsrc, int voffset,
                                                               int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v2i32");

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kWaves, 1) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int B, int H, int Hkv, int N, float c,
    int neg_q, float v_descale, int n_qblocks) {
  using T = Tile8<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * T::kStage];

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
  const i32x4_t k_rsrc = make_buffer_rsrc(K + head_kv * D, (uint32_t)N * T::kRowBytes);
  const i32x4_t v_rsrc = make_buffer_rsrc(V + head_kv * D, (uint32_t)N * T::kRowBytes);

  const int first = q0 + wave * 32;   // this wave's first query row
  const int qi = first + col;

  // ---- Q fragments (B operands of S^T): bytes 64s + 32*grp .. +31 of the row
  i32x8_t qf[T::kKSteps];
  {
    const uint32_t flip = neg_q ? 0x80808080u : 0u;   // exact sign flip for a negative c
    const bool ok = qi < N;
    const uint8_t* qrow = Q + (head_q + (ok ? qi : 0)) * D + 32 * grp;
#pragma unroll
    for (int s = 0; s < T::kKSteps; ++s) {
      const u32x4_t lo = ok ? *reinterpret_cast<const u32x4_t*>(qrow + 64 * s) : u32x4_t{0, 0, 0, 0};
      const u32x4_t hi =
          ok ? *reinterpret_cast<const u32x4_t*>(qrow + 64 * s + 16) : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qf[s][i] = (int32_t)(lo[i] ^ flip);
        qf[s][4 + i] = (int32_t)(hi[i] ^ flip);
      }
    }
  }

  const int q_hi = min(q0 + kBM, N);
  int n_kt = (N + kBN - 1) / kBN;
  if (CAUSAL) n_kt = min(n_kt, (q_hi - 1) / kBN + 1);

  // ---- K tile copy: wave-wide instruction j fills LDS slots 64j .. 64j+63 ---
  // Per-lane offsets of this wave's copy slots within a tile, fixed for the
  // whole loop; pad slots get 2^31, which with any tile base below 2^31 lands
  // past the buffer's range and reads as zero (no per-copy select).
  constexpr int kKCopiesPerWave = (T::kKCopies + kWaves - 1) / kWaves;
  uint32_t k_off[kKCopiesPerWave];
#pragma unroll
  for (int i = 0; i < kKCopiesPerWave; ++i) {
    const int slot = 64 * (kWaves * i + wave) + lane;
    const int row = slot / T::kKSlots;
    const int chunk = slot - row * T::kKSlots;
    k_off[i] = chunk < T::kChunks ? (uint32_t)(row * T::kRowBytes + 16 * chunk) : 0x80000000u;
  }
  auto issue_k_tile = [&](int k0, int buf) {
    uint8_t* kdst = smem + buf * T::kStage;
    const uint32_t base = (uint32_t)k0 * T::kRowBytes;
#pragma unroll
    for (int i = 0; i < kKCopiesPerWave; ++i) {
      const int j = kWaves * i + wave;
      if (j < T::kKCopies) buffer_load_lds16(k_rsrc, kdst + 1024 * j, (int)(base + k_off[i]));
    }
  };
  // ---- V tile: thread = (4-key group, 8-column chunk) loads 4 x 8 bytes and
  // stores the 8 columns as 4-byte words (4 keys each) into V^T
  const int v_kg4 = tid & 15;
  const int v_dc = tid >> 4;
  const bool v_loader = tid < T::kVPieces;
  u32x2_t vreg[4];
  auto load_v_tile = [&](int k0) {
    if (v_loader) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vreg[r] = fattn_llvm_raw_buffer_load_v2i32(
            v_rsrc, (k0 + 4 * v_kg4 + r) * T::kRowBytes + 8 * v_dc, 0, 0);
    }
  };
  auto store_v_tile = [&](int buf) {
    if (v_loader) {
      uint8_t* vt = smem + buf * T::kStage + T::kKTile + vt_pos(4 * v_kg4);
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        // bytes of rows 0/1 and 2/3 interleaved, then whole columns
        const uint32_t lo01 = byte_perm(vreg[1][w], vreg[0][w], 0x05010400u);
        const uint32_t hi01 = byte_perm(vreg[1][w], vreg[0][w], 0x07030602u);
        const uint32_t lo23 = byte_perm(vreg[3][w], vreg[2][w], 0x05010400u);
        const uint32_t hi23 = byte_perm(vreg[3][w], vreg[2][w], 0x07030602u);
        const uint32_t colw[4] = {byte_perm(lo23, lo01, 0x05040100u),
                                  byte_perm(lo23, lo01, 0x07060302u),
                                  byte_perm(hi23, hi01, 0x05040100u),
                                  byte_perm(hi23, hi01, 0x07060302u)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int cidx = 8 * v_dc + 4 * w + i;
          *reinterpret_cast<uint32_t*>(vt + vt_row(cidx, T::kVtStride)) = colw[i];
        }
      }
    }
  };

  // ---- running state (log2 units) -------------------------------------------
  float m2 = kNegInf;
  float l = 0.f;   // this lane's keys only; lane pairs are summed at the end
  f32x16_t oacc[T::kDBlocks];
#pragma unroll
  for (int cb = 0; cb < T::kDBlocks; ++cb) oacc[cb] = f32x16_t{};

  // per-lane LDS offsets: K operand row `col`, V^T operand row `col`
  const int k_lane = col * T::kKStride + 32 * grp;
  const int vt_lane = col * T::kVtStride + 64 * (col >> 4) + 32 * grp;

  auto ld32 = [](const uint8_t* p) {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(p);
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(p + 16);
    return i32x8_t{(int32_t)lo[0], (int32_t)lo[1], (int32_t)lo[2], (int32_t)lo[3],
                   (int32_t)hi[0], (int32_t)hi[1], (int32_t)hi[2], (int32_t)hi[3]};
  };

  // ---- main loop: one barrier per tile, LDS double-buffered ----------------
  load_v_tile(0);
  issue_k_tile(0, 0);
  wait_vmem_all();
  store_v_tile(0);
  if (n_kt > 1) issue_k_tile(kBN, 1);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    const int k0 = kt * kBN;
    const uint8_t* kt_lds = smem + buf * T::kStage;
    const uint8_t* vt_lds = kt_lds + T::kKTile;
    if (kt + 1 < n_kt) load_v_tile(k0 + kBN);   // lands during this tile's compute

    const bool act = (first < N) && !(CAUSAL && k0 > first + 31);
    const bool msk = (k0 + kBN > N) || (CAUSAL && k0 + kBN - 1 > first);
    if (act) {
      // S^T = K Q^T: two 32-key blocks, D/64 contraction steps each
      f32x16_t sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb] = f32x16_t{};
      // contraction step outermost: consecutive steps go to different
      // accumulators; operand reads kept two steps ahead
#pragma unroll
      for (int s = 0; s < T::kKSteps; ++s)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          sacc[kb] = mfma_fp8(ld32(kt_lds + k_lane + 32 * kb * T::kKStride + 64 * s), qf[s],
                              sacc[kb]);
      reads_ahead_fp8<2 * T::kKSteps>();
      if (msk) {
        asm volatile("" ::: "memory");   // a real branch: unmasked tiles pay nothing
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kj = k0 + 32 * kb + 8 * (r >> 2) + 4 * grp + (r & 3);
            if ((kj >= N) || (CAUSAL && kj > qi)) sacc[kb][r] = kNegInf;
          }
      }
      float smax = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sacc[kb][r]);
      if (__builtin_expect(__any(smax * c > m2 + kSlack), 0)) {
        // raise the reference to the row max and rebase l and O
        asm volatile("" ::: "memory");
        const float m_new = fmaxf(m2, pair_max(smax) * c);
        const float corr = (m_new == kNegInf) ? 1.f : fast_exp2(m2 - m_new);
        l *= corr;
#pragma unroll
        for (int cb = 0; cb < T::kDBlocks; ++cb) oacc[cb] *= corr;
        m2 = m_new;
      }
      // weights relative to m - kPShift, in (0, 2^8]; fp32 sum, e4m3 operand
      const float mref = m2 - kPShift;
      float sa = 0.f, sb = 0.f;
      i32x8_t pf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(sacc[kb][4 * w + i], c, -mref));
          sa += p[0] + p[2];
          sb += p[1] + p[3];
          // the old-value operand only supplies bits 16..31, which the second
          // conversion overwrites: any live register avoids a zero fill
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __builtin_bit_cast(int, p[0]), false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
          pf[4 * kb + w] = word;
        }
      l += sa + sb;
      // O^T += V^T P^T: one 64-key step per 32-row d block
#pragma unroll
      for (int cb = 0; cb < T::kDBlocks; ++cb)
        oacc[cb] = mfma_fp8(ld32(vt_lds + vt_lane + 32 * cb * T::kVtStride + 128 * cb), pf,
                            oacc[cb]);
      reads_ahead_fp8<T::kDBlocks>();
    }

    // tile kt+1 (K copy, V registers) must have landed; V^T goes into the
    // other buffer, which nobody has read since the previous barrier; then every
    // wave must be done with buffer `buf` before its K is overwritten
    wait_vmem_all();
    if (kt + 1 < n_kt) store_v_tile(buf ^ 1);
    __syncthreads();
    if (kt + 2 < n_kt) issue_k_tile(k0 + 2 * kBN, buf);
  }

  // ---- epilogue: O = acc * dv / l, LSE = (m - kPShift + log2 l) ln 2 --------
  const float lt = pair_sum(l);
  if (qi < N) {
    const float inv = v_descale / lt;
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
    if (grp == 0) LSE[head_q + qi] = (m2 - kPShift + fast_log2(lt)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const Fp8FwdArgs& a) {
  const int n_qblocks = (a.N + kBM - 1) / kBM;
  const long long items = (long long)n_qblocks * a.B * a.H;
  // c > 0 lets masked scores (-inf) give exp2(-inf) = 0 directly; a negative
  // product of scale and descales flips the sign of Q instead (exact in fp8)
  const float cs = a.scale * a.descale_q * a.descale_k;
  const float c = fmaxf(fabsf(cs) * kLog2e, 1e-30f);
  const int neg_q = cs < 0.f ? 1 : 0;
  return launch_kernel(fwd_fp8_kernel<D, CAUSAL>, dim3((unsigned)items), dim3(64 * kWaves), 0,
                       a.stream, static_cast<const uint8_t*>(a.q),
                       static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v),
                       static_cast<uint16_t*>(a.o), a.lse, a.B, a.H, a.Hkv, a.N, c, neg_q,
                       a.descale_v, n_qblocks);
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch_one<128, true>(a) : launch_one<128, false>(a);
  return a.causal ? launch_one<64, true>(a) : launch_one<64, false>(a);
}

}  // namespace fattn
