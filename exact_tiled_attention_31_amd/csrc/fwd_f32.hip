// Exact tiled attention forward with fp32 storage and fp32 arithmetic.
//
// Same method as the bf16 kernel ("LLM Architecture Refresh [3]: Flash
// Attention Is Exact", section 4, with the running statistics of section 2
// and the causal tile skip of section 7), for single-precision inputs where
// bf16 matrix cores would not meet fp32 accuracy.  One wave owns 64 query
// rows, one row per lane, with its query vector and output accumulator in
// VGPRs; 32-key tiles of K and V are staged in LDS and read by broadcast.
// Scores, the running max/sum and the output all stay in fp32.
#include "common.hpp"
#include "launch.hpp"

namespace fattn {
namespace {

constexpr int kRows = 64;   // query rows per workgroup (one wave)
constexpr int kKeys = 32;   // keys per tile
constexpr float kNegInf = -__builtin_inff();

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows, 1) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int B, int H, int Hkv, int N, float c,
    int n_qblocks) {
  __shared__ __attribute__((aligned(16))) float sK[kKeys * D];
  __shared__ __attribute__((aligned(16))) float sV[kKeys * D];

  const int tid = threadIdx.x;
  const int BH = B * H;
  const int item_q = blockIdx.x / BH;
  const int bh = blockIdx.x - item_q * BH;
  const int qb = CAUSAL ? (n_qblocks - 1 - item_q) : item_q;
  const int b = bh / H;
  const int h = bh - b * H;
  const int g = h / (H / Hkv);
  const int q0 = qb * kRows;
  const int qi = q0 + tid;

  const size_t head_q = (size_t)bh * N;
  const size_t head_kv = ((size_t)b * Hkv + g) * N;
  const float* Kh = K + head_kv * D;
  const float* Vh = V + head_kv * D;

  float q[D];
  float acc[D];
  {
    const float* qrow = Q + (head_q + (qi < N ? qi : 0)) * D;
#pragma unroll
    for (int i = 0; i < D; i += 4) {
      float4 x = qi < N ? *reinterpret_cast<const float4*>(qrow + i) : make_float4(0, 0, 0, 0);
      q[i] = x.x; q[i + 1] = x.y; q[i + 2] = x.z; q[i + 3] = x.w;
    }
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] = 0.f;
  }
  float m2 = kNegInf, l = 0.f;

  const int q_hi = min(q0 + kRows, N);
  int n_kt = (N + kKeys - 1) / kKeys;
  if (CAUSAL) n_kt = min(n_kt, (q_hi - 1) / kKeys + 1);

  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * kKeys;
    __syncthreads();
    for (int e = tid * 4; e < kKeys * D; e += kRows * 4) {
      const int row = e / D;
      const int cidx = e - row * D;
      const int kr = k0 + row;
      float4 kx = make_float4(0, 0, 0, 0), vx = make_float4(0, 0, 0, 0);
      if (kr < N) {
        kx = *reinterpret_cast<const float4*>(Kh + (size_t)kr * D + cidx);
        vx = *reinterpret_cast<const float4*>(Vh + (size_t)kr * D + cidx);
      }
      *reinterpret_cast<float4*>(&sK[e]) = kx;
      *reinterpret_cast<float4*>(&sV[e]) = vx;
    }
    __syncthreads();

    float t[kKeys];
    float tmax = kNegInf;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < D; i += 4) {
        const float4 kx = *reinterpret_cast<const float4*>(&sK[j * D + i]);
        dot = fmaf(q[i], kx.x, dot);
        dot = fmaf(q[i + 1], kx.y, dot);
        dot = fmaf(q[i + 2], kx.z, dot);
        dot = fmaf(q[i + 3], kx.w, dot);
      }
      const int kj = k0 + j;
      const bool visible = kj < N && (!CAUSAL || kj <= qi);
      t[j] = visible ? dot * c : kNegInf;
      tmax = fmaxf(tmax, t[j]);
    }
    const float m_new = fmaxf(m2, tmax);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float corr = fast_exp2(m2 - m_use);
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      t[j] = fast_exp2(t[j] - m_use);
      psum += t[j];
    }
    l = l * corr + psum;
#pragma unroll
    for (int i = 0; i < D; i += 4) {
      float a0 = acc[i] * corr, a1 = acc[i + 1] * corr, a2 = acc[i + 2] * corr,
            a3 = acc[i + 3] * corr;
#pragma unroll
      for (int j = 0; j < kKeys; ++j) {
        const float4 vx = *reinterpret_cast<const float4*>(&sV[j * D + i]);
        a0 = fmaf(t[j], vx.x, a0);
        a1 = fmaf(t[j], vx.y, a1);
        a2 = fmaf(t[j], vx.z, a2);
        a3 = fmaf(t[j], vx.w, a3);
      }
      acc[i] = a0; acc[i + 1] = a1; acc[i + 2] = a2; acc[i + 3] = a3;
    }
    m2 = m_new;
  }

  if (qi < N) {
    const float inv = 1.f / l;
    float* orow = O + (head_q + qi) * D;
#pragma unroll
    for (int i = 0; i < D; i += 4)
      *reinterpret_cast<float4*>(orow + i) =
          make_float4(acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv);
    LSE[head_q + qi] = (m2 + fast_log2(l)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const FwdArgs& a) {
  const int n_qblocks = (a.N + kRows - 1) / kRows;
  const long long items = (long long)n_qblocks * a.B * a.H;
  const float c = a.scale * kLog2e;
  return launch_kernel(fwd_f32_kernel<D, CAUSAL>, dim3((unsigned)items), dim3(kRows), 0,
                       a.stream, static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                       static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, a.B,
                       a.H, a.Hkv, a.N, c, n_qblocks);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch_one<128, true>(a) : launch_one<128, false>(a);
  return a.causal ? launch_one<64, true>(a) : launch_one<64, false>(a);
}

}  // namespace fattn
