// Internal launcher declarations (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace fattn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, N, d;
  bool causal;
  float scale;
  hipStream_t stream;
  int window = 0;   // > 0: local attention, query i sees keys i - window + 1 .. i
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dO;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // workspace: D_i = sum_j P_ij dP_ij (recomputed by the D pass), fp32 [B, H, N]
  int B, H, Hkv, N, d;
  bool causal;
  float scale;
  hipStream_t stream;
};

// FP8 (OCP e4m3) forward: q, k, v hold codes whose values are descale * e4m3(code).
struct Fp8FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;     // bf16
  float* lse;
  int B, H, Hkv, N, d;
  bool causal;
  float scale, descale_q, descale_k, descale_v;
  hipStream_t stream;
};

hipError_t launch_fwd_bf16(const FwdArgs& a);
// Debug builds (FATTN_DEVICE_COUNTERS): copy the bf16 forward's four device
// counters to `out` (synchronous) and optionally zero them; otherwise
// hipErrorNotSupported.
hipError_t fwd_counters(unsigned long long* out, bool reset);
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_bwd_bf16(const BwdArgs& a);

// Launch a kernel and return the runtime's verdict on exactly this launch.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                         hipStream_t stream, Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count mismatch");
  std::tuple<KArgs...> held(std::forward<Args>(args)...);
  return std::apply(
      [&](auto&... x) {
        void* argv[] = {static_cast<void*>(&x)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, shmem,
                               stream);
      },
      held);
}

}  // namespace fattn
