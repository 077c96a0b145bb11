// The libfattn C ABI: argument validation and dispatch.  Everything here runs
// on the host and returns before any launch when an argument is rejected.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fattn.h"
#include "launch.hpp"

// Fixed device scratch of the allocation-free backward (fa_bwd_noalloc): the
// per-row D terms, fp32 [B, H, N], for at most kNoAllocRows rows (16 MiB).
// Each GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` names a host-side stand-in, not a device address:
// its device address is looked up once per device (scratch_on_device) and
// only that pointer is handed to kernels.
constexpr long long kNoAllocRows = 1LL << 22;
static __device__ __align__(256) float scratch[kNoAllocRows];

namespace fattn {
namespace {

constexpr long double kMaxElems = 4611686018427387904.0L;   // 2^62
constexpr long long kMaxRows = 2147483647LL;                // 2^31 - 1
// The bf16 and fp8 forwards address one head's K and V, and the backward's
// dK/dV kernel one head's Q and dO, through a buffer resource with a 32-bit
// byte range and signed 32-bit offsets.  The last tile of a head forms row
// offsets up to 63 rows past N (those rows read as zero), so N + 64 rows must
// stay addressable: (N + 64) * d * elem bytes are at most 2^31 - 1.
constexpr long long kMaxHeadBytes = 2147483647LL;           // 2^31 - 1
constexpr long long kTileRowSlack = 64;                     // rows past N a key tile may address

struct Range {
  uintptr_t lo, hi;   // [lo, hi)
};

Range range_of(const void* p, long double bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Sizes shared by forward and backward.  Returns FA_OK, or the error code.
// `empty` is set when there is nothing to compute.
int check_sizes(int B, int H, int Hkv, int N, int d, bool* empty) {
  *empty = false;
  if (B < 0 || N < 0 || H <= 0 || Hkv <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if ((long double)B * H * N * d > kMaxElems) return FA_ERR_INVALID_ARG;
  if ((long long)B * H * N > kMaxRows) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B == 0 || N == 0) *empty = true;
  return FA_OK;
}

int check_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
              int B, int H, int Hkv, int N, int d, float scale, size_t elem, bool* empty,
              size_t out_elem = 0) {
  if (out_elem == 0) out_elem = elem;
  int st = check_sizes(B, H, Hkv, N, d, empty);
  if (st != FA_OK || *empty) return st;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (elem <= 2 && ((long long)N + kTileRowSlack) * d * (long long)elem > kMaxHeadBytes)
    return FA_ERR_INVALID_ARG;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return FA_ERR_INVALID_ARG;
  const long double qbytes = (long double)B * H * N * d * elem;
  const long double kvbytes = (long double)B * Hkv * N * d * elem;
  const long double obytes = (long double)B * H * N * d * out_elem;
  const long double lbytes = (long double)B * H * N * 4;
  const Range rq = range_of(q, qbytes), rk = range_of(k, kvbytes), rv = range_of(v, kvbytes);
  const Range ro = range_of(o, obytes), rl = range_of(lse, lbytes);
  if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv)) return FA_ERR_INVALID_ARG;
  if (overlaps(rl, rq) || overlaps(rl, rk) || overlaps(rl, rv) || overlaps(rl, ro))
    return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

}  // namespace
}  // namespace fattn

using namespace fattn;

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
  bool empty = false;
  int st = check_fwd(q, k, v, o, lse, B, H, Hkv, N, d, scale, 2, &empty);
  if (st != FA_OK || empty) return st;
  FwdArgs a{q, k, v, o, lse, B, H, Hkv, N, d, causal != 0, scale, stream};
  return status_of(launch_fwd_bf16(a));
}

extern "C" int fa_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Hkv, int N, int d, int window, float scale,
                            hipStream_t stream) {
  bool empty = false;
  int st = check_fwd(q, k, v, o, lse, B, H, Hkv, N, d, scale, 2, &empty);
  if (st != FA_OK || empty) return st;
  if (window < 1) return FA_ERR_INVALID_ARG;
  FwdArgs a{q, k, v, o, lse, B, H, Hkv, N, d, true, scale, stream, window};
  return status_of(launch_fwd_bf16(a));
}

extern "C" int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int Hkv, int N, int d, int causal, float scale,
                          float descale_q, float descale_k, float descale_v,
                          hipStream_t stream) {
  bool empty = false;
  int st = check_fwd(q, k, v, o, lse, B, H, Hkv, N, d, scale, 1, &empty, 2);
  if (st != FA_OK || empty) return st;
  for (float s : {descale_q, descale_k, descale_v})
    if (!(isfinite(s) && s > 0.f)) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale * descale_q * descale_k)) return FA_ERR_INVALID_ARG;
  Fp8FwdArgs a{q, k, v, o, lse, B, H, Hkv, N, d, causal != 0, scale,
               descale_q, descale_k, descale_v, stream};
  return status_of(launch_fwd_fp8(a));
}

extern "C" int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int H, int Hkv, int N, int d, int causal, float scale,
                          hipStream_t stream) {
  bool empty = false;
  int st = check_fwd(q, k, v, o, lse, B, H, Hkv, N, d, scale, 4, &empty);
  if (st != FA_OK || empty) return st;
  FwdArgs a{q, k, v, o, lse, B, H, Hkv, N, d, causal != 0, scale, stream};
  return status_of(launch_fwd_f32(a));
}

extern "C" size_t fa_bwd_workspace_bytes(int B, int H, int Hkv, int N, int d) {
  bool empty = false;
  if (check_sizes(B, H, Hkv, N, d, &empty) != FA_OK || empty) return 0;
  // D_i = sum_j P_ij dP_ij per query row (recomputed by the backward's D
  // pass), fp32, rounded up to 256 bytes.
  const size_t bytes = (size_t)B * H * N * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

namespace fattn {
namespace {

// Validation shared by fa_bwd and fa_bwd_noalloc; `ws_bytes` is the size of a
// caller-supplied workspace (checked for alignment and overlap), or 0 when the
// library's own scratch is used.
int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dO, const void* dq, const void* dk, const void* dv,
              const void* workspace, size_t ws_bytes, int B, int H, int Hkv, int N, int d,
              float scale, bool* empty) {
  int st = check_sizes(B, H, Hkv, N, d, empty);
  if (st != FA_OK || *empty) return st;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (((long long)N + kTileRowSlack) * d * 2 > kMaxHeadBytes) return FA_ERR_INVALID_ARG;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (ws_bytes && !workspace) return FA_ERR_INVALID_ARG;
  const void* p16[] = {q, k, v, o, dO, dq, dk, dv, workspace};
  for (const void* p : p16)
    if (p && !aligned(p, 16)) return FA_ERR_INVALID_ARG;
  if (!aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  const long double qb = (long double)B * H * N * d * 2;
  const long double kvb = (long double)B * Hkv * N * d * 2;
  const long double lb = (long double)B * H * N * 4;
  const Range in[] = {range_of(q, qb), range_of(k, kvb), range_of(v, kvb),
                      range_of(o, qb), range_of(lse, lb), range_of(dO, qb)};
  const Range out[] = {range_of(dq, qb), range_of(dk, kvb), range_of(dv, kvb),
                       range_of(workspace, (long double)ws_bytes)};
  const int n_out = ws_bytes ? 4 : 3;
  for (int i = 0; i < n_out; ++i) {
    for (const Range& r : in)
      if (overlaps(out[i], r)) return FA_ERR_INVALID_ARG;
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(out[i], out[j])) return FA_ERR_INVALID_ARG;
  }
  return FA_OK;
}

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream).  Looked up once per device, with that device
// current, and kept; later calls reuse it.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_on_device(hipStream_t stream, float** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace fattn

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dO, void* dq, void* dk, void* dv,
                      void* workspace, int B, int H, int Hkv, int N, int d, int causal,
                      float scale, hipStream_t stream) {
  bool empty = false;
  const size_t ws_bytes = fa_bwd_workspace_bytes(B, H, Hkv, N, d);
  int st = check_bwd(q, k, v, o, lse, dO, dq, dk, dv, workspace, ws_bytes, B, H, Hkv, N, d,
                     scale, &empty);
  if (st != FA_OK || empty) return st;
  BwdArgs a{q, k, v, o, lse, dO, dq, dk, dv, static_cast<float*>(workspace),
            B, H, Hkv, N, d, causal != 0, scale, stream};
  return status_of(launch_bwd_bf16(a));
}

extern "C" int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dO, void* dq, void* dk, void* dv,
                              int B, int H, int Hkv, int N, int d, int causal, float scale,
                              hipStream_t stream) {
  bool empty = false;
  int st = check_bwd(q, k, v, o, lse, dO, dq, dk, dv, nullptr, 0, B, H, Hkv, N, d, scale,
                     &empty);
  if (st != FA_OK || empty) return st;
  if ((long long)B * H * N > kNoAllocRows) return FA_ERR_TOO_LARGE;
  float* ws = nullptr;
  if (scratch_on_device(stream, &ws) != hipSuccess) return FA_ERR_HIP;
  BwdArgs a{q, k, v, o, lse, dO, dq, dk, dv, ws, B, H, Hkv, N, d, causal != 0, scale, stream};
  return status_of(launch_bwd_bf16(a));
}

extern "C" int fa_debug_counters(unsigned long long* out, int reset) {
  if (!out) return FA_ERR_INVALID_ARG;
  const hipError_t e = fwd_counters(out, reset != 0);
  if (e == hipErrorNotSupported) return FA_ERR_UNSUPPORTED;
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported configuration";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime refused the launch";
    case FA_ERR_TOO_LARGE:
      return "FA_ERR_TOO_LARGE: the problem exceeds the fixed scratch of fa_bwd_noalloc";
    default: return "unknown libfattn status";
  }
}
