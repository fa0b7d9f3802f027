// C ABI entry points (declared in include/fp8q.h): argument checks on the
// host, then the kernel launch on the caller's stream.  Nothing here touches
// the device before every check has passed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/fp8q.h"
#include "fp8q_internal.h"

namespace {

thread_local std::string g_last_error;

fp8q_status fail(fp8q_status st, const char *fn, const char *what) {
  g_last_error = std::string(fn) + ": " + what;
  return st;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The GEMM kernels address one tile's operands (at most 256 rows of K bytes)
// with 32-bit buffer offsets.
constexpr int64_t kMaxGemmK = (int64_t)1 << 22;

// Per-device check that the current device is a gfx950 (cached).
using fp8q::kMaxDevices;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];

fp8q_status check_device(const char *fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(FP8Q_EDEVICE, fn, e != hipSuccess ? hipGetErrorString(e) : "no usable HIP device");
  std::call_once(g_dev_once[dev], [dev]() {
    hipDeviceProp_t prop;
    g_dev_ok[dev] = (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                     std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 0;
  });
  if (!g_dev_ok[dev]) return fail(FP8Q_EDEVICE, fn, "current device is not gfx950 (MI355X)");
  return FP8Q_OK;
}

fp8q_status launched(hipError_t e, const char *fn) {
  if (e != hipSuccess) return fail(FP8Q_EHIP, fn, hipGetErrorString(e));
  return FP8Q_OK;
}

#define FP8Q_REQUIRE(cond, st, msg) \
  do {                              \
    if (!(cond)) return fail(st, __func__, msg); \
  } while (0)

}  // namespace

extern "C" {

fp8q_status fp8_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q,
                                float *scales, int mode, void *stream) {
  g_last_error.clear();
  FP8Q_REQUIRE(M >= 0 && K >= 0, FP8Q_EINVAL, "negative size");
  FP8Q_REQUIRE(mode == FP8Q_SCALE_AMAX || mode == FP8Q_SCALE_POW2, FP8Q_EINVAL, "unknown scale mode");
  FP8Q_REQUIRE(K > 0 && K % 128 == 0, FP8Q_ESHAPE, "K must be a positive multiple of 128");
  // eight lanes per block: M*K/128 blocks give 8*M*K/128 work-items, below 2^32
  FP8Q_REQUIRE(M <= (((int64_t)1 << 29) - 1) / (K / 128), FP8Q_ESHAPE, "M*K/128 must be below 2^29");
  if (M == 0) return FP8Q_OK;
  FP8Q_REQUIRE(x && q && scales, FP8Q_EINVAL, "null pointer");
  FP8Q_REQUIRE(aligned16(x) && aligned16(q) && aligned16(scales), FP8Q_EALIGN,
               "pointers must be 16-byte aligned");
  fp8q_status st = check_device(__func__);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_quant_act_1x128(x, M, K, q, scales, mode, (hipStream_t)stream), __func__);
}

fp8q_status fp8_rmsnorm_quant_1x128(const uint16_t *x, const uint16_t *gamma, int64_t M, int64_t K, float eps,
                                    uint8_t *q, float *scales, int mode, void *stream) {
  g_last_error.clear();
  FP8Q_REQUIRE(M >= 0 && K >= 0, FP8Q_EINVAL, "negative size");
  FP8Q_REQUIRE(mode == FP8Q_SCALE_AMAX || mode == FP8Q_SCALE_POW2, FP8Q_EINVAL, "unknown scale mode");
  FP8Q_REQUIRE(std::isfinite(eps) && eps >= 0.0f, FP8Q_EINVAL, "eps must be finite and >= 0");
  FP8Q_REQUIRE(K > 0 && K % 128 == 0 && K <= 8192, FP8Q_ESHAPE, "K must be a multiple of 128 in [128, 8192]");
  // one wave of 64 lanes per row: the launch's 64*M work-items must stay
  // below 2^32, the limit of a dispatch's grid size
  FP8Q_REQUIRE(M < ((int64_t)1 << 26), FP8Q_ESHAPE, "M must be below 2^26");
  if (M == 0) return FP8Q_OK;
  FP8Q_REQUIRE(x && gamma && q && scales, FP8Q_EINVAL, "null pointer");
  FP8Q_REQUIRE(aligned16(x) && aligned16(gamma) && aligned16(q) && aligned16(scales), FP8Q_EALIGN,
               "pointers must be 16-byte aligned");
  fp8q_status st = check_device(__func__);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_rmsnorm_quant_1x128(x, gamma, M, K, eps, q, scales, mode, (hipStream_t)stream),
                  __func__);
}

fp8q_status fp8_quant_weight_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q,
                                     float *scales, int mode, void *stream) {
  g_last_error.clear();
  FP8Q_REQUIRE(N >= 0 && K >= 0, FP8Q_EINVAL, "negative size");
  FP8Q_REQUIRE(mode == FP8Q_SCALE_AMAX || mode == FP8Q_SCALE_POW2, FP8Q_EINVAL, "unknown scale mode");
  FP8Q_REQUIRE(K > 0 && K % 128 == 0, FP8Q_ESHAPE, "K must be a positive multiple of 128");
  FP8Q_REQUIRE(N % 128 == 0, FP8Q_ESHAPE, "N must be a multiple of 128");
  if (N == 0) return FP8Q_OK;
  FP8Q_REQUIRE(w && q && scales, FP8Q_EINVAL, "null pointer");
  FP8Q_REQUIRE(aligned16(w) && aligned16(q) && aligned16(scales), FP8Q_EALIGN,
               "pointers must be 16-byte aligned");
  fp8q_status st = check_device(__func__);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_quant_weight_128x128(w, N, K, q, scales, mode, (hipStream_t)stream),
                  __func__);
}

fp8q_status fp8_quant_weight_128x128_batched(const fp8q_weight_job *jobs, int32_t count, int64_t total_tiles,
                                             int mode, void *stream) {
  g_last_error.clear();
  FP8Q_REQUIRE(count >= 0 && total_tiles >= 0, FP8Q_EINVAL, "negative count or tile total");
  FP8Q_REQUIRE(mode == FP8Q_SCALE_AMAX || mode == FP8Q_SCALE_POW2, FP8Q_EINVAL, "unknown scale mode");
  FP8Q_REQUIRE(total_tiles < ((int64_t)1 << 31), FP8Q_ESHAPE, "more than 2^31 - 1 tiles in one batch");
  if (count == 0 || total_tiles == 0) return FP8Q_OK;
  FP8Q_REQUIRE(jobs != nullptr, FP8Q_EINVAL, "null pointer");
  FP8Q_REQUIRE((reinterpret_cast<uintptr_t>(jobs) & 7u) == 0, FP8Q_EALIGN, "job table must be 8-byte aligned");
  fp8q_status st = check_device(__func__);
  if (st != FP8Q_OK) return st;
  {
    // the kernel reads the table: it must be memory the device can read
    hipPointerAttribute_t attr;
    const hipError_t e = hipPointerGetAttributes(&attr, jobs);
    (void)hipGetLastError();  // an unknown pointer leaves an error that would surface at the launch
    FP8Q_REQUIRE(e == hipSuccess && (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged),
                 FP8Q_EINVAL, "job table must be in device memory");
  }
  return launched(fp8q::launch_quant_weight_batched(jobs, count, total_tiles, mode, (hipStream_t)stream),
                  __func__);
}

fp8q_status fp8_quant_act_dual(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *scales,
                               uint8_t *q_t, float *scales_t, int mode, void *stream) {
  g_last_error.clear();
  FP8Q_REQUIRE(M >= 0 && K >= 0, FP8Q_EINVAL, "negative size");
  FP8Q_REQUIRE(mode == FP8Q_SCALE_AMAX || mode == FP8Q_SCALE_POW2, FP8Q_EINVAL, "unknown scale mode");
  FP8Q_REQUIRE(K > 0 && K % 128 == 0, FP8Q_ESHAPE, "K must be a positive multiple of 128");
  FP8Q_REQUIRE((q == nullptr) == (scales == nullptr), FP8Q_EINVAL,
               "q and scales must both be given or both be null");
  if (M == 0) return FP8Q_OK;
  FP8Q_REQUIRE(x && q_t && scales_t, FP8Q_EINVAL, "null pointer");
  FP8Q_REQUIRE(aligned16(x) && aligned16(q) && aligned16(scales) && aligned16(q_t) && aligned16(scales_t),
               FP8Q_EALIGN, "pointers must be 16-byte aligned");
  fp8q_status st = check_device(__func__);
  if (st != FP8Q_OK) return st;
  return launched(
      fp8q::launch_quant_dual(x, M, K, q, scales, q_t, scales_t, mode, false, (hipStream_t)stream), __func__);
}

fp8q_status fp8_quant_weight_128x128_dual(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *scales,
                                          uint8_t *q_t, float *scales_t, int mode, void *stream) {
  g_last_error.clear();
  FP8Q_REQUIRE(N >= 0 && K >= 0, FP8Q_EINVAL, "negative size");
  FP8Q_REQUIRE(mode == FP8Q_SCALE_AMAX || mode == FP8Q_SCALE_POW2, FP8Q_EINVAL, "unknown scale mode");
  FP8Q_REQUIRE(K > 0 && K % 128 == 0, FP8Q_ESHAPE, "K must be a positive multiple of 128");
  FP8Q_REQUIRE(N % 128 == 0, FP8Q_ESHAPE, "N must be a multiple of 128");
  FP8Q_REQUIRE((q == nullptr) == (scales == nullptr), FP8Q_EINVAL,
               "q and scales must both be given or both be null");
  if (N == 0) return FP8Q_OK;
  FP8Q_REQUIRE(w && q_t && scales_t, FP8Q_EINVAL, "null pointer");
  FP8Q_REQUIRE(aligned16(w) && aligned16(q) && aligned16(scales) && aligned16(q_t) && aligned16(scales_t),
               FP8Q_EALIGN, "pointers must be 16-byte aligned");
  fp8q_status st = check_device(__func__);
  if (st != FP8Q_OK) return st;
  return launched(
      fp8q::launch_quant_dual(w, N, K, q, scales, q_t, scales_t, mode, true, (hipStream_t)stream), __func__);
}

}  // extern "C"

namespace {

fp8q_status gemm_entry(const char *fn, const uint8_t *a_q, const float *a_s, const uint8_t *b_q,
                       const float *b_s, uint16_t *y, int64_t M, int64_t N, int64_t K, bool pow2,
                       void *stream) {
  g_last_error.clear();
  if (!(M >= 0 && N >= 0 && K >= 0)) return fail(FP8Q_EINVAL, fn, "negative size");
  if (!(K > 0 && K % 128 == 0)) return fail(FP8Q_ESHAPE, fn, "K must be a positive multiple of 128");
  if (N % 128 != 0) return fail(FP8Q_ESHAPE, fn, "N must be a multiple of 128");
  if (K > kMaxGemmK) return fail(FP8Q_ESHAPE, fn, "K larger than 4194304");
  if (!(M <= (int64_t)1 << 31 && N <= (int64_t)1 << 31)) return fail(FP8Q_EINVAL, fn, "M or N too large");
  if (M == 0 || N == 0) return FP8Q_OK;
  if (!(a_q && a_s && b_q && b_s && y)) return fail(FP8Q_EINVAL, fn, "null pointer");
  if (!(aligned16(a_q) && aligned16(a_s) && aligned16(b_q) && aligned16(b_s) && aligned16(y)))
    return fail(FP8Q_EALIGN, fn, "pointers must be 16-byte aligned");
  fp8q_status st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_blockscaled_gemm(a_q, a_s, b_q, b_s, y, M, N, K, pow2, (hipStream_t)stream), fn);
}

fp8q_status gemm_quant_entry(const char *fn, const uint8_t *a_q, const float *a_s, const uint8_t *b_q,
                             const float *b_s, uint8_t *y_q, float *y_s, int64_t M, int64_t N, int64_t K, int mode,
                             void *stream) {
  g_last_error.clear();
  if (mode != FP8Q_SCALE_AMAX && mode != FP8Q_SCALE_POW2) return fail(FP8Q_EINVAL, fn, "unknown mode");
  if (!(M >= 0 && N >= 0 && K >= 0)) return fail(FP8Q_EINVAL, fn, "negative size");
  if (!(K > 0 && K % 128 == 0)) return fail(FP8Q_ESHAPE, fn, "K must be a positive multiple of 128");
  if (N % 128 != 0) return fail(FP8Q_ESHAPE, fn, "N must be a multiple of 128");
  if (K > kMaxGemmK) return fail(FP8Q_ESHAPE, fn, "K larger than 4194304");
  if (!(M <= (int64_t)1 << 31 && N <= (int64_t)1 << 31)) return fail(FP8Q_EINVAL, fn, "M or N too large");
  if (M == 0 || N == 0) return FP8Q_OK;
  if (!(a_q && a_s && b_q && b_s && y_q && y_s)) return fail(FP8Q_EINVAL, fn, "null pointer");
  if (!(aligned16(a_q) && aligned16(a_s) && aligned16(b_q) && aligned16(b_s) && aligned16(y_q) && aligned16(y_s)))
    return fail(FP8Q_EALIGN, fn, "pointers must be 16-byte aligned");
  fp8q_status st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return launched(
      fp8q::launch_blockscaled_gemm_quant(a_q, a_s, b_q, b_s, y_q, y_s, M, N, K, mode, (hipStream_t)stream), fn);
}

fp8q_status swiglu_entry(const char *fn, const uint8_t *a_q, const float *a_s, const uint8_t *b_q,
                         const float *b_s, uint8_t *h_q, float *h_s, int64_t M, int64_t F, int64_t K, int mode,
                         void *stream) {
  g_last_error.clear();
  if (mode != FP8Q_SCALE_AMAX && mode != FP8Q_SCALE_POW2) return fail(FP8Q_EINVAL, fn, "unknown mode");
  if (!(M >= 0 && F >= 0 && K >= 0)) return fail(FP8Q_EINVAL, fn, "negative size");
  if (!(K > 0 && K % 128 == 0)) return fail(FP8Q_ESHAPE, fn, "K must be a positive multiple of 128");
  if (F % 128 != 0) return fail(FP8Q_ESHAPE, fn, "F must be a multiple of 128");
  if (K > kMaxGemmK) return fail(FP8Q_ESHAPE, fn, "K larger than 4194304");
  if (!(M <= (int64_t)1 << 31 && F <= (int64_t)1 << 30)) return fail(FP8Q_EINVAL, fn, "M or F too large");
  if (M == 0 || F == 0) return FP8Q_OK;
  if (!(a_q && a_s && b_q && b_s && h_q && h_s)) return fail(FP8Q_EINVAL, fn, "null pointer");
  if (!(aligned16(a_q) && aligned16(a_s) && aligned16(b_q) && aligned16(b_s) && aligned16(h_q) && aligned16(h_s)))
    return fail(FP8Q_EALIGN, fn, "pointers must be 16-byte aligned");
  fp8q_status st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return launched(
      fp8q::launch_blockscaled_gemm_swiglu_quant(a_q, a_s, b_q, b_s, h_q, h_s, M, F, K, mode, (hipStream_t)stream),
      fn);
}

fp8q_status wgrad_entry(const char *fn, const uint8_t *a_q, const float *a_s, const uint8_t *b_q,
                        const float *b_s, uint16_t *y, int64_t M, int64_t N, int64_t K, bool pow2, void *stream) {
  g_last_error.clear();
  if (!(M >= 0 && N >= 0 && K >= 0)) return fail(FP8Q_EINVAL, fn, "negative size");
  if (!(K > 0 && K % 128 == 0)) return fail(FP8Q_ESHAPE, fn, "K must be a positive multiple of 128");
  if (N % 128 != 0) return fail(FP8Q_ESHAPE, fn, "N must be a multiple of 128");
  if (K > kMaxGemmK) return fail(FP8Q_ESHAPE, fn, "K larger than 4194304");
  if (!(M <= (int64_t)1 << 31 && N <= (int64_t)1 << 31)) return fail(FP8Q_EINVAL, fn, "M or N too large");
  if (M == 0 || N == 0) return FP8Q_OK;
  if (!(a_q && a_s && b_q && b_s && y)) return fail(FP8Q_EINVAL, fn, "null pointer");
  if (!(aligned16(a_q) && aligned16(a_s) && aligned16(b_q) && aligned16(b_s) && aligned16(y)))
    return fail(FP8Q_EALIGN, fn, "pointers must be 16-byte aligned");
  fp8q_status st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_blockscaled_gemm_wgrad(a_q, a_s, b_q, b_s, y, M, N, K, pow2, (hipStream_t)stream),
                  fn);
}

fp8q_status grouped_entry(const char *fn, const uint8_t *a_q, const float *a_s, const uint8_t *b_q,
                          const float *b_s, const int32_t *group_offsets, int32_t G, int64_t M_total, int64_t N,
                          int64_t K, uint16_t *y, bool pow2, void *stream) {
  g_last_error.clear();
  if (G < 1) return fail(FP8Q_EINVAL, fn, "G must be >= 1");
  if (!(M_total >= 0 && N >= 0 && K >= 0)) return fail(FP8Q_EINVAL, fn, "negative size");
  if (!(K > 0 && K % 128 == 0)) return fail(FP8Q_ESHAPE, fn, "K must be a positive multiple of 128");
  if (N % 128 != 0) return fail(FP8Q_ESHAPE, fn, "N must be a multiple of 128");
  if (K > kMaxGemmK) return fail(FP8Q_ESHAPE, fn, "K larger than 4194304");
  if (!(M_total < ((int64_t)1 << 31) && N <= ((int64_t)1 << 31)))
    return fail(FP8Q_EINVAL, fn, "M_total or N too large");
  if (M_total == 0 || N == 0) return FP8Q_OK;
  if (!(a_q && a_s && b_q && b_s && y && group_offsets)) return fail(FP8Q_EINVAL, fn, "null pointer");
  if (!(aligned16(a_q) && aligned16(a_s) && aligned16(b_q) && aligned16(b_s) && aligned16(y) &&
        aligned16(group_offsets)))
    return fail(FP8Q_EALIGN, fn, "pointers must be 16-byte aligned");
  fp8q_status st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_grouped_gemm(a_q, a_s, b_q, b_s, group_offsets, G, M_total, N, K, y, pow2,
                                            (hipStream_t)stream),
                  fn);
}

fp8q_status gather_entry(const char *fn, const uint8_t *a_q, const float *a_s, int64_t T, const uint8_t *b_q,
                         const float *b_s, const int32_t *group_offsets, const int32_t *row_index, int32_t G,
                         int64_t M_total, int64_t N, int64_t K, uint16_t *y, int mode, void *stream) {
  g_last_error.clear();
  if (mode != FP8Q_SCALE_AMAX && mode != FP8Q_SCALE_POW2) return fail(FP8Q_EINVAL, fn, "unknown mode");
  if (G < 1) return fail(FP8Q_EINVAL, fn, "G must be >= 1");
  if (!(T >= 0 && M_total >= 0 && N >= 0 && K >= 0)) return fail(FP8Q_EINVAL, fn, "negative size");
  if (!(K > 0 && K % 128 == 0)) return fail(FP8Q_ESHAPE, fn, "K must be a positive multiple of 128");
  if (N % 128 != 0) return fail(FP8Q_ESHAPE, fn, "N must be a multiple of 128");
  if (K > kMaxGemmK) return fail(FP8Q_ESHAPE, fn, "K larger than 4194304");
  if (!(M_total < ((int64_t)1 << 31) && N <= ((int64_t)1 << 31)))
    return fail(FP8Q_EINVAL, fn, "M_total or N too large");
  // Gathered rows are addressed by 32-bit byte offsets into the token matrix.
  if (T >= ((int64_t)1 << 31) / K) return fail(FP8Q_ESHAPE, fn, "token matrix T*K must be below 2^31 bytes");
  if (M_total == 0 || N == 0) return FP8Q_OK;
  if (T == 0) return fail(FP8Q_EINVAL, fn, "T must be positive when there are routed rows");
  if (!(a_q && a_s && b_q && b_s && y && group_offsets && row_index))
    return fail(FP8Q_EINVAL, fn, "null pointer");
  if (!(aligned16(a_q) && aligned16(a_s) && aligned16(b_q) && aligned16(b_s) && aligned16(y) &&
        aligned16(group_offsets) && aligned16(row_index)))
    return fail(FP8Q_EALIGN, fn, "pointers must be 16-byte aligned");
  fp8q_status st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_grouped_gemm_gather(a_q, a_s, T, b_q, b_s, group_offsets, row_index, G, M_total, N,
                                                   K, y, mode == FP8Q_SCALE_POW2, (hipStream_t)stream),
                  fn);
}

fp8q_status grouped_swiglu_entry(const char *fn, const uint8_t *a_q, const float *a_s, int64_t T,
                                 const uint8_t *b_q, const float *b_s, const int32_t *group_offsets,
                                 const int32_t *row_index, int32_t G, int64_t M_total, int64_t F, int64_t K,
                                 uint8_t *h_q, float *h_s, int mode, void *stream) {
  g_last_error.clear();
  if (mode != FP8Q_SCALE_AMAX && mode != FP8Q_SCALE_POW2) return fail(FP8Q_EINVAL, fn, "unknown mode");
  if (G < 1) return fail(FP8Q_EINVAL, fn, "G must be >= 1");
  if (!(T >= 0 && M_total >= 0 && F >= 0 && K >= 0)) return fail(FP8Q_EINVAL, fn, "negative size");
  if (!(K > 0 && K % 128 == 0)) return fail(FP8Q_ESHAPE, fn, "K must be a positive multiple of 128");
  if (F % 128 != 0) return fail(FP8Q_ESHAPE, fn, "F must be a multiple of 128");
  if (K > kMaxGemmK) return fail(FP8Q_ESHAPE, fn, "K larger than 4194304");
  if (!(M_total < ((int64_t)1 << 31) && F <= ((int64_t)1 << 30)))
    return fail(FP8Q_EINVAL, fn, "M_total or F too large");
  // Gathered rows are addressed by 32-bit byte offsets into the token matrix.
  if (row_index && T >= ((int64_t)1 << 31) / K)
    return fail(FP8Q_ESHAPE, fn, "token matrix T*K must be below 2^31 bytes");
  if (M_total == 0 || F == 0) return FP8Q_OK;
  if (row_index && T == 0) return fail(FP8Q_EINVAL, fn, "T must be positive when there are routed rows");
  if (!(a_q && a_s && b_q && b_s && h_q && h_s && group_offsets)) return fail(FP8Q_EINVAL, fn, "null pointer");
  if (!(aligned16(a_q) && aligned16(a_s) && aligned16(b_q) && aligned16(b_s) && aligned16(h_q) && aligned16(h_s) &&
        aligned16(group_offsets) && aligned16(row_index)))
    return fail(FP8Q_EALIGN, fn, "pointers must be 16-byte aligned");
  fp8q_status st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_grouped_gemm_swiglu_quant(a_q, a_s, T, b_q, b_s, group_offsets, row_index, G,
                                                         M_total, F, K, h_q, h_s, mode, (hipStream_t)stream),
                  fn);
}

}  // namespace

extern "C" {

fp8q_status fp8_blockscaled_gemm(const uint8_t *a_q, const float *a_s, const uint8_t *b_q,
                                 const float *b_s, uint16_t *y, int64_t M, int64_t N, int64_t K,
                                 void *stream) {
  return gemm_entry(__func__, a_q, a_s, b_q, b_s, y, M, N, K, false, stream);
}

fp8q_status fp8_blockscaled_gemm_pow2(const uint8_t *a_q, const float *a_s, const uint8_t *b_q,
                                      const float *b_s, uint16_t *y, int64_t M, int64_t N, int64_t K,
                                      void *stream) {
  return gemm_entry(__func__, a_q, a_s, b_q, b_s, y, M, N, K, true, stream);
}

fp8q_status fp8_blockscaled_gemm_quant(const uint8_t *a_q, const float *a_s, const uint8_t *b_q,
                                       const float *b_s, uint8_t *y_q, float *y_s, int64_t M, int64_t N,
                                       int64_t K, int mode, void *stream) {
  return gemm_quant_entry(__func__, a_q, a_s, b_q, b_s, y_q, y_s, M, N, K, mode, stream);
}

fp8q_status fp8_blockscaled_gemm_swiglu_quant(const uint8_t *a_q, const float *a_s, const uint8_t *b_q,
                                              const float *b_s, uint8_t *h_q, float *h_s, int64_t M, int64_t F,
                                              int64_t K, int mode, void *stream) {
  return swiglu_entry(__func__, a_q, a_s, b_q, b_s, h_q, h_s, M, F, K, mode, stream);
}

fp8q_status fp8_blockscaled_gemm_wgrad(const uint8_t *a_q, const float *a_s, const uint8_t *b_q,
                                       const float *b_s, uint16_t *y, int64_t M, int64_t N, int64_t K,
                                       void *stream) {
  return wgrad_entry(__func__, a_q, a_s, b_q, b_s, y, M, N, K, false, stream);
}

fp8q_status fp8_blockscaled_gemm_wgrad_pow2(const uint8_t *a_q, const float *a_s, const uint8_t *b_q,
                                            const float *b_s, uint16_t *y, int64_t M, int64_t N, int64_t K,
                                            void *stream) {
  return wgrad_entry(__func__, a_q, a_s, b_q, b_s, y, M, N, K, true, stream);
}

fp8q_status fp8_grouped_gemm(const uint8_t *a_q, const float *a_s, const uint8_t *b_q,
                             const float *b_s, const int32_t *group_offsets, int32_t G,
                             int64_t M_total, int64_t N, int64_t K, uint16_t *y, void *stream) {
  return grouped_entry(__func__, a_q, a_s, b_q, b_s, group_offsets, G, M_total, N, K, y, false, stream);
}

fp8q_status fp8_grouped_gemm_pow2(const uint8_t *a_q, const float *a_s, const uint8_t *b_q,
                                  const float *b_s, const int32_t *group_offsets, int32_t G,
                                  int64_t M_total, int64_t N, int64_t K, uint16_t *y, void *stream) {
  return grouped_entry(__func__, a_q, a_s, b_q, b_s, group_offsets, G, M_total, N, K, y, true, stream);
}

fp8q_status fp8_grouped_gemm_gather(const uint8_t *a_q, const float *a_s, int64_t T, const uint8_t *b_q,
                                    const float *b_s, const int32_t *group_offsets, const int32_t *row_index,
                                    int32_t G, int64_t M_total, int64_t N, int64_t K, uint16_t *y, int mode,
                                    void *stream) {
  return gather_entry(__func__, a_q, a_s, T, b_q, b_s, group_offsets, row_index, G, M_total, N, K, y, mode,
                      stream);
}

fp8q_status fp8_grouped_gemm_swiglu_quant(const uint8_t *a_q, const float *a_s, int64_t T, const uint8_t *b_q,
                                          const float *b_s, const int32_t *group_offsets, const int32_t *row_index,
                                          int32_t G, int64_t M_total, int64_t F, int64_t K, uint8_t *h_q,
                                          float *h_s, int mode, void *stream) {
  return grouped_swiglu_entry(__func__, a_q, a_s, T, b_q, b_s, group_offsets, row_index, G, M_total, F, K, h_q, h_s,
                              mode, stream);
}

fp8q_status fp8_kv_cache_append(const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos,
                                uint8_t *k_cache, float *k_scale, uint8_t *v_cache, float *v_scale, int32_t B,
                                int32_t Hkv, int64_t S, int mode, void *stream) {
  g_last_error.clear();
  FP8Q_REQUIRE(mode == FP8Q_SCALE_AMAX || mode == FP8Q_SCALE_POW2, FP8Q_EINVAL, "unknown scale mode");
  FP8Q_REQUIRE(B >= 0 && Hkv >= 0 && S >= 0, FP8Q_EINVAL, "negative size");
  if (B == 0 || Hkv == 0) return FP8Q_OK;
  FP8Q_REQUIRE(k_new && v_new && pos && k_cache && k_scale && v_cache && v_scale, FP8Q_EINVAL, "null pointer");
  FP8Q_REQUIRE(aligned16(k_new) && aligned16(v_new) && aligned16(pos) && aligned16(k_cache) &&
                   aligned16(k_scale) && aligned16(v_cache) && aligned16(v_scale),
               FP8Q_EALIGN, "pointers must be 16-byte aligned");
  fp8q_status st = check_device(__func__);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_kv_cache_append(k_new, v_new, pos, k_cache, k_scale, v_cache, v_scale, B, 1, Hkv, S,
                                               mode, (hipStream_t)stream),
                  __func__);
}

fp8q_status fp8_kv_cache_append_tokens(const uint16_t *k_new, const uint16_t *v_new, const int32_t *start,
                                       uint8_t *k_cache, float *k_scale, uint8_t *v_cache, float *v_scale,
                                       int32_t B, int32_t T, int32_t Hkv, int64_t S, int mode, void *stream) {
  g_last_error.clear();
  FP8Q_REQUIRE(mode == FP8Q_SCALE_AMAX || mode == FP8Q_SCALE_POW2, FP8Q_EINVAL, "unknown scale mode");
  FP8Q_REQUIRE(B >= 0 && T >= 0 && Hkv >= 0 && S >= 0, FP8Q_EINVAL, "negative size");
  if ((int64_t)B * T * Hkv == 0) return FP8Q_OK;
  FP8Q_REQUIRE((int64_t)B * T * Hkv < ((int64_t)1 << 34), FP8Q_ESHAPE, "B*T*Hkv must be below 2^34");
  FP8Q_REQUIRE(k_new && v_new && start && k_cache && k_scale && v_cache && v_scale, FP8Q_EINVAL, "null pointer");
  FP8Q_REQUIRE(aligned16(k_new) && aligned16(v_new) && aligned16(start) && aligned16(k_cache) &&
                   aligned16(k_scale) && aligned16(v_cache) && aligned16(v_scale),
               FP8Q_EALIGN, "pointers must be 16-byte aligned");
  fp8q_status st = check_device(__func__);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_kv_cache_append(k_new, v_new, start, k_cache, k_scale, v_cache, v_scale, B, T, Hkv,
                                               S, mode, (hipStream_t)stream),
                  __func__);
}

fp8q_status fp8_attention_prefill(const uint8_t *q_q, const float *q_s, const uint8_t *k_cache,
                                  const float *k_scale, const uint8_t *v_cache, const float *v_scale,
                                  const int32_t *start, uint16_t *out, int32_t B, int32_t T, int32_t Hq,
                                  int32_t Hkv, int64_t S, void *stream) {
  g_last_error.clear();
  FP8Q_REQUIRE(B >= 0 && T >= 0 && Hq >= 0 && Hkv >= 0 && S >= 0, FP8Q_EINVAL, "negative size");
  FP8Q_REQUIRE(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0, FP8Q_ESHAPE, "Hq must be a positive multiple of Hkv");
  if ((int64_t)B * T * Hq == 0) return FP8Q_OK;
  FP8Q_REQUIRE((int64_t)(T + 63) / 64 * B * Hq < ((int64_t)1 << 31) && S < ((int64_t)1 << 31), FP8Q_ESHAPE,
               "ceil(T/64)*B*Hq and S must be below 2^31");
  FP8Q_REQUIRE(q_q && q_s && k_cache && k_scale && v_cache && v_scale && start && out, FP8Q_EINVAL,
               "null pointer");
  FP8Q_REQUIRE(aligned16(q_q) && aligned16(q_s) && aligned16(k_cache) && aligned16(k_scale) && aligned16(v_cache) &&
                   aligned16(v_scale) && aligned16(start) && aligned16(out),
               FP8Q_EALIGN, "pointers must be 16-byte aligned");
  fp8q_status st = check_device(__func__);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_attention_prefill(q_q, q_s, k_cache, k_scale, v_cache, v_scale, start, out, B, T, Hq,
                                                 Hkv, S, (hipStream_t)stream),
                  __func__);
}

int64_t fp8_attention_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int64_t S) {
  if (B < 0 || Hq < 0 || Hkv < 1 || S < 0) return 0;
  int64_t nch, ct;
  fp8q::attention_decode_split((int64_t)B * Hkv, S, nch, ct);
  return nch <= 1 ? 0 : (int64_t)B * Hq * nch * (128 + 2) * (int64_t)sizeof(float);
}

fp8q_status fp8_attention_decode(const uint8_t *q_q, const float *q_s, const uint8_t *k_cache,
                                 const float *k_scale, const uint8_t *v_cache, const float *v_scale,
                                 const int32_t *seq_len, uint16_t *out, int32_t B, int32_t Hq, int32_t Hkv,
                                 int64_t S, void *workspace, int64_t workspace_bytes, void *stream) {
  g_last_error.clear();
  FP8Q_REQUIRE(B >= 0 && Hq >= 0 && Hkv >= 0 && S >= 0, FP8Q_EINVAL, "negative size");
  FP8Q_REQUIRE(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0, FP8Q_ESHAPE, "Hq must be a positive multiple of Hkv");
  const int32_t grp = Hq / Hkv;
  FP8Q_REQUIRE(grp == 1 || grp == 2 || grp == 4 || grp == 8, FP8Q_ESHAPE, "Hq / Hkv must be 1, 2, 4 or 8");
  // 256 lanes per (sequence, key/value head) workgroup: below 2^32 work-items
  FP8Q_REQUIRE((int64_t)B * Hkv < ((int64_t)1 << 24), FP8Q_ESHAPE, "B * Hkv must be below 2^24");
  if (B == 0) return FP8Q_OK;
  FP8Q_REQUIRE(q_q && q_s && k_cache && k_scale && v_cache && v_scale && seq_len && out, FP8Q_EINVAL,
               "null pointer");
  FP8Q_REQUIRE(aligned16(q_q) && aligned16(q_s) && aligned16(k_cache) && aligned16(k_scale) &&
                   aligned16(v_cache) && aligned16(v_scale) && aligned16(seq_len) && aligned16(out) &&
                   aligned16(workspace),
               FP8Q_EALIGN, "pointers must be 16-byte aligned");
  FP8Q_REQUIRE(workspace == nullptr || workspace_bytes >= fp8_attention_decode_workspace_size(B, Hq, Hkv, S),
               FP8Q_EINVAL, "workspace smaller than fp8_attention_decode_workspace_size()");
  fp8q_status st = check_device(__func__);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_attention_decode(q_q, q_s, k_cache, k_scale, v_cache, v_scale, seq_len, out, B, Hq,
                                                Hkv, S, static_cast<float *>(workspace), (hipStream_t)stream),
                  __func__);
}

int32_t fp8_blockscaled_gemm_tile_plan(int64_t M, int64_t N, int swiglu, int64_t *rows_large) {
  if (M < 1 || N < 128 || N % 128 != 0 || M > ((int64_t)1 << 31) || N > ((int64_t)1 << 31)) return -1;
  int64_t rows, panels;
  fp8q::dense_tile_plan(M, N, swiglu == 0, rows, panels);
  if (rows_large) *rows_large = rows;
  return (int32_t)panels;
}

int64_t fp8_moe_permute_workspace_size(int64_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1 || E > 1024 || T > (((int64_t)1 << 31) - 1) / k) return 0;
  return fp8q::moe_permute_workspace_bytes(T * k, E);
}

fp8q_status fp8_moe_permute(const int32_t *expert_ids, int64_t T, int32_t k, int32_t E, int32_t n_shared,
                            int32_t *group_offsets, int32_t *row_index, int32_t *entry_row, void *workspace,
                            int64_t workspace_bytes, void *stream) {
  g_last_error.clear();
  FP8Q_REQUIRE(T >= 0 && n_shared >= 0, FP8Q_EINVAL, "negative size");
  FP8Q_REQUIRE(k >= 1, FP8Q_EINVAL, "k must be at least 1");
  FP8Q_REQUIRE(E >= 1 && E <= 1024, FP8Q_ESHAPE, "E must be in [1, 1024]");
  FP8Q_REQUIRE(T <= (((int64_t)1 << 31) - 1) / ((int64_t)k + n_shared), FP8Q_ESHAPE,
               "T * (k + n_shared) must be below 2^31");
  FP8Q_REQUIRE(group_offsets && workspace, FP8Q_EINVAL, "null pointer");
  FP8Q_REQUIRE(T == 0 || (expert_ids && row_index), FP8Q_EINVAL, "null pointer");
  FP8Q_REQUIRE(aligned16(expert_ids) && aligned16(group_offsets) && aligned16(row_index) && aligned16(entry_row) &&
                   aligned16(workspace),
               FP8Q_EALIGN, "pointers must be 16-byte aligned");
  FP8Q_REQUIRE(workspace_bytes >= fp8_moe_permute_workspace_size(T, k, E), FP8Q_EINVAL,
               "workspace smaller than fp8_moe_permute_workspace_size()");
  fp8q_status st = check_device(__func__);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_moe_permute(expert_ids, T, k, E, n_shared, group_offsets, row_index, entry_row,
                                           workspace, (hipStream_t)stream),
                  __func__);
}

fp8q_status fp8_attention_decode_noalloc(const uint8_t *q_q, const float *q_s, const uint8_t *k_cache,
                                         const float *k_scale, const uint8_t *v_cache, const float *v_scale,
                                         const int32_t *seq_len, uint16_t *out, int32_t B, int32_t Hq,
                                         int32_t Hkv, int64_t S, void *stream) {
  g_last_error.clear();
  FP8Q_REQUIRE(B >= 0 && Hq >= 0 && Hkv >= 0 && S >= 0, FP8Q_EINVAL, "negative size");
  FP8Q_REQUIRE(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0, FP8Q_ESHAPE, "Hq must be a positive multiple of Hkv");
  const int32_t grp = Hq / Hkv;
  FP8Q_REQUIRE(grp == 1 || grp == 2 || grp == 4 || grp == 8, FP8Q_ESHAPE, "Hq / Hkv must be 1, 2, 4 or 8");
  FP8Q_REQUIRE((int64_t)B * Hkv < ((int64_t)1 << 24), FP8Q_ESHAPE, "B * Hkv must be below 2^24");
  // the scratch array covers every call the split rule allows; checked anyway
  FP8Q_REQUIRE(fp8_attention_decode_workspace_size(B, Hq, Hkv, S) <= fp8q::attention_noalloc_scratch_bytes(),
               FP8Q_ESHAPE, "needs more scratch than FP8Q_NOALLOC_SCRATCH_BYTES");
  if (B == 0) return FP8Q_OK;
  FP8Q_REQUIRE(q_q && q_s && k_cache && k_scale && v_cache && v_scale && seq_len && out, FP8Q_EINVAL,
               "null pointer");
  FP8Q_REQUIRE(aligned16(q_q) && aligned16(q_s) && aligned16(k_cache) && aligned16(k_scale) &&
                   aligned16(v_cache) && aligned16(v_scale) && aligned16(seq_len) && aligned16(out),
               FP8Q_EALIGN, "pointers must be 16-byte aligned");
  fp8q_status st = check_device(__func__);
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_attention_decode_noalloc(q_q, q_s, k_cache, k_scale, v_cache, v_scale, seq_len, out,
                                                        B, Hq, Hkv, S, (hipStream_t)stream),
                  __func__);
}

const char *fp8q_status_string(int status) {
  switch (status) {
    case FP8Q_OK: return "ok";
    case FP8Q_EINVAL: return "invalid argument";
    case FP8Q_ESHAPE: return "unsupported shape";
    case FP8Q_EALIGN: return "misaligned pointer";
    case FP8Q_EDEVICE: return "unsupported or missing device";
    case FP8Q_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *fp8q_last_error(void) { return g_last_error.c_str(); }

int fp8q_abi_version(void) { return FP8Q_ABI_VERSION; }

}  // extern "C"
