// api.hip -- status strings and the codec probe entry points.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_common.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4kv.h"
#include "nvfp4kv_diag.h"

namespace nvfp4 {

__global__ void diag_e2m1_kernel(const float* y, long long n, uint8_t* out) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    out[i] = (uint8_t)(__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[i], 0.0f, 1.0f, 0) & 0xfu);
}

__global__ void diag_candidates_kernel(const float* t, long long n, uint8_t* s6, uint8_t* s4) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    const uint32_t s = candidate_codes(t[i]);
    s6[i] = (uint8_t)(s & 0xffu);
    s4[i] = (uint8_t)(s >> 8);
  }
}

__global__ void diag_recip_kernel(const uint8_t* s, long long n, float* r) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    r[i] = recip_e4m3(__builtin_amdgcn_cvt_f32_fp8((int)s[i], 0));
}

__global__ void diag_bf16_kernel(const float* x, long long n, uint16_t* out) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    out[i] = (uint16_t)(pack_bf16x2(x[i], 0.0f) & 0xffffu);
}

static unsigned diag_grid(long long n) {
  long long b = (n + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" NVFP4KV_API const char* nvfp4_status_string(int status) noexcept {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_NULL: return "NVFP4_ERR_NULL: a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "NVFP4_ERR_SHAPE: invalid sizes (negative, not divisible, or above the limits)";
    case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN: a pointer is not aligned as documented";
    case NVFP4_ERR_ALIAS: return "NVFP4_ERR_ALIAS: an output overlaps an input or another output";
    case NVFP4_ERR_WORKSPACE: return "NVFP4_ERR_WORKSPACE: workspace missing or too small";
    case NVFP4_ERR_MODE: return "NVFP4_ERR_MODE: unknown mode";
    case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP: a HIP kernel launch failed";
    default: return "NVFP4: unknown status";
  }
}

extern "C" NVFP4KV_API int nvfp4_diag_e2m1_encode(const float* y, long long n, uint8_t* codes, void* stream) noexcept {
  if (n < 0) return NVFP4_ERR_SHAPE;
  if (n == 0) return NVFP4_OK;
  if (!y || !codes) return NVFP4_ERR_NULL;
  (void)hipGetLastError();
  diag_e2m1_kernel<<<diag_grid(n), 256, 0, as_stream(stream)>>>(y, n, codes);
  return launch_status();
}

extern "C" NVFP4KV_API int nvfp4_diag_candidates(const float* t, long long n, uint8_t* s6, uint8_t* s4,
                                                 void* stream) noexcept {
  if (n < 0) return NVFP4_ERR_SHAPE;
  if (n == 0) return NVFP4_OK;
  if (!t || !s6 || !s4) return NVFP4_ERR_NULL;
  (void)hipGetLastError();
  diag_candidates_kernel<<<diag_grid(n), 256, 0, as_stream(stream)>>>(t, n, s6, s4);
  return launch_status();
}

extern "C" NVFP4KV_API int nvfp4_diag_reciprocal(const uint8_t* s, long long n, float* r, void* stream) noexcept {
  if (n < 0) return NVFP4_ERR_SHAPE;
  if (n == 0) return NVFP4_OK;
  if (!s || !r) return NVFP4_ERR_NULL;
  (void)hipGetLastError();
  diag_recip_kernel<<<diag_grid(n), 256, 0, as_stream(stream)>>>(s, n, r);
  return launch_status();
}

extern "C" NVFP4KV_API int nvfp4_diag_bf16_round(const float* x, long long n, uint16_t* out, void* stream) noexcept {
  if (n < 0) return NVFP4_ERR_SHAPE;
  if (n == 0) return NVFP4_OK;
  if (!x || !out) return NVFP4_ERR_NULL;
  (void)hipGetLastError();
  diag_bf16_kernel<<<diag_grid(n), 256, 0, as_stream(stream)>>>(x, n, out);
  return launch_status();
}
