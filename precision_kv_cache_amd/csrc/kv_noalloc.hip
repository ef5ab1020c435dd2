// kv_noalloc.hip -- nvfp4_kv_smooth_quantize for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation): the same kernels, with their workspace
// in a fixed device array of this library instead of a caller's buffer.
//
// `scratch` is a file-scope device array, one copy per GPU, held until the
// process ends.  In host code its name is only a host-side stand-in: its
// device address, different on every GPU, is taken once per device with
// hipGetSymbolAddress (with that device current) on the entry point's first
// call there, kept in g_scratch, and only that address is ever passed to a
// kernel.  Every call on a GPU shares that GPU's array: the kernels clear the
// counters and ready words they use at the start of each call, and calls
// that overlap in time on one GPU race.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "host_common.hpp"
#include "nvfp4kv.h"

namespace nvfp4 {

int kv_quantize_check(const uint16_t* k, const uint16_t* v, int H, int T, int D, int chunk_len, int mode,
                      const uint8_t* k_codes, const uint8_t* v_codes, const uint8_t* k_scales,
                      const uint8_t* v_scales, const float* k_tensor_scale, const float* v_tensor_scale,
                      const float* k_mean, const unsigned long long* choice_counts, const void* workspace,
                      size_t ws_range);
int kv_quantize_launch(const uint16_t* k, const uint16_t* v, int H, int T, int D, int chunk_len, int mode,
                       uint8_t* k_codes, uint8_t* v_codes, uint8_t* k_scales, uint8_t* v_scales,
                       float* k_tensor_scale, float* v_tensor_scale, float* k_mean,
                       unsigned long long* choice_counts, void* workspace, size_t workspace_bytes,
                       unsigned* err_word, hipStream_t s);

namespace {

static_assert(NVFP4_KV_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");

static __device__ __align__(256) uint8_t scratch[NVFP4_KV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];  // per device: the device address of `scratch`

// The device address of this device's `scratch` (nullptr on failure).
void* scratch_address(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace
}  // namespace nvfp4

using namespace nvfp4;

extern "C" NVFP4KV_API int nvfp4_kv_smooth_quantize_noalloc(const uint16_t* k, const uint16_t* v, int H, int T,
                                                            int D, int chunk_len, int mode, uint8_t* k_codes,
                                                            uint8_t* v_codes, uint8_t* k_scales,
                                                            uint8_t* v_scales, float* k_tensor_scale,
                                                            float* v_tensor_scale, float* k_mean,
                                                            unsigned long long* choice_counts,
                                                            unsigned* error_word, void* stream) noexcept {
  // the error word is one more output: checked against the inputs and the other outputs
  const int rc = kv_quantize_check(k, v, H, T, D, chunk_len, mode, k_codes, v_codes, k_scales, v_scales,
                                   k_tensor_scale, v_tensor_scale, k_mean, choice_counts, error_word, 4);
  if (rc != NVFP4_OK || H == 0 || T == 0) return rc;
  if (!aligned(error_word, 4)) return NVFP4_ERR_ALIGN;
  const size_t need = nvfp4_kv_workspace_bytes(H, T, D, chunk_len);
  if (need > (size_t)NVFP4_KV_NOALLOC_SCRATCH_BYTES) return NVFP4_ERR_WORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_HIP;
  void* ws = scratch_address(dev);
  if (!ws) return NVFP4_ERR_HIP;
  // a timed-out wait is recorded in the caller's word when given, else only in
  // the scratch's own header word, which nothing reads
  unsigned* err = error_word ? error_word : static_cast<unsigned*>(ws);
  return kv_quantize_launch(k, v, H, T, D, chunk_len, mode, k_codes, v_codes, k_scales, v_scales, k_tensor_scale,
                            v_tensor_scale, k_mean, choice_counts, ws, NVFP4_KV_NOALLOC_SCRATCH_BYTES, err,
                            as_stream(stream));
}
