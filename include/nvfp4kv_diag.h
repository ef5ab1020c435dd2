/*
 * nvfp4kv_diag.h -- device-side probes of the quantizer's number-format
 * steps, for exhaustive conversion tests.  Each entry point runs, over an
 * array, exactly the device routine the quantize / dequantize kernels use
 * for that step, so the tests can sweep every fp32 input of a range against
 * the CPU reference.  Same conventions as nvfp4kv.h: device pointers,
 * caller-owned buffers, asynchronous on `stream`, negative status on bad
 * arguments before any HIP call.
 */
#ifndef NVFP4KV_DIAG_H
#define NVFP4KV_DIAG_H

#include <stddef.h>
#include <stdint.h>

#include "nvfp4kv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* codes[i] = E2M1 code of y[i] (sign in bit 3), as the block encoder forms
 * it: round to nearest even on the code, saturation at 6. */
NVFP4KV_API int nvfp4_diag_e2m1_encode(const float* y, long long n, uint8_t* codes, void* stream) NVFP4KV_NOEXCEPT;

/* For a block maximum t[i] >= 0: s6[i] = E4M3(fl(t/6)), s4[i] = E4M3(fl(t/4)),
 * the two candidate scale bytes of the 4/6 rule. */
NVFP4KV_API int nvfp4_diag_candidates(const float* t, long long n, uint8_t* s6, uint8_t* s4, void* stream) NVFP4KV_NOEXCEPT;

/* r[i] = fl(1 / S) for S = E4M3 value of byte s[i] (0 when S = 0), the
 * element-encode reciprocal. */
NVFP4KV_API int nvfp4_diag_reciprocal(const uint8_t* s, long long n, float* r, void* stream) NVFP4KV_NOEXCEPT;

/* out[i] = bf16 round-to-nearest-even of x[i], as the dequantizer packs it. */
NVFP4KV_API int nvfp4_diag_bf16_round(const float* x, long long n, uint16_t* out, void* stream) NVFP4KV_NOEXCEPT;

#ifdef __cplusplus
}
#endif

#endif /* NVFP4KV_DIAG_H */
