/*
 * nvfp4kv.h -- C ABI of the MI355X (gfx950) NVFP4 "Four-Over-Six" KV-cache
 * quantizer: per-chunk K smoothing + NVFP4 quantization with the 4/6
 * adaptive block scale, the matching dequantize, and the activation (1D +
 * random Hadamard) and weight (2D tile) quantizers of the same format.
 *
 * Source of the method: the summary page "LongLive-2.0: An NVFP4 Parallel
 * Infrastructure for Long Video Generation" (paper.rainbus.top, paper
 * 2605.18739):
 *   - inference pipeline, step 7: per chunk of F_c = 8 frames
 *     (T_c = F_c * L_f tokens), K is smoothed by subtracting its mean, then K
 *     and V are quantized into an NVFP4 cache with the 4/6 block scale;
 *   - full-stack NVFP4: the 4/6 block scale keeps whichever of two FP8
 *     block-scale candidates (+-6 or +-4) gives the lower MSE;
 *   - training pipeline, step 4: 2D block scales for weights, 1D block scales
 *     for activations, random Hadamard transform against outliers.
 *
 * Format (the page names NVFP4 without defining it; these are the readings):
 *   element  : E2M1, 4 bits, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, sign bit 3
 *   block    : 16 consecutive elements along the last dimension (K/V: the
 *              head channel; activations: the column), or a 16x16 tile (weights)
 *   scale    : one OCP E4M3FN byte per block (bias 7, subnormals, max 448)
 *   tensor   : one fp32 decode scale g_dec per (chunk, tensor) (KV) or per
 *              tensor (1D / 2D); the encoder uses g_enc = C / A, g_dec = A / C
 *              with A the largest |value| after smoothing / rotation and
 *              C = 1792 (4/6 and fixed-4) or 2688 (fixed-6)
 *   codes    : byte j of a block = element 2j (low nibble) | element 2j+1 << 4
 *   dequant  : x = bf16( ((v * S) * g_dec) [+ mean] ), each step one fp32
 *              rounding, bf16 by round to nearest even
 *
 * Conventions shared by every entry point:
 *   - All array pointers are DEVICE pointers unless noted; bf16 travels as
 *     uint16_t bit patterns; every array is dense row-major as documented.
 *   - The caller allocates and owns every buffer, including the workspace.
 *     The library never allocates, frees or synchronizes, and keeps no
 *     mutable global state.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     stream-ordered and asynchronous: a return of NVFP4_OK means the work
 *     was enqueued.
 *   - Argument errors return a negative status before any HIP call and with
 *     no side effects.  A launch failure returns NVFP4_ERR_HIP.  Nothing
 *     throws across the ABI.
 *   - Inputs are read-only and must be finite, with |x| < 2^127 after
 *     smoothing, and the largest magnitude A of each scale group must be 0 or
 *     at least 2^-117 (so that C / A is finite).  Other input gives
 *     unspecified values but never an invalid access.
 *   - Outputs must not overlap inputs or each other (NVFP4_ERR_ALIAS).
 *   - H == 0 or T == 0 (rows == 0) is a valid empty call: NVFP4_OK, no work.
 */
#ifndef NVFP4KV_H
#define NVFP4KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4KV_API __attribute__((visibility("default")))
#ifdef __cplusplus
#define NVFP4KV_NOEXCEPT noexcept
#else
#define NVFP4KV_NOEXCEPT
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = -1,      /* a required pointer is NULL                       */
  NVFP4_ERR_SHAPE = -2,     /* negative size, T % chunk_len, D % 16, limits      */
  NVFP4_ERR_ALIGN = -3,     /* a pointer is not aligned as documented            */
  NVFP4_ERR_ALIAS = -4,     /* an output overlaps an input or another output     */
  NVFP4_ERR_WORKSPACE = -5, /* workspace NULL or smaller than required           */
  NVFP4_ERR_MODE = -6,      /* unknown mode                                      */
  NVFP4_ERR_HIP = -7        /* a HIP launch failed                               */
} nvfp4_status;

typedef enum {
  NVFP4_MODE_4OVER6 = 0, /* best of the +-6 and +-4 candidates (ties -> +-6) */
  NVFP4_MODE_FIXED6 = 1, /* textbook NVFP4: +-6 only, C = 2688               */
  NVFP4_MODE_FIXED4 = 2  /* +-4 only, C = 1792                               */
} nvfp4_mode;

/* Kernels of nvfp4_kv_smooth_quantize.  By default, for D == 128, one
 * launch whose grid interleaves the statistics tiles of each (chunk, tensor)
 * unit with the quantize tiles of an earlier unit; the quantize tiles re-read
 * their rows from the Infinity Cache, so K and V are read from HBM about
 * once.  Other shapes, or the option bit below, take the two-pass kernels (a
 * statistics pass, then a quantize pass that reads K and V again).  Both give
 * the same results. */
#define NVFP4_KV_TWO_PASS 0x100

/* Largest supported head dimension / row length for the KV entry points. */
#define NVFP4_KV_MAX_D 4096

/* Human-readable name of a status code (static storage, never NULL). */
NVFP4KV_API const char* nvfp4_status_string(int status) NVFP4KV_NOEXCEPT;

/* Workspace bytes nvfp4_kv_smooth_quantize needs for this shape (0 for an
 * invalid shape).  Host function, no HIP call. */
NVFP4KV_API size_t nvfp4_kv_workspace_bytes(int H, int T, int D, int chunk_len) NVFP4KV_NOEXCEPT;

/* Byte offset, inside the workspace of nvfp4_kv_smooth_quantize, of the
 * 32-bit error word of the default (overlapped) kernel for this shape, or -1
 * when the shape takes the two-pass kernels (which never wait).  Each call
 * clears the word; once the call has completed (the stream synchronized), a
 * non-zero value there means one of the kernel's bounded waits timed out and
 * the call's outputs are invalid.  Host function, no HIP call. */
NVFP4KV_API long long nvfp4_kv_error_word_offset(int H, int T, int D, int chunk_len) NVFP4KV_NOEXCEPT;

/*
 * K smoothing + 4/6 NVFP4 quantization of one layer's K and V
 * (inference pipeline, step 7; full-stack NVFP4).
 *
 *   k, v          bf16 [H, T, D]; T = n_chunks * chunk_len; 16-byte aligned.
 *   H, T, D       heads, tokens, head dimension (D % 16 == 0, D <= 4096).
 *   chunk_len     T_c, tokens per chunk; each chunk gets its own K mean and
 *                 its own tensor scales.
 *   mode          nvfp4_mode, optionally | NVFP4_KV_TWO_PASS.
 *   k_codes, v_codes     out, uint8 [H, T, D/2], 8-byte aligned.
 *   k_scales, v_scales   out, E4M3FN bytes [H, T, D/16].
 *   k_tensor_scale, v_tensor_scale  out, fp32 [n_chunks], g_dec per chunk.
 *   k_mean        out, fp32 [n_chunks, H, D]: the per-chunk channel mean of K
 *                 (sum over the chunk's tokens, rounded once to fp32), 16-byte
 *                 aligned.  Pass it to nvfp4_dequantize to restore K.
 *   choice_counts out, nullable, uint64 [2][2]: {K, V} x {blocks that kept +-6,
 *                 blocks that kept +-4}; overwritten by this call.
 *   workspace     device scratch of at least nvfp4_kv_workspace_bytes(),
 *                 256-byte aligned; contents on entry are ignored.  Calls
 *                 that share a workspace must be ordered on one stream.
 *
 * The overlapped kernel's quantize tiles wait, through words in the
 * workspace, for statistics tiles that precede them in the grid; each wait
 * is bounded, and if one ever timed out the tile would stop early and leave
 * its results invalid (the workspace's error word is then non-zero).
 *
 * Smoothing: k' = fl(K - mean) in fp32.  V is quantized as is.
 */
NVFP4KV_API int nvfp4_kv_smooth_quantize(const uint16_t* k, const uint16_t* v, int H, int T, int D, int chunk_len,
                                         int mode, uint8_t* k_codes, uint8_t* v_codes, uint8_t* k_scales,
                                         uint8_t* v_scales, float* k_tensor_scale, float* v_tensor_scale,
                                         float* k_mean, unsigned long long* choice_counts, void* workspace,
                                         size_t workspace_bytes, void* stream) NVFP4KV_NOEXCEPT;

/*
 * Dequantize an NVFP4 cache tensor back to bf16 (the consumer side of
 * inference pipeline, step 7).
 *
 *   codes         uint8 [H, T, D/2] (8-byte aligned), scales E4M3FN [H, T, D/16].
 *   tensor_scale  fp32 [T / chunk_len]: g_dec per chunk.
 *   mean          nullable fp32 [T / chunk_len, H, D] (16-byte aligned): added
 *                 back after scaling (pass k_mean to restore K; NULL for V).
 *   out           bf16 [H, T, D], 16-byte aligned.
 * A 1D activation tensor [rows, cols] is dequantized with H = 1, T = rows,
 * D = cols, chunk_len = rows, mean = NULL (the rotation is not undone).
 */
NVFP4KV_API int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                 const float* mean, int H, int T, int D, int chunk_len, uint16_t* out, void* stream) NVFP4KV_NOEXCEPT;

/* Workspace bytes of nvfp4_quantize_1d / nvfp4_quantize_2d (under 9 KB: the
 * tensor maximum and per-workgroup partial maxima). */
NVFP4KV_API size_t nvfp4_quantize_1d_workspace_bytes(int rows, int cols) NVFP4KV_NOEXCEPT;
NVFP4KV_API size_t nvfp4_quantize_2d_workspace_bytes(int rows, int cols) NVFP4KV_NOEXCEPT;

/*
 * Activation quantizer (training pipeline, step 4): 1D 16-element blocks
 * along each row of x [rows, cols] (cols % 16 == 0), one tensor scale, 4/6
 * block scales.  With hadamard != 0 every block is first rotated by the
 * 16-point random-sign Hadamard transform u = s * x, Sylvester H_16 in
 * natural order, times 1/4, where bit j of sign_mask set means s_j = -1.
 *
 *   x             bf16 [rows, cols], 16-byte aligned.
 *   codes         out, uint8 [rows, cols/2] (8-byte aligned); scales out [rows, cols/16].
 *   tensor_scale  out, fp32 [1], g_dec.
 *   workspace     >= nvfp4_quantize_1d_workspace_bytes(), 256-byte aligned.
 */
NVFP4KV_API int nvfp4_quantize_1d(const uint16_t* x, int rows, int cols, int mode, int hadamard,
                                  uint32_t sign_mask, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                  void* workspace, size_t workspace_bytes, void* stream) NVFP4KV_NOEXCEPT;

/*
 * Weight quantizer (training pipeline, step 4): 2D 16x16 tiles of
 * w [rows, cols] (rows % 16 == 0, cols % 16 == 0), one E4M3 scale and one 4/6
 * choice per tile (the tile error adds the 16 tile rows' errors as a
 * pairwise tree), one tensor scale.
 *
 *   w             bf16 [rows, cols], 16-byte aligned.
 *   codes         out, uint8 [rows, cols/2] (8-byte aligned); scales out [rows/16, cols/16].
 *   tensor_scale  out, fp32 [1].
 */
NVFP4KV_API int nvfp4_quantize_2d(const uint16_t* w, int rows, int cols, int mode, uint8_t* codes,
                                  uint8_t* scales, float* tensor_scale, void* workspace, size_t workspace_bytes,
                                  void* stream) NVFP4KV_NOEXCEPT;

/* Dequantize a 2D-tile tensor: out bf16 [rows, cols] (16-byte aligned). */
NVFP4KV_API int nvfp4_dequantize_2d(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                    int rows, int cols, uint16_t* out, void* stream) NVFP4KV_NOEXCEPT;

/* Largest number of key ranges one attention call takes. */
#define NVFP4_ATTN_MAX_RANGES 8

/*
 * Softmax attention of bf16 queries over key ranges of one layer's NVFP4 KV
 * cache, decoding the cache on load.  The cache is the one built in inference
 * pipeline step 7 (smoothed K and V per chunk); the ranges express step 9's
 * key set: a global sink (the first S_g frames), a shot sink (the first S_s
 * frames of the current shot, START / LEN only) and the recent window.  The
 * page gives no attention formula; the reading is ordinary softmax attention
 * over the values the cache represents:
 *   K[j] = v * S * g_K[c] + k_mean[c],  V[j] = v * S * g_V[c],  c = j / chunk_len,
 *   out = sum_j softmax_j(softmax_scale * q . K[j]) V[j],
 *   lse = ln sum_j exp(softmax_scale * q . K[j]).
 *
 *   q             bf16 [H, Tq, D], 16-byte aligned.
 *   H, Tq, D      query heads, queries per head, head dimension (D == 128).
 *   k_*, v_*      the cache as nvfp4_kv_smooth_quantize writes it for
 *                 H_kv heads and T tokens: codes uint8 [H_kv, T, D/2]
 *                 (k_codes 8-byte aligned, v_codes 2-byte aligned), scales
 *                 E4M3FN [H_kv, T, D/16], tensor scales fp32 [T / chunk_len].
 *   k_mean        nullable fp32 [T / chunk_len, H_kv, D] (16-byte aligned);
 *                 NULL means K was stored without smoothing.
 *   H_kv          cache heads; query head h reads cache head h / (H / H_kv).
 *   key_ranges    HOST int [n_ranges][2] = (start, len) in tokens, each inside
 *                 [0, T); the key set is their concatenation (a key listed
 *                 twice counts twice).  n_ranges <= NVFP4_ATTN_MAX_RANGES.
 *   softmax_scale finite and > 0; 1/sqrt(D) is the usual value.
 *   out           out, bf16 [H, Tq, D], 8-byte aligned.  With no keys: 0.
 *   lse           out, nullable fp32 [H, Tq] (natural log); -inf with no keys.
 *
 * Arithmetic: K is decoded to v * S, exact in bf16, so the logits are exact
 * up to fp32 accumulation (g_K, the softmax scale and the mean term
 * q . k_mean[c] are applied in fp32 per chunk); V is decoded to
 * bf16(v * S * g_V); P V accumulates in fp32 on the matrix cores with P
 * rounded to bf16, and out is rounded to bf16.
 */
NVFP4KV_API int nvfp4_kv_attention(const uint16_t* q, int H, int Tq, int D, const uint8_t* k_codes,
                                   const uint8_t* k_scales, const float* k_tensor_scale, const float* k_mean,
                                   const uint8_t* v_codes, const uint8_t* v_scales, const float* v_tensor_scale,
                                   int H_kv, int T, int chunk_len, const int* key_ranges, int n_ranges,
                                   float softmax_scale, uint16_t* out, float* lse,
                                   void* stream) NVFP4KV_NOEXCEPT;

#ifdef __cplusplus
}
#endif

#endif /* NVFP4KV_H */
