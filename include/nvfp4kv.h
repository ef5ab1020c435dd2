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
 *     was enqueued.  They enqueue kernels only (workspace counters are
 *     cleared by a kernel, never a memset), so they may be captured into a
 *     HIP graph and replayed; a replay reuses the captured workspace, so
 *     replays and other calls on that workspace must not overlap in time.
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

/* Byte offset, inside the workspace of nvfp4_kv_smooth_quantize, of its
 * sticky 32-bit error word: 0 (the first word) for every valid shape, -1 for
 * an invalid one.  The word belongs to the caller: the library never clears
 * it.  A call whose overlapped kernel had one of its bounded waits time out
 * sets it to non-zero, and that call's outputs are invalid; so a zero word,
 * read once the stream has synchronized, vouches for every call on the
 * workspace since the caller last zeroed it.  The two-pass kernels never wait
 * and never set it.  Host function, no HIP call. */
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
 *                 over the chunk's tokens, 16-byte aligned.  The overlapped
 *                 kernel adds the tokens in fp32 runs of 8 and the runs in
 *                 fp64, so the mean is within 8 * 2^-24 * max(|m|, mean |K|)
 *                 of the exact one (the two-pass kernels add every token in
 *                 fp64).  Pass it to nvfp4_dequantize to restore K.
 *   choice_counts out, nullable, uint64 [2][2]: {K, V} x {blocks that kept +-6,
 *                 blocks that kept +-4}; overwritten by this call.
 *   workspace     device scratch of at least nvfp4_kv_workspace_bytes(),
 *                 256-byte aligned.  Its first 256 bytes are a header whose
 *                 first word is the sticky error word (zero it before the
 *                 first call); the rest of the contents on entry are
 *                 ignored.  Calls that share a workspace must be ordered on
 *                 one stream.
 *
 * The overlapped kernel's quantize tiles wait, through words in the
 * workspace, for statistics tiles that precede them in the grid; each wait
 * is bounded, and if one ever timed out the tile would stop early, leave its
 * results invalid and set the sticky error word.
 *
 * Smoothing: k' = fl(K - mean) in fp32.  V is quantized as is.
 */
NVFP4KV_API int nvfp4_kv_smooth_quantize(const uint16_t* k, const uint16_t* v, int H, int T, int D, int chunk_len,
                                         int mode, uint8_t* k_codes, uint8_t* v_codes, uint8_t* k_scales,
                                         uint8_t* v_scales, float* k_tensor_scale, float* v_tensor_scale,
                                         float* k_mean, unsigned long long* choice_counts, void* workspace,
                                         size_t workspace_bytes, void* stream) NVFP4KV_NOEXCEPT;

/* Bytes of the device array nvfp4_kv_smooth_quantize_noalloc uses instead of
 * a workspace (one per GPU): enough for one layer of 24 heads x 56320 tokens
 * x 128 channels in chunks of 7040 tokens. */
#define NVFP4_KV_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * nvfp4_kv_smooth_quantize without a workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, results and kernels as
 * nvfp4_kv_smooth_quantize, except:
 *   - no workspace: the kernels use a device array of this library, one per
 *     GPU, of NVFP4_KV_NOALLOC_SCRATCH_BYTES bytes, held until the process
 *     ends.  The call allocates and frees nothing.  A shape whose
 *     nvfp4_kv_workspace_bytes() exceeds that size returns
 *     NVFP4_ERR_WORKSPACE before any HIP call.
 *   - every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (on different streams, or from several threads) race
 *     and give invalid results.  Order them on one stream.  The array keeps
 *     the last call's contents; each call clears the counters it needs.
 *   - error_word: nullable device pointer to a caller-owned uint32 (4-byte
 *     aligned, no overlap with the other arguments).  A call whose bounded
 *     waits timed out ORs 1 into it (the library never clears it), and that
 *     call's outputs are invalid.
 *   - the first call on a GPU looks up the array's device address there
 *     (hipGetSymbolAddress, with that GPU current) and keeps it; a failure
 *     returns NVFP4_ERR_HIP.  `stream` must belong to the current device.
 */
NVFP4KV_API int nvfp4_kv_smooth_quantize_noalloc(const uint16_t* k, const uint16_t* v, int H, int T, int D,
                                                 int chunk_len, int mode, uint8_t* k_codes, uint8_t* v_codes,
                                                 uint8_t* k_scales, uint8_t* v_scales, float* k_tensor_scale,
                                                 float* v_tensor_scale, float* k_mean,
                                                 unsigned long long* choice_counts, unsigned* error_word,
                                                 void* stream) NVFP4KV_NOEXCEPT;

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

/*
 * Dequantize a weight quantized with 2D tiles (the inverse of
 * nvfp4_quantize_2d; LongLive-2.0 summary page, training pipeline, step 4,
 * and its full-stack NVFP4 section: weights carry one block scale per 16x16
 * tile).  Every element of tile (r / 16, c / 16) decodes as
 * bf16((v * S_tile) * g_dec), each step one fp32 rounding.
 *
 *   codes         uint8 [rows, cols/2] (8-byte aligned), low nibble = even column.
 *   scales        E4M3FN bytes [rows/16, cols/16].
 *   tensor_scale  fp32 [1], g_dec.
 *   out           bf16 [rows, cols], 16-byte aligned; must not overlap an input.
 * rows % 16 == 0 and cols % 16 == 0, else NVFP4_ERR_SHAPE.
 */
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
 *   workspace     nullable, 256-byte aligned, workspace_bytes long: room to
 *                 split each query block's key list over up to four
 *                 workgroups (the split fills the GPU's CUs more evenly; a
 *                 small kernel then merges the partial results per query
 *                 row).  nvfp4_kv_attention_workspace_bytes() is enough for
 *                 every split; NULL or less than two splits' worth runs
 *                 unsplit.  A workspace of at least
 *                 nvfp4_kv_attention_staged_workspace_bytes() for the same
 *                 key list also holds the decoded image of every 64-key tile
 *                 (35 KB per tile and cache head): the call then decodes each
 *                 tile once, in a staging kernel, instead of once per query
 *                 block, with bit-identical results.  Contents on entry
 *                 ignored.
 *
 * Arithmetic: K is decoded to v * S, exact in bf16, so the logits are exact
 * up to fp32 accumulation (g_K, the softmax scale and the mean term
 * q . k_mean[c] are applied in fp32 per chunk); V is decoded to
 * bf16(v * S * g_V); P V accumulates in fp32 on the matrix cores with P
 * rounded to bf16, and out is rounded to bf16.  With key splits each split
 * keeps its fp32 sums and reference maximum; the merge rescales them in fp32
 * and rounds out to bf16 once.
 */
NVFP4KV_API size_t nvfp4_kv_attention_workspace_bytes(int H, int Tq, int D) NVFP4KV_NOEXCEPT;
/*
 * Workspace bytes for every key split plus the decoded tile images of the
 * key list (key_ranges, n_ranges over a cache of H_kv heads, T tokens and
 * chunk_len-token chunks; the same arguments nvfp4_kv_attention and
 * nvfp4_kv_attention_chunked take).  0 for arguments those calls reject; for
 * a key list of more than 65536 chunk pieces, which runs unstaged, just the
 * split bytes.
 */
NVFP4KV_API size_t nvfp4_kv_attention_staged_workspace_bytes(int H, int Tq, int D, int H_kv, int T, int chunk_len,
                                                             const int* key_ranges, int n_ranges) NVFP4KV_NOEXCEPT;
NVFP4KV_API int nvfp4_kv_attention(const uint16_t* q, int H, int Tq, int D, const uint8_t* k_codes,
                                   const uint8_t* k_scales, const float* k_tensor_scale, const float* k_mean,
                                   const uint8_t* v_codes, const uint8_t* v_scales, const float* v_tensor_scale,
                                   int H_kv, int T, int chunk_len, const int* key_ranges, int n_ranges,
                                   float softmax_scale, uint16_t* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream) NVFP4KV_NOEXCEPT;

/*
 * The same attention over a chunk-major cache: codes uint8 [T / chunk_len,
 * H_kv, chunk_len, D/2], scales [T / chunk_len, H_kv, chunk_len, D/16]; that
 * is, chunk c is the [H_kv, chunk_len, ...] output of one
 * nvfp4_kv_smooth_quantize call on that chunk, and chunks follow one another
 * (the slot layout of the streaming cache below).  Key j still means token
 * j % chunk_len of chunk j / chunk_len; tensor scales and k_mean are indexed
 * by chunk as above.  Every other argument and rule is that of
 * nvfp4_kv_attention.
 */
NVFP4KV_API int nvfp4_kv_attention_chunked(const uint16_t* q, int H, int Tq, int D, const uint8_t* k_codes,
                                           const uint8_t* k_scales, const float* k_tensor_scale,
                                           const float* k_mean, const uint8_t* v_codes, const uint8_t* v_scales,
                                           const float* v_tensor_scale, int H_kv, int T, int chunk_len,
                                           const int* key_ranges, int n_ranges, float softmax_scale,
                                           uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                                           void* stream) NVFP4KV_NOEXCEPT;

/*
 * W4A4 GEMM on NVFP4 operands (training pipeline, step 4: weights with 2D
 * block scales, activations with 1D block scales; inference pipeline, step
 * 6: the W4A4 model).  The page gives no formula; the reading is the product
 * of the two dequantized operands along their shared K axis:
 *   out[m][n] = bf16( g_A g_W sum_k (v S)_A[m][k] (v S)_W[n][k] ),
 * v the E2M1 values, S the E4M3 block scales, g the tensor scales.  A
 * rotation applied before quantization (the random Hadamard transform) is
 * not undone: rotate both operands along K with the same signs to get the
 * unrotated product.
 *
 *   a_codes, a_scales  the activation as nvfp4_quantize_1d writes it: codes
 *                      uint8 [M, K/2] (16-byte aligned), scales E4M3FN [M, K/16]
 *                      (2-byte aligned); a_tensor_scale fp32 [1].
 *   w_codes, w_scales  the weight [N, K]: codes uint8 [N, K/2] (16-byte
 *                      aligned); scales [N/16, K/16] when w_2d != 0 (the 2D
 *                      tiles of nvfp4_quantize_2d) or [N, K/16] (1D blocks of
 *                      nvfp4_quantize_1d); w_tensor_scale fp32 [1].
 *   K % 64 == 0 and K >= 64; N % 16 == 0; M >= 0.
 *   out                bf16 [M, N], 8-byte aligned.
 * Arithmetic: each operand element decodes exactly to fp16 (v * S has at
 * most 6 significant bits and lies in [2^-10, 2688]), the products
 * accumulate in fp32 on the matrix cores, g_A g_W multiplies the sum once,
 * and the result rounds to bf16.
 */
NVFP4KV_API int nvfp4_gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
                                int M, int K, const uint8_t* w_codes, const uint8_t* w_scales,
                                const float* w_tensor_scale, int N, int w_2d, uint16_t* out,
                                void* stream) NVFP4KV_NOEXCEPT;

/*
 * V with its 16-element blocks along the token axis: block = 16 consecutive
 * tokens of one (head, channel), so that a P V product can contract over
 * blocks (the V-blocking variant of inference pipeline, step 7; same 4/6
 * block scale and one tensor scale per (chunk, V) as nvfp4_kv_smooth_quantize).
 *
 *   v             bf16 [H, T, D], 16-byte aligned; D % 64 == 0, D <= 4096.
 *   chunk_len     % 16 == 0; T % chunk_len == 0 (blocks never cross a chunk).
 *   mode          nvfp4_mode.
 *   codes         out, uint8 [H, D, T/2] (8-byte aligned): byte j of a row =
 *                 token 2j (low nibble) | token 2j+1 << 4.
 *   scales        out, E4M3FN [H, D, T/16].
 *   tensor_scale  out, fp32 [T / chunk_len], g_dec per chunk.
 *   workspace     >= nvfp4_kv_quantize_v_tblocks_workspace_bytes(), 256-byte
 *                 aligned.  Its first 32-bit word is a sticky error word that
 *                 the library never clears (zero it before the first call):
 *                 a call whose bounded waits timed out sets it, and that
 *                 call's outputs are invalid.  The rest of the contents on
 *                 entry are ignored.
 * Every block is encoded exactly as the blocks of nvfp4_kv_smooth_quantize's
 * V: z = fl(v * g_enc) with g_enc = fl(C / A), A the chunk's largest |V|, the
 * 4/6 choice on fp32 errors, E2M1 round to nearest even.
 */
NVFP4KV_API size_t nvfp4_kv_quantize_v_tblocks_workspace_bytes(int H, int T, int D,
                                                               int chunk_len) NVFP4KV_NOEXCEPT;
NVFP4KV_API int nvfp4_kv_quantize_v_tblocks(const uint16_t* v, int H, int T, int D, int chunk_len, int mode,
                                            uint8_t* codes, uint8_t* scales, float* tensor_scale, void* workspace,
                                            size_t workspace_bytes, void* stream) NVFP4KV_NOEXCEPT;

/*
 * 3-bit / 2-bit KV cache (directions to extend, item 6: compress the KV
 * cache further to 3 or 2 bits; the smoothing and the cache as inference
 * pipeline, step 7; the two-candidate block scale as full-stack NVFP4).  The
 * page defines no format; the one here keeps the NVFP4 layout:
 *   element  sign bit + magnitude: 3 bits {0, 0.5, 1, 1.5} (E1M1), 2 bits
 *            {0, 1} (E1M0); nearest magnitude, ties to the even code,
 *            saturating, sign bit = the sign bit of y (so -0 is possible);
 *   block    16 consecutive channels, one E4M3FN scale; one fp32 g_dec per
 *            (chunk, tensor); the K mean and smoothing of the 4-bit path;
 *   choice   (mode NVFP4_MODE_4OVER6) of the candidates t_b / c_a and
 *            t_b / c_b the one with the lower fp32 error, ties keep c_a:
 *            3 bits: c_a = 1.5, c_b = 1; 2 bits: c_a = 1, c_b = 1.5 (c_a maps
 *            the block maximum onto the largest magnitude).
 *            NVFP4_MODE_FIXED6 keeps c_a only, NVFP4_MODE_FIXED4 c_b only;
 *   C        the encode scale maps the largest |value| to 448 * the smallest
 *            divisor the mode uses;
 *   codes    [H, T, D * bits / 8]: element i of a block at bits
 *            [bits * i, bits * i + bits) of its 2 * bits bytes, least
 *            significant bit first; blocks in channel order.
 *
 *   k, v, H, T, D, chunk_len, k_mean, tensor scales, scales: as
 *                 nvfp4_kv_smooth_quantize.
 *   bits          3 or 2 (else NVFP4_ERR_SHAPE).
 *   k_codes, v_codes  out, [H, T, D * bits / 8], 2-byte (3 bits) or 4-byte
 *                 (2 bits) aligned.
 *   choice_counts out, nullable, uint64 [2][2]: {K, V} x {kept c_a, kept c_b}.
 *   mode          as above, optionally | NVFP4_KV_TWO_PASS: for D = 128 the
 *                 call runs the overlapped kernel of nvfp4_kv_smooth_quantize
 *                 (statistics and quantize tiles in one launch), otherwise, or
 *                 with the bit, the two-pass kernels.  Both write the same
 *                 bytes given the same mean.
 *   workspace     >= nvfp4_kv_workspace_bytes(), 256-byte aligned; its first
 *                 word is the sticky error word, as for
 *                 nvfp4_kv_smooth_quantize (zero it before the first call),
 *                 and the rest of its contents on entry are ignored.
 */
NVFP4KV_API int nvfp4_kv_smooth_quantize_lowbit(const uint16_t* k, const uint16_t* v, int H, int T, int D,
                                                int chunk_len, int bits, int mode, uint8_t* k_codes,
                                                uint8_t* v_codes, uint8_t* k_scales, uint8_t* v_scales,
                                                float* k_tensor_scale, float* v_tensor_scale, float* k_mean,
                                                unsigned long long* choice_counts, void* workspace,
                                                size_t workspace_bytes, void* stream) NVFP4KV_NOEXCEPT;

/* Dequantize a 3-bit / 2-bit cache tensor: x = bf16( ((v * S) * g_dec)
 * [+ mean] ), each step one fp32 rounding.  codes [H, T, D * bits / 8]
 * (aligned as above), scales [H, T, D / 16], tensor_scale [T / chunk_len],
 * mean nullable [T / chunk_len, H, D] (16-byte aligned), out bf16 [H, T, D]
 * (16-byte aligned). */
NVFP4KV_API int nvfp4_dequantize_lowbit(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                        const float* mean, int H, int T, int D, int chunk_len, int bits,
                                        uint16_t* out, void* stream) NVFP4KV_NOEXCEPT;

/* ---------------------------------------------------------------------------
 * Streaming NVFP4 KV cache (inference pipeline, steps 7 to 9 of the summary
 * page): chunks arrive one at a time and each is quantized (K smoothed, 4/6
 * block scales) straight into a slot of caller-allocated device storage;
 * attention then reads
 *   - the global sink: the first S_g frames of the video (chunk 0),
 *   - the shot sink: the first S_s frames of the current shot, a START / LEN
 *     view into the cache (no copy) that is rebound when the prompt
 *     switches (nvfp4_kv_cache_begin_chunk with new_shot = 1),
 *   - the window: the last W committed chunks.
 * A sink that lies inside the window is not listed again; sinks in chunk 0
 * are merged (the longer of the two).  The page gives the sink structure and
 * no slot or eviction policy; the one here: the new chunk takes an empty
 * slot, else the slot of the oldest chunk that the current key set does not
 * read.  So the append of chunk c never writes memory that an attention call
 * on the committed state (the chunks before c) reads, and may run on another
 * stream at the same time as those calls.  Attention calls issued before the
 * previous nvfp4_kv_cache_end_chunk must be complete, or ordered before the
 * append, since the slot it takes may have been read by them.
 *
 * The state is this plain struct, owned by the caller (host memory); every
 * cache call below is a host function, and only _append and _attention
 * enqueue device work (on `stream`).  Storage: `layers` consecutive layer
 * blocks of nvfp4_kv_cache_layer_bytes() each (256-byte aligned), each block
 * holding, at the byte offsets nvfp4_kv_cache_offsets() reports:
 *   k_codes, v_codes    uint8 [capacity, heads, chunk_len, head_dim / 2]
 *   k_scales, v_scales  E4M3FN [capacity, heads, chunk_len, head_dim / 16]
 *   k_tensor_scale, v_tensor_scale  fp32 [capacity]
 *   k_mean              fp32 [capacity, heads, head_dim]
 * Slot s holds one chunk exactly as nvfp4_kv_smooth_quantize writes it, and
 * the key set is given in slot coordinates: key j is token j % chunk_len of
 * slot j / chunk_len (the chunk-major layout of nvfp4_kv_attention_chunked).
 */
#define NVFP4_CACHE_MAX_SLOTS 64

typedef struct {
  /* geometry, set by nvfp4_kv_cache_init */
  int layers, heads, head_dim, chunk_len, capacity;
  int frame_tokens, sink_frames, shot_frames, window;
  /* state */
  long long chunks;       /* chunks committed so far */
  long long shot_chunk;   /* first chunk of the current shot */
  long long pending;      /* chunk between begin and end, -1 when none */
  int pending_slot;       /* its slot */
  int pending_new_shot;   /* it starts a new shot */
  long long slot_chunk[NVFP4_CACHE_MAX_SLOTS]; /* chunk held by each slot, -1 = empty */
} nvfp4_kv_cache_t;

/* Bytes of one layer block of the storage; 0 for an invalid geometry. */
NVFP4KV_API size_t nvfp4_kv_cache_layer_bytes(int heads, int head_dim, int chunk_len, int capacity) NVFP4KV_NOEXCEPT;

/* Byte offsets, inside a layer block, of k_codes, v_codes, k_scales,
 * v_scales, k_tensor_scale, v_tensor_scale, k_mean (in that order) into
 * off[7].  Host function. */
NVFP4KV_API int nvfp4_kv_cache_offsets(const nvfp4_kv_cache_t* c, size_t* off) NVFP4KV_NOEXCEPT;

/* Sets up an empty cache.  frame_tokens = L_f; sink_frames = S_g and
 * shot_frames = S_s (each at most one chunk: frames * frame_tokens <=
 * chunk_len; 0 disables that sink); window = W in 1 .. NVFP4_ATTN_MAX_RANGES
 * - 2; capacity (slots per layer) in W + 3 .. NVFP4_CACHE_MAX_SLOTS.  The
 * first chunk starts the first shot.  head_dim % 16 == 0, <= 4096 (the
 * attention call needs 128).  Host function; the storage is not touched. */
NVFP4KV_API int nvfp4_kv_cache_init(nvfp4_kv_cache_t* c, int layers, int heads, int head_dim, int chunk_len,
                                    int capacity, int frame_tokens, int sink_frames, int shot_frames,
                                    int window) NVFP4KV_NOEXCEPT;

/* Starts chunk `chunks` (the next one): picks its slot (returned, >= 0), and
 * with new_shot != 0 makes it the first chunk of a new shot once committed.
 * NVFP4_ERR_SHAPE if a chunk is already pending.  Host function. */
NVFP4KV_API int nvfp4_kv_cache_begin_chunk(nvfp4_kv_cache_t* c, int new_shot) NVFP4KV_NOEXCEPT;

/* Quantizes one layer of the pending chunk into its slot:
 * nvfp4_kv_smooth_quantize(k, v, heads, chunk_len, head_dim, chunk_len,
 * mode, ...) with the slot's arrays as outputs.  k, v bf16 [heads,
 * chunk_len, head_dim]; storage (device, 256-byte aligned) of at least
 * layers * nvfp4_kv_cache_layer_bytes() bytes; workspace as for that call
 * (nvfp4_kv_workspace_bytes(heads, chunk_len, head_dim, chunk_len)).  Calls
 * for different layers may run on different streams. */
NVFP4KV_API int nvfp4_kv_cache_append(const nvfp4_kv_cache_t* c, void* storage, size_t storage_bytes, int layer,
                                      const uint16_t* k, const uint16_t* v, int mode, void* workspace,
                                      size_t workspace_bytes, void* stream) NVFP4KV_NOEXCEPT;

/* Commits the pending chunk (all its layers appended): it joins the window,
 * and becomes the shot sink's chunk if it started a new shot.  Host. */
NVFP4KV_API int nvfp4_kv_cache_end_chunk(nvfp4_kv_cache_t* c) NVFP4KV_NOEXCEPT;

/* The committed key set as (start, len) ranges in slot coordinates, into
 * ranges[NVFP4_ATTN_MAX_RANGES][2] (host); returns the count (>= 0), or a
 * negative status.  Order: global sink, shot sink, window chunks oldest first
 * (adjacent slots merged).  Host function. */
NVFP4KV_API int nvfp4_kv_cache_key_ranges(const nvfp4_kv_cache_t* c, int* ranges) NVFP4KV_NOEXCEPT;

/* Attention of q (bf16 [Hq, Tq, head_dim], Hq a multiple of heads) over the
 * committed key set of one layer: nvfp4_kv_attention_chunked with that
 * layer's slot arrays, T = capacity * chunk_len and the ranges above
 * (workspace as there: nullable). */
NVFP4KV_API int nvfp4_kv_cache_attention(const nvfp4_kv_cache_t* c, const void* storage, size_t storage_bytes,
                                         int layer, const uint16_t* q, int Hq, int Tq, float softmax_scale,
                                         uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                                         void* stream) NVFP4KV_NOEXCEPT;

#ifdef __cplusplus
}
#endif

#endif /* NVFP4KV_H */
