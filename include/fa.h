/*
 * fa.h - C ABI of the MI355X (gfx950) fused-attention library.
 *
 * What the library computes (the definition every entry point reaches, up to
 * floating-point rounding order):
 *
 *   For batch b, query head h, query row i, with kv head g = floor(h * Hkv / Hq):
 *     J_i  = { j : 0 <= j < Skv, and (causal == 0 or j <= i + Skv - Sq) }
 *     s_ij = scale * sum_c q[b,h,i,c] * k[b,g,j,c]
 *     o[b,h,i,:] = sum_{j in J_i} softmax_j(s_i.) * v[b,g,j,:]
 *
 * Sources (the five web pages on small-batch fused attention):
 *   - "Real-time inference optimisation" (llmapi-app.pages.dev), section
 *     "Flash Attention optimisation": the tiled kernel with a running max m,
 *     running sum l and rescaled accumulator, normalised by l at the end.
 *   - "FlashRT-HF-kernels" (zingnex.cn), section "attention optimisation":
 *     FlashAttention-style tiling, online softmax, causal-mask optimisation for
 *     autoregressive generation, MQA/GQA; "Paged Attention" in the operator list.
 *   - "TensorRT support for FlashAttention" (yongjin360.com): the plugin's
 *     enqueue launches one kernel on Q, K, V, O with heads, seq_len_q,
 *     seq_len_kv, head_dim and a stream; it must answer shape/format queries or
 *     inference fails (hence the explicit status codes below).
 *   - "FasterTransformer source review" (pptc.cn), sections 1.1 and 3.1:
 *     context (prefill) is compute-bound, generation (decode) is memory-bound;
 *     section 2.3: the KV cache is preallocated and owned by the caller.
 *
 * Readings where the pages are silent (stated once here, used throughout):
 *   - causal alignment is bottom-right: query row i sits at absolute position
 *     Skv - Sq + i (equals top-left when Sq == Skv); causal with Sq > Skv is
 *     rejected with FA_ERR_SHAPE;
 *   - consecutive query heads share a kv head (g = floor(h * Hkv / Hq));
 *   - a row with no visible key (decode with seqlen 0) has output 0;
 *   - outputs have the dtype of q; bf16 rounding is round-to-nearest-even;
 *     all accumulation is fp32.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, contiguous row-major, and must be
 *     16-byte aligned (FA_ERR_ALIGN otherwise).
 *   - Every buffer is owned by the caller. The library never allocates, frees,
 *     copies or synchronises; it only enqueues kernels on `stream`
 *     (a hipStream_t; NULL means the default stream), so every call is safe to
 *     capture into a HIP graph.
 *   - Arguments are validated on the host before any launch; a failure returns
 *     its code and enqueues nothing. Device-resident integers (seqlens,
 *     block_table) are not read on the host; kernels clamp seqlens to
 *     [0, max_kv_len].
 *   - A launch error returns FA_ERR_HIP. Only the status of this call's own
 *     launches is reported: an error left pending by earlier runtime calls is
 *     neither reported nor cleared (the library never calls hipGetLastError).
 *     The decode entry points launch two kernels (one when every sequence
 *     fits one split); if the second launch fails, the first has been
 *     enqueued. Faults inside a kernel surface, as
 *     with any HIP work, at the caller's next synchronisation.
 *   - The library keeps no mutable global state and is re-entrant; calls on
 *     different streams that share a workspace race.
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                         */
  FA_ERR_SHAPE = 2,       /* a size is <= 0, Hq % Hkv != 0, causal with Sq > Skv */
  FA_ERR_UNSUPPORTED = 3, /* head_dim or page size the kernels do not provide    */
  FA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned             */
  FA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required             */
  FA_ERR_HIP = 6,         /* the HIP runtime rejected a launch                   */
  FA_ERR_ARG = 7          /* scale not finite, tokens_per_split invalid, ...     */
} fa_status;

/* Human-readable name of a status code (static storage, never NULL). */
const char* fa_status_string(fa_status s);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

/*
 * fa_prefill - causal or non-causal MQA/GQA attention over bf16 tensors
 * (the fused tiled kernel of the "Flash Attention optimisation" section of the
 * real-time inference page, with the causal mask and head sharing of the
 * FlashRT-HF-kernels page).
 *
 *   q, o : bf16 [B, Hq,  Sq,  d]     k, v : bf16 [B, Hkv, Skv, d]
 *   d    : 32, 64, 96, 128 or 256 (FA_ERR_UNSUPPORTED otherwise)
 *   scale: multiplier of q.k (normally 1/sqrt(d)); must be finite
 *   causal: 0 or 1; bottom-right aligned (see above)
 *
 * QK^T and PV run on bf16 MFMA with fp32 accumulation; the probabilities are
 * rounded to bf16 before the PV product; o is rounded to bf16 (RNE).
 * d = 64, 96 and 128 run on the two-group ping-pong kernel (d = 96 with its
 * LDS rows padded to 16 chunks of 16 bytes); d = 32 and 256 on a one-group
 * kernel (one 128-row query tile per work-group, 64-key K/V blocks
 * double-buffered in LDS; d = 256 at one wave per SIMD for its 128
 * accumulator registers).
 * o must not alias q, k or v.
 */
fa_status fa_prefill(const void* q, const void* k, const void* v, void* o,
                     int B, int Hq, int Hkv, int Sq, int Skv, int d,
                     float scale, int causal, void* stream);

/*
 * fa_prefill_f32 - the same operation with fp32 q, k, v, o and fp32 arithmetic
 * throughout (no bf16 rounding anywhere). Same arguments and layouts as
 * fa_prefill; d is 32, 64, 96, 128 or 256. Grids of at least 64 query tiles
 * of 128 rows (over heads and batch) at d <= 128 run on the fp32 matrix cores
 * (full fp32 products and sums); smaller ones on fp32 vector FMA.
 */
fa_status fa_prefill_f32(const void* q, const void* k, const void* v, void* o,
                         int B, int Hq, int Hkv, int Sq, int Skv, int d,
                         float scale, int causal, void* stream);

/*
 * fa_prefill_cache - fa_prefill with K and V read from a KV cache: the chunked
 * prefill of a serving loop, where each sequence's Sq new tokens have been
 * appended to its cache and attend to all of its cached tokens. Context and
 * generation phases with a KV cache are the FasterTransformer walkthrough's
 * sections 3.1 and 3.2; the cache layouts, page size and block table are
 * those of fa_decode (the paged sketch of the real-time inference page).
 *
 *   q, o        : bf16 [B, Hq, Sq, d], the new queries of each sequence.
 *   kcache, vcache, block_table, page_size, max_kv_len : as for fa_decode
 *                 (contiguous bf16 [B, max_kv_len, Hkv, d], or pages of 16
 *                 tokens through the block table).
 *   seqlens     : int32 [B] device array: cached tokens of each sequence,
 *                 the Sq new ones included, clamped to [0, max_kv_len].
 *   causal      : 1 -> query row i of sequence b sees cached tokens
 *                 j <= i + seqlens[b] - Sq (the new tokens are the last Sq);
 *                 a row that sees no token (seqlens[b] < Sq) gives zeros.
 *                 0 -> every row sees all seqlens[b] tokens (zeros if none).
 *   scale, d, stream, errors : as for fa_prefill (d = 32, 64, 96, 128 or
 *                 256), plus FA_ERR_NULL for a NULL seqlens and
 *                 FA_ERR_UNSUPPORTED for a page size other than 16.
 * The same kernels as fa_prefill compute it. At d = 64, 96 and 128 the
 * ping-pong kernel takes one query tile per work-group (the sequences' tiles
 * ordered by cached length, longest first), so with a cache holding exactly
 * fa_prefill's K and V the two agree to rounding; at d = 32 and 256 the
 * one-group kernel runs as for fa_prefill (at d = 32 with the same bits;
 * d = 256 may differ from fa_prefill's key-split kernel by rounding).
 * For the same seqlens the paged and contiguous caches give bitwise equal
 * results.
 */
fa_status fa_prefill_cache(const void* q, const void* kcache, const void* vcache,
                           const int32_t* block_table, const int32_t* seqlens, void* o,
                           int B, int Hq, int Hkv, int Sq, int d, int max_kv_len,
                           int page_size, float scale, int causal, void* stream);

/*
 * fa_decode_split_tokens - the KV tokens each split work-group of fa_decode
 * covers (n_split = ceil(max_kv_len / result) splits per sequence; this sizes
 * the workspace).
 * tokens_per_split == 0 asks for the default. With S = B * Hkv *
 * ceil((Hq/Hkv)/16) split streams: max_kv_len rounded up to a multiple of 32
 * (one split per sequence, so fa_decode is one launch) when max_kv_len <= 512,
 * or when max_kv_len <= 2048 and 8 * S >= max_kv_len; otherwise the smallest
 * power of two in [64, 1024] for which S * n_split stays near 256 work-groups
 * (one per compute unit), so long sequences are split finely enough to fill
 * the GPU; 1024 keeps a 262144-token sequence at 256 splits.
 * With the default and B <= 4096, fa_decode itself may then enlarge the split
 * to 5/4, 3/2 or 2 times this value (a multiple of 32, at most 2048) once it
 * sees seqlens on the device: it takes the size with the fewest tokens per
 * work-group slot over the rounds of resident split work-groups (two per
 * compute unit, one at d = 256) that the live splits need, the smallest on a
 * tie. Splits only
 * get larger, so the workspace always suffices.
 * Any other value must be a positive multiple of 32, at most 2048, and is
 * returned unchanged and used as given. Returns 0 for invalid arguments.
 */
int fa_decode_split_tokens(int B, int Hq, int Hkv, int max_kv_len, int tokens_per_split);

/*
 * fa_decode_workspace_bytes - bytes of device workspace fa_decode needs:
 * fp32 partial outputs [B, Hq, n_split, d] and partial log-sum-exps
 * [B, Hq, n_split], each rounded up to 256 bytes, with n_split as above, then
 * 256 bytes whose first int32 receives the split size the call used.
 * Returns 0 for invalid arguments.
 */
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int max_kv_len, int tokens_per_split);

/*
 * fa_decode - one query token per sequence attending to all of its cached
 * keys (the paged attention of the FlashRT-HF-kernels operator list and of the
 * real-time inference page's paged sketch, with the page combination done by a
 * log-sum-exp merge instead of the sketch's plain sum, which is wrong).
 *
 *   q, o        : bf16 [B, Hq, d]
 *   block_table : NULL  -> contiguous cache, kcache/vcache bf16 [B, max_kv_len, Hkv, d]
 *                 !NULL -> paged cache, kcache/vcache bf16 [num_pages, 16, Hkv, d];
 *                          block_table int32 [B, ceil(max_kv_len/16)], entry
 *                          [b][p] is the physical page of tokens 16p..16p+15 of
 *                          sequence b; entries p >= ceil(seqlens[b]/16) are never
 *                          used and may hold anything (they may be read, within
 *                          the row, before seqlens is known, so the whole table
 *                          must be allocated); the pages used must be in range
 *                          (not checked).
 *   seqlens     : int32 [B] device array, tokens cached for each sequence,
 *                 clamped to [0, max_kv_len]; length 0 gives o = 0.
 *   page_size   : must be 16 when block_table != NULL (ignored otherwise).
 *   tokens_per_split : KV tokens per split work-group; 0 -> the default of
 *                 fa_decode_split_tokens; otherwise a positive multiple of 32,
 *                 at most 2048.
 *   workspace   : device scratch of at least fa_decode_workspace_bytes(...)
 *                 bytes, 16-byte aligned; contents undefined after the call.
 *   d           : 32, 64, 96, 128 or 256.  Hq / Hkv query heads share one
 *                 kv head. (At d = 96, and at d = 32 over one-byte caches,
 *                 the kernel pads its LDS rows to a power of two of 16-byte
 *                 chunks; the cache layout is unpadded.)
 *
 * Two kernels run in stream order: a split-KV kernel writing per-split
 * (normalised output, log-sum-exp), then the log-sum-exp merge into o.
 * When every sequence fits one split (max_kv_len <= the split size; the
 * default gives this for short capacities, see fa_decode_split_tokens), the
 * split kernel writes o itself and the
 * merge is not launched: one kernel per call, with the bits the merge would
 * give (a single split has weight exactly 1). The workspace is still required.
 * For the same tokens_per_split and seqlens (the default split size depends on
 * them) the paged and contiguous paths perform the same arithmetic in the same
 * order, so their results are bitwise equal.
 */
fa_status fa_decode(const void* q, const void* kcache, const void* vcache,
                    const int32_t* block_table, const int32_t* seqlens, void* o,
                    int B, int Hq, int Hkv, int d, int max_kv_len, int page_size,
                    int tokens_per_split, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_fp8 - fa_decode over a KV cache stored as 8-bit floats, one byte
 * per element: the low-precision KV cache of the FasterTransformer source
 * walkthrough (section 3.3, an 8-bit KV cache that halves the bytes a decode
 * step reads) in the FP8 form of the FlashRT project summary (8-bit floating
 * point with one scale per tensor).
 *
 *   kcache, vcache : uint8 OCP FP8 E4M3 codes (bias 7, no infinities, codes
 *                    0x7F / 0xFF are NaN) in the layouts of fa_decode;
 *                    element value = k_scale * E4M3(code) for K and
 *                    v_scale * E4M3(code) for V.
 *   k_scale, v_scale : finite and > 0, else FA_ERR_ARG.
 *   Every other argument, the workspace (same size and use) and the errors
 *   are those of fa_decode; q and o stay bf16. K and V are widened to bf16
 *   exactly (every E4M3 value is a bf16 value), so the result is that of
 *   fa_decode on the dequantised cache up to the rounding of the scales.
 */
fa_status fa_decode_fp8(const void* q, const void* kcache, const void* vcache,
                        const int32_t* block_table, const int32_t* seqlens, void* o,
                        int B, int Hq, int Hkv, int d, int max_kv_len, int page_size,
                        int tokens_per_split, float scale, float k_scale, float v_scale,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_int8 - fa_decode over a KV cache stored as signed 8-bit integers,
 * one byte per element: the INT8 KV cache of the FasterTransformer source
 * walkthrough (section 3.3, an 8-bit KV cache that halves the bytes a
 * decode step reads), with one scale per tensor.
 *
 *   kcache, vcache : int8 codes (two's complement, -128..127) in the layouts
 *                    of fa_decode; element value = k_scale * code for K and
 *                    v_scale * code for V.
 *   k_scale, v_scale : finite and > 0, else FA_ERR_ARG.
 *   Every other argument, the workspace (same size and use) and the errors
 *   are those of fa_decode; q and o stay bf16. K and V are widened to bf16
 *   exactly (every integer in -128..127 is a bf16 value), so the result is
 *   that of fa_decode on the dequantised cache up to the rounding of the
 *   scales. There is no NaN code: slots past a sequence's length are never
 *   read, whatever they hold.
 */
fa_status fa_decode_int8(const void* q, const void* kcache, const void* vcache,
                         const int32_t* block_table, const int32_t* seqlens, void* o,
                         int B, int Hq, int Hkv, int d, int max_kv_len, int page_size,
                         int tokens_per_split, float scale, float k_scale, float v_scale,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_merge_lse - combine R rows of S partial attention results by
 * log-sum-exp (the merge step that replaces the per-page sum of the paged
 * sketch on the real-time inference page):
 *   M = max_s lse[r,s];  w_s = exp(lse[r,s] - M)
 *   o[r,:] = sum_s w_s * o_parts[r,s,:] / sum_s w_s;  lse_out[r] = M + ln(sum_s w_s)
 * Splits with lse = -inf are empty and are skipped (their o_parts are never
 * read); a row whose splits are all empty gets o = 0 and lse_out = -inf.
 *
 *   o_parts : fp32 [R, S, d] (each part already normalised by its own sum)
 *   lse     : fp32 [R, S] natural-log log-sum-exp of each part's scores
 *   o       : [R, d], bf16 when out_bf16 != 0, else fp32
 *   lse_out : fp32 [R] or NULL
 *   d       : 32, 64, 96, 128 or 256
 */
fa_status fa_merge_lse(const float* o_parts, const float* lse, void* o, float* lse_out,
                       int R, int S, int d, int out_bf16, void* stream);

/*
 * fa_decode_noalloc - fa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc. It takes no workspace. The split partials live in a
 * device array inside the library (16 MiB, one per GPU, held until the process
 * ends); the call itself allocates, frees and copies nothing.
 *
 *   Arguments, layouts, results and every status of fa_decode (bf16 cache),
 *   without workspace and workspace_bytes.
 *   FA_ERR_WORKSPACE: the sizes need more than 16 MiB of partials, i.e.
 *     fa_decode_workspace_bytes(B, Hq, Hkv, d, max_kv_len, tokens_per_split)
 *     > 16777216 (for example B * Hq * ceil(max_kv_len / split) > 31,000 rows
 *     at d = 128).
 *   FA_ERR_HIP: the array's device address could not be obtained.
 *
 * The first call on a device looks up the array's address on that device; make
 * it outside graph capture. All calls on one GPU share its array, which keeps
 * the last call's contents (nothing in it needs clearing): calls that can
 * overlap on one GPU (different streams, or replays of several captured
 * graphs without ordering) race and must be serialised by the caller.
 */
fa_status fa_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                            const int32_t* block_table, const int32_t* seqlens, void* o,
                            int B, int Hq, int Hkv, int d, int max_kv_len, int page_size,
                            int tokens_per_split, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
