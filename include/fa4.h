/*
 * fa4.h - block-scaled low-bit fused attention on AMD MI355X (gfx950): the C ABI.
 *
 * Four entry points make up the path:
 *   fa4_quantize_blockscaled  Q/K -> 4-bit E2M1 with block scales (MXFP4 or NVFP4), V -> FP8 E4M3
 *                             (fa4_quantize_prefill: Q, K and V of a prefill in one launch)
 *   fa4_select_tiles          ThriftAttention-style choice of the 128x128 tiles computed in bf16
 *   fa4_attn_fwd              fused prefill attention (scaled-MFMA QK^T and PV, FP32 online softmax)
 *   fa4_decode_paged          decode attention over a paged FP4 (NVFP4 or MXFP4) KV cache
 *                             (fa4_decode_paged_noalloc: the same without a caller workspace)
 *
 * Conventions shared by every call:
 *   - Every pointer in an argument struct is a DEVICE pointer owned by the caller and must stay valid
 *     until the work enqueued on `stream` has finished. The library allocates nothing and keeps no
 *     state apart from a thread-local error string.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls enqueue work and return at once.
 *   - Arguments are validated before anything is enqueued; a failed check returns its status and
 *     enqueues nothing. fa4_last_error() then names the failed check. Launch failures return
 *     FA4_ERR_HIP; faults inside a kernel surface at the caller's next synchronisation.
 *   - Inputs must be finite; non-finite inputs give unspecified values but never out-of-bounds access.
 *   - All reductions are deterministic: equal inputs give bitwise-equal outputs.
 *   - Element sizes: codes are bytes; 4-bit codes are packed two per byte, element 2i in bits 3:0 and
 *     element 2i+1 in bits 7:4. E2M1 value grid: {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign bit.
 *     E4M3 is the OCP "fn" variant (largest finite 448, no infinities). E8M0 byte c means 2^(c-127).
 */
#ifndef FA4_H
#define FA4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA4_OK = 0,
  FA4_ERR_NULL = 1,          /* a required pointer is NULL                              */
  FA4_ERR_SHAPE = 2,         /* a size is out of range or inconsistent                   */
  FA4_ERR_UNSUPPORTED = 3,   /* a valid but unimplemented combination (format, d, flags) */
  FA4_ERR_ALIGN = 4,         /* a pointer is not aligned as documented                   */
  FA4_ERR_WORKSPACE = 5,     /* workspace missing or smaller than required               */
  FA4_ERR_HIP = 6            /* the HIP runtime reported an error                        */
} fa4_status;

enum { FA4_F32 = 0, FA4_BF16 = 1 };                      /* input element types       */
enum { FA4_MXFP4 = 0, FA4_NVFP4 = 1, FA4_FP8_TOKEN = 2, FA4_MXFP8 = 3, FA4_MXFP4_KEYS = 4 }; /* quantized formats */
enum { FA4_P_FP8 = 0, FA4_P_NVFP4 = 1, FA4_P_MXFP4 = 2 };  /* probability formats (decode: FP8, NVFP4;
                                                               prefill: FP8, MXFP4)        */
enum { FA4_HADAMARD128 = 1u << 0, FA4_DUAL_RESIDUAL = 1u << 1, FA4_SCALE_SEARCH = 1u << 2 }; /* quantizer flags */

/* ------------------------------------------------------------------------------------------------
 * Quantization.
 *
 * Source pages: "MXFP vs NVFP4" (tqpw.cn 81738) sections 2.1-2.2 (MXFP4: 32-element blocks with an
 * E8M0 scale; NVFP4: 16-element blocks with an E4M3 scale and an FP32 tensor scale);
 * "General notes on quantization" (zdszero) (X ~ s * Q; per-token / per-group / per-tensor scales);
 * "BitDecoding-FP4" (dual-residual query quantization, Hadamard rotation before key quantization);
 * "MpFA QK4V8" sections 2.1-2.2 (Q and K in 4 bits, V in 8 bits).
 *
 * Input rows: the tensor is a set of groups g = o * heads + h (o < outer, h < heads), each holding
 * `rows` rows of d elements; row r of group (o, h) starts at element
 *     o * stride_outer + h * stride_head + r * stride_row        (element strides, not bytes).
 * row_counts (optional, [outer] int32): only rows r < row_counts[o] exist (a ragged batch).
 * page_table (optional, [outer][max_pages] int32): write rows into a paged cache; row r of group
 * (o, h) goes to output row (page_table[o][r / page_size] * heads + h) * page_size + r % page_size.
 * Without a page table, row r of group g goes to output row g * rows + r.
 *
 * Formats (per output row of d elements):
 *   FA4_MXFP4: codes [d/2] bytes; block_scales [d/32] E8M0: per 32 elements, amax = max|x|, scale =
 *              the smallest power of two 2^e with 6 * 2^e >= amax (e = -127 if amax = 0), codes =
 *              E2M1(x * 2^-e) rounded to nearest even. `scales` unused (may be NULL).
 *   FA4_NVFP4: codes [d/2]; block_scales [d/16] E4M3; scales = tensor scale per group [outer*heads]
 *              float: s_t = amax_group / 2688 (1 if that float32 quotient is zero, i.e. amax = 0 or
 *              below ~2.7e-42; all block scales are then 0), s_b = E4M3(amax_block / (6 s_t)),
 *              codes = E2M1(x / (E4M3value(s_b) * s_t)) (float32, IEEE division); value = code*s_b*s_t.
 *   FA4_MXFP8: codes [d] E4M3; block_scales [d/32] E8M0: per 32 elements, the smallest power of two
 *              2^e with 448 * 2^e >= amax (e = -127 if amax = 0), codes = E4M3(x * 2^-e) rounded to
 *              nearest even ("MXFP vs NVFP4" sections 2.1 and 4.2). `scales` unused.
 *   FA4_FP8_TOKEN: codes [d] E4M3; scales = per-row float [out rows]: s = amax_row / 448 (1 if zero),
 *              codes = E4M3(x / s). block_scales unused.
 *   FA4_MXFP4_KEYS (4-bit V for fa4_attn_fwd; "MpFA QK4V8" section 6 names 4-bit V): MXFP4 with the
 *              32-element blocks along the rows (the keys) of each column, i.e. the MXFP4 rule above
 *              applied to the columns. codes [groups][d][rows/2]: column c's values along the rows, two
 *              per byte, low nibble first, and within each block of 32 rows code position j holds row
 *              8 ((j >> 2) & 3) + 4 (j >> 4) + (j & 3) of the block (the key order of the attention's FP8
 *              probability operand); block_scales [groups][d][rows/32] E8M0. rows % 32 == 0; no flags,
 *              residual, row norms, paging, ragged rows, smoothing or fold outputs.
 * flags: FA4_HADAMARD128 rotates each row by the Sylvester Hadamard matrix H_128 / sqrt(128) (float64,
 *        rounded to float32) before quantizing (d must be 128; NVFP4 or MXFP4 only).
 *        FA4_DUAL_RESIDUAL (NVFP4 or MXFP4): `out` receives Q1 = F(x) and `residual` receives
 *        Q2 = F(float32(x - dequant(Q1))) in the same format F (`residual->fmt` must equal
 *        `out->fmt`); NVFP4 residuals get their own tensor scales, MXFP4 ones need none.
 *        FA4_SCALE_SEARCH (MXFP4 or NVFP4, not with FA4_DUAL_RESIDUAL): per-block scale search
 *        ("BitDecoding-FP4", outlier-aware key quantization). Candidates: MXFP4 exponents e, e - 1;
 *        NVFP4 E4M3 block-scale codes c, c - 1, c + 1, c - 2 within [1, 126] (e, c: the round-to-
 *        nearest scales above; the NVFP4 tensor scale is not searched, a zero c is kept). Each is
 *        scored by the block's squared error sum (x - x^)^2 in float64, summed as a balanced binary
 *        tree over the block's elements in index order; the first candidate in the listed order with
 *        the smallest error wins.
 * channel_scale (optional, [heads][d] float): static smoothing. Element c of a row of head h is
 *        multiplied by channel_scale[h * d + c] (float32 product) before rotation and quantization
 *        (row_norm2 still describes the unscaled rows). fa4_smoothing_factors produces power-of-two
 *        factors, for which the products are exact.
 * fold_w / fold_scale (FP8_TOKEN, optional, unpaged, rows a multiple of 128): the data that folds the
 *        per-token V scale into the attention probabilities. For each 128-row tile j of a group,
 *        fold_scale[j] = 2^e (a float), e = the smallest integer with 448 * 2^e >= max of the tile's
 *        scales (clamped to [-127, 127]), and for each row c, fold_w[c] = s[c] * 2^-e (exact, <= 448).
 *        fa4_attn_fwd consumes both arrays.
 * row_norm2 (optional, [outer*heads*rows] float, unpaged only): squared L2 norm of each UNROTATED
 *        input row, float64 pairwise (binary-tree) sum over d, rounded to float32.
 * During the call the tensor-scale array holds intermediate maxima; it holds s_t when the work ends.
 * Requirements: d in {64, 128}; x and codes 16-byte aligned, block and tensor scales 4-byte aligned;
 * strides multiples of 16 bytes (8 bf16 or 4 float elements). Returns FA4_ERR_* without enqueuing on
 * a failed check.
 */
typedef struct {
  const void *x;               /* input elements (FA4_F32 float or FA4_BF16 bf16 bits)            */
  int32_t dtype;               /* FA4_F32 or FA4_BF16                                             */
  int32_t d;                   /* row length: 64 or 128                                           */
  int64_t outer;               /* number of outer indices o                                       */
  int32_t heads;               /* heads per outer index                                           */
  int64_t rows;                /* rows per group (the maximum when row_counts is given)            */
  int64_t stride_outer, stride_head, stride_row;   /* element strides                             */
  const int32_t *row_counts;   /* optional [outer]                                                */
  const int32_t *page_table;   /* optional [outer][max_pages]                                     */
  int32_t page_size, max_pages;
  int64_t num_pages;           /* pages in the output cache (paged output only)                   */
  const float *channel_scale;  /* optional [heads][d] static smoothing factors                    */
} fa4_qinput;

typedef struct {
  int32_t fmt;                 /* FA4_MXFP4, FA4_NVFP4 or FA4_FP8_TOKEN                           */
  uint8_t *codes;
  uint8_t *block_scales;
  float *scales;               /* NVFP4: [outer*heads] tensor scales; FP8_TOKEN: [out rows]       */
  float *fold_w;               /* FP8_TOKEN, optional: [out rows] P-fold factor w (see below)     */
  float *fold_scale;           /* FP8_TOKEN, optional: [out rows / 128] tile maximum of the scales */
} fa4_qoutput;

fa4_status fa4_quantize_blockscaled(const fa4_qinput *in, uint32_t flags, const fa4_qoutput *out,
                                    const fa4_qoutput *residual, float *row_norm2, void *stream);

/* The three quantizations of a prefill in one launch.
 *
 * Source pages: "MpFA QK4V8" sections 2.1-2.2 (Q and K in 4 bits, V in 8 bits, quantized before the
 * attention kernel); "MXFP vs NVFP4" (tqpw.cn 81738) section 3.1 (fused quantization kernels with
 * coalesced global-memory access).
 * Writes exactly what three fa4_quantize_blockscaled calls with flags = 0 would write: q and k into
 * q_out and k_out (both FA4_MXFP4 or both FA4_MXFP8, with row norms into q_norm2 / k_norm2 when both
 * are given), v into v_out (FA4_FP8_TOKEN with fold_w and fold_scale, or FA4_MXFP4_KEYS, 4-bit V, when
 * Q and K are MXFP4 and d = 128). Inputs as for
 * fa4_quantize_blockscaled; q, k and v share dtype and d, are unpaged and not ragged (row_counts NULL),
 * and v's rows are a multiple of 128 (FP8) or 32 (4-bit V). Rotation, the dual residual, the scale
 * search and NVFP4 are not offered here (use the separate calls). One launch lets the three streams' start-up and
 * drain overlap, which matters at a few tens of MB per tensor.
 */
fa4_status fa4_quantize_prefill(const fa4_qinput *q, const fa4_qinput *k, const fa4_qinput *v,
                                const fa4_qoutput *q_out, const fa4_qoutput *k_out, const fa4_qoutput *v_out,
                                float *q_norm2, float *k_norm2, void *stream);

/* Static smoothing factors for outlier-aware key quantization.
 *
 * Source page: "BitDecoding-FP4" (sns.style digest): static smoothing, with the Hadamard rotation and
 * the scale search, spreads key outliers before FP4 quantization.
 * From calibration tensors q (heads Hq) and k (heads Hkv, Hq % Hkv == 0, same d; layouts as
 * fa4_qinput, unpaged; channel_scale ignored): amax_K[kv][c] = max |k| over outer and rows of key
 * head kv; amax_Q[kv][c] = max |q| over outer, rows and the query heads kv*G .. kv*G+G-1 (G = Hq/Hkv).
 * With e = floor(log2 amax): k = floor((e_K - e_Q + 1) / 2), clamped to [-20, 20], and k = 0 when either
 * maximum is zero. Output: k_scale [Hkv][d] = 2^-k, q_scale [Hq][d] = 2^k (the same for the heads of
 * a group), to be passed as channel_scale when quantizing K and Q: QK^T is unchanged (exact products).
 * Requirements as fa4_quantize_blockscaled's input (alignment, d in {64, 128}); outputs 4-byte aligned.
 */
fa4_status fa4_smoothing_factors(const fa4_qinput *q_calib, const fa4_qinput *k_calib, float *q_scale,
                                 float *k_scale, void *stream);

/* ------------------------------------------------------------------------------------------------
 * Tile selection.
 *
 * Source page: "ThriftAttention" (ai-feeds.com summary), Method step 2 and Limitations: 128x128
 * query-key tiles are scored cheaply from norms and the top ~5% are computed in high precision.
 *
 * q_norm2 [B][Hq][Lq], k_norm2 [B][Hkv][Lk]: squared row norms (fa4_quantize_blockscaled's row_norm2).
 * a_i = max q_norm2 over q-tile i, b_j = max k_norm2 over k-tile j (key head h / (Hq/Hkv));
 * score_ij = float32(a_i * b_j). Candidates are the valid tiles: all tiles if !causal, else those with
 * 128 j <= (Lk - Lq) + 128 i + 127 (query i sits at key position Lk - Lq + i). Per (b, h) the
 * k = ceil(num * N_valid / den) best candidates are chosen, ordered by score (descending) then by
 * linear index i * (Lk/128) + j (ascending), so the choice is unique.
 * Output: bitmap [B][Hq][Lq/128][Lk/128] bytes (1 = bf16 tile), counts [B][Hq] int32 (optional).
 * Requirements: Lq, Lk multiples of 128; Lq/128 <= 1024; Lk/128 <= 4096; Hq % Hkv == 0;
 * 0 <= num <= den, den > 0.
 */
fa4_status fa4_select_tiles(const float *q_norm2, const float *k_norm2, int32_t B, int32_t Hq,
                            int32_t Hkv, int32_t Lq, int32_t Lk, int32_t causal, int32_t num,
                            int32_t den, uint8_t *bitmap, int32_t *counts, void *stream);

/* ------------------------------------------------------------------------------------------------
 * Prefill attention.
 *
 * Source pages: "MpFA QK4V8" sections 2.1-2.2, 3.2-3.4 (4-bit QK^T with in-kernel block scales, 8-bit
 * PV, FP32 online softmax, tiling); "ThriftAttention" Method step 3 (selected tiles in high precision
 * merged through the same online softmax); "BitDecoding-FP4" (probabilities quantized with a scale
 * that cannot underflow); "General notes on quantization" (scale factoring / merging of scales).
 *
 * For query row r of head h (key head kv = h / (Hq/Hkv), query position Lk - Lq + r) and each
 * 128-key tile j holding an unmasked key (key c unmasked if !causal or c <= r + Lk - Lq):
 *   S = softmax_scale * q~ . k~ with the dequantized Q/K codes (or the bf16 originals if selected);
 *   all per-tile scales are powers of two: r = ceil(tile row max of S log2(e)), P' = 2^(S log2(e) - r);
 *   unselected: 2^e = the tile's fold_scale, w_c = s_v[c] 2^-e (fold_w), P^ = E4M3(P' w_c),
 *               T = 2^e * sum_c P^ * E4M3value(Vcode_c)     (FP8 x FP8 products);
 *   selected:   T = sum_c bf16(P') * v_c with the bf16 originals;
 *   O = sum_j 2^(r_j - m) T_j / sum_j 2^(r_j - m) sum_c P'   (m = max_j r_j), LSE = m ln 2 + ln(denominator).
 * Layouts: q_codes [B][Hq][Lq][d/2] (MXFP8: [d] E4M3), q_scales [B][Hq][Lq][d/32] (MXFP4, MXFP8: E8M0)
 * or [d/16] (NVFP4) with q_tscale [B*Hq]; k_* likewise over [B][Hkv][Lk]; v_codes [B][Hkv][Lk][d] E4M3 with v_scales
 * [B][Hkv][Lk], v_fold_w [B][Hkv][Lk] and v_fold_scale [B][Hkv][Lk/128] (the quantizer's fold
 * outputs); q_bf16 [B][Hq][Lq][d], k_bf16 / v_bf16 [B][Hkv][Lk][d] (bf16 bits; required when
 * bitmap is given); bitmap [B][Hq][Lq/128][Lk/128] or NULL; o [B][Hq][Lq][d] float; lse [B][Hq][Lq]
 * float or NULL. Requirements: d = 128 (or 64 for MXFP4 without a bitmap); Lq, Lk multiples of 128;
 * Lq <= Lk when causal; Hq % Hkv == 0; every pointer 16-byte aligned.
 * 4-bit V (v_fmt = FA4_MXFP4_KEYS; MXFP4 Q/K, d = 128): v_codes [B][Hkv][d][Lk/2] and v_block_scales as
 * fa4_quantize_blockscaled's FA4_MXFP4_KEYS output; v_scales and v_fold_* are not read. Quantized tiles
 * then take P^ = E4M3(448 P') and T = (1/448) sum_c P^ v^_c with the dequantized 4-bit values v^ (FP4
 * V^T times FP8 P^T in one block-scaled MFMA); selected tiles (with a bitmap) read v_bf16 as usual.
 * FP4 probabilities (p_fmt = FA4_P_MXFP4; MXFP4 Q/K, d = 128; "BitDecoding-FP4": probabilities
 * in FP4 under a scale that cannot underflow, "MXFP vs NVFP4" section 2.1: the MX block): in each
 * unselected tile row, P' w_c over 32 consecutive keys (keys 128 j + 32 b .. + 31) is one MXFP4 block:
 * 2^e_b = the smallest power of two with 6 * 2^e_b >= its largest P' w, P^ = E2M1(P' w 2^-e_b) 2^e_b,
 * T = 2^e * sum_c P^ * E4M3value(Vcode_c) (FP8 V^T times FP4 P^T in one block-scaled MFMA, e_b and the
 * tile weight as P^T's E8M0 operand scale). With 4-bit V the block is P' itself (nothing to fold, no 448)
 * and T = sum_c P^ v^_c: FP4 V^T times FP4 P^T, both block scales inside the product. p_fmt = 0
 * (FA4_P_FP8) keeps the FP8 probabilities above.
 */
typedef struct {
  int32_t fmt;                                  /* FA4_MXFP4, FA4_NVFP4 or FA4_MXFP8 (Q and K) */
  const uint8_t *q_codes, *q_scales; const float *q_tscale;
  const uint8_t *k_codes, *k_scales; const float *k_tscale;
  const uint8_t *v_codes; const float *v_scales;
  const float *v_fold_w, *v_fold_scale;        /* fa4_quantize_blockscaled's FP8 fold outputs     */
  const uint16_t *q_bf16, *k_bf16, *v_bf16;
  const uint8_t *bitmap;
  int32_t B, Hq, Hkv, Lq, Lk, d, causal;
  float softmax_scale;
  float *o;
  float *lse;
  int32_t v_fmt;                               /* 0 or FA4_FP8_TOKEN: v_codes/v_scales/v_fold_* as above;
                                                  FA4_MXFP4_KEYS: 4-bit V (see below)                  */
  const uint8_t *v_block_scales;               /* FA4_MXFP4_KEYS: E8M0 [B][Hkv][d][Lk/32]             */
  int32_t p_fmt;                               /* FA4_P_FP8 (0) or FA4_P_MXFP4 (see above)            */
} fa4_attn_args;

fa4_status fa4_attn_fwd(const fa4_attn_args *a, void *stream);

/* ------------------------------------------------------------------------------------------------
 * Paged decode.
 *
 * Source page: "BitDecoding-FP4" (sns.style digest): native FP4 KV-cache decode over pages (NVFP4 and
 * MXFP4 caches), dual-residual query (q ~ Q1 + Q2, both FP4), underflow-aware probability scaling,
 * query heads of one GQA group stacked into one matrix-core tile.
 *
 * For sequence b and query head h (key head kv = h / (Hq/Hkv)) over keys c < ctx_len[b]:
 *   q^ = dequant(Q1) + dequant(Q2); S_c = softmax_scale * q^ . k^_c with the dequantized keys;
 *   per 128-key tile (from position 0, the last one partial): m~ = tile max, P' = exp(S - m~),
 *   P^ = E4M3(448 P'), T = (1/448) sum_c P^ v^_c; O = sum e^(m~-m) T / sum e^(m~-m) sum P'.
 * fmt selects the format of Q1, Q2, K and V (all alike):
 *   FA4_NVFP4: q1_scales/q2_scales [B][Hq][d/16] E4M3 with q1_tscale/q2_tscale [B*Hq];
 *              k_scales/v_scales [num_pages][Hkv][page_size][d/16] E4M3 with k_tscale/v_tscale [B][Hkv].
 *   FA4_MXFP4: q1_scales/q2_scales [B][Hq][d/32] E8M0; k_scales/v_scales [num_pages][Hkv][page_size]
 *              [d/32] E8M0; the four tensor-scale pointers are not read (may be NULL).
 * Other layouts: q1_codes/q2_codes [B][Hq][d/2]; k_codes/v_codes [num_pages][Hkv][page_size][d/2];
 * page_table [B][max_pages] (entries past ceil(ctx_len[b]/page_size) are not read); o [B][Hq][d] float.
 * p_fmt selects the format of the probabilities before PV:
 *   FA4_P_FP8 (0, the default): P^ = E4M3(448 P') as above.
 *   FA4_P_NVFP4: FP4 with E4M3 scales per 16 keys (the case in which a block scale can round to zero).
 *              Each tile row of P' (its largest element exactly 1) is one NVFP4 group: tensor scale
 *              s_t = fl32(1/2688), block scale s_b = E4M3(amax_b / fl32(6 s_t)) per 16 keys from the
 *              tile start, P^ = E2M1(P' / (s_b s_t)) * s_b * s_t, T = sum_c P^ v^_c. A block scale is
 *              zero only when the block's largest probability is under 2^-10/448 of the tile's.
 * The work is split over key ranges; partial results go to a caller-provided workspace of
 * fa4_decode_workspace_bytes(a) bytes (256-byte aligned) and are merged by a second kernel.
 * Requirements: d = 128; page_size = 64; Hq a multiple of Hkv with at most 64 query heads per key head
 * (groups of up to 4 of them share one pass over the key head's pages, so 4 per key head reads the
 * cache once and 8 reads it twice); 0 <= ctx_len[b] <= max_pages * page_size (a sequence with
 * ctx_len[b] = 0 reads no page and gets O = 0, in both geometries).
 *
 * MLA geometry (d_v = 512; "BitDecoding-FP4" reports the method on MLA attention as well): every query
 * head of sequence b attends to one shared latent row per token, whose d = 576 values (512 latent, 64
 * rotary) are the key and whose first d_v = 512 values are the value; q1/q2 hold each head's absorbed
 * query. Probability tiles are one 64-key page (otherwise as above, P^ = E4M3(448 P')).
 *   fmt = FA4_MXFP4, p_fmt = FA4_P_FP8, Hq = 16, Hkv = 1, d = 576, page_size = 64.
 *   q1_codes/q2_codes [B][Hq][288], q1_scales/q2_scales [B][Hq][18] E8M0.
 *   k_codes [num_pages][9][64][32] and k_scales [num_pages][9][64][2] E8M0: slice j of a page holds
 *   columns 64 j .. 64 j + 63 of its 64 rows (fa4_quantize_blockscaled's paged output for the rows
 *   taken as nine 64-wide heads). v_codes, v_scales and the tensor scales are not read (may be NULL).
 *   o [B][Hq][512] float. Workspace: fa4_decode_workspace_bytes(a).
 */
typedef struct {
  int32_t fmt;                                  /* FA4_NVFP4 or FA4_MXFP4 (Q1, Q2, K and V)     */
  const uint8_t *q1_codes, *q1_scales; const float *q1_tscale;
  const uint8_t *q2_codes, *q2_scales; const float *q2_tscale;
  const uint8_t *k_codes, *k_scales, *v_codes, *v_scales;
  const float *k_tscale, *v_tscale;
  const int32_t *page_table, *ctx_len;
  int32_t B, Hq, Hkv, d, page_size, max_pages;
  int64_t num_pages;
  float softmax_scale;
  float *o;
  int32_t p_fmt;                                /* FA4_P_FP8 (0) or FA4_P_NVFP4                 */
  int32_t d_v;                                  /* 0: GQA geometry; 512: MLA geometry (below)   */
} fa4_decode_args;

size_t fa4_decode_workspace_bytes(const fa4_decode_args *a);
fa4_status fa4_decode_paged(const fa4_decode_args *a, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * fa4_decode_paged without a workspace argument, for callers that cannot allocate device memory (code
 * recorded into a HIP graph, tight serving loops, harnesses that forbid allocation). It computes exactly
 * what fa4_decode_paged computes, with the same kernels and the same validation, and allocates nothing:
 * the split partials go to a scratch array of FA4_DECODE_SCRATCH_BYTES that the library holds as a
 * device global on every GPU it runs on, for the life of the process. Its address on the current device
 * is looked up once per device, on that device's first call.
 *   - Returns FA4_ERR_WORKSPACE, enqueuing nothing, when fa4_decode_workspace_bytes(a) exceeds
 *     FA4_DECODE_SCRATCH_BYTES (for example 64 sequences of 32K tokens need 17 MB in the GQA geometry and
 *     34 MB in the MLA geometry).
 *   - Every call on one GPU uses that GPU's one array, and nothing in it needs to start at any value (each
 *     call writes every partial it reads). Calls that overlap on one GPU (on different streams, or from
 *     different threads without ordering) race on it: order them, or use fa4_decode_paged with
 *     workspaces of their own.
 */
#define FA4_DECODE_SCRATCH_BYTES ((size_t)40 << 20)
fa4_status fa4_decode_paged_noalloc(const fa4_decode_args *a, void *stream);

/* ------------------------------------------------------------------------------------------------ */
const char *fa4_status_string(int status);   /* static text of a status code                        */
const char *fa4_last_error(void);            /* detail of this thread's last failed call ("" if none) */

#ifdef __cplusplus
}
#endif
#endif /* FA4_H */
