/*
 * sage.h -- C ABI of the MI355X (gfx950) quantized attention forward pass.
 *
 * The method (SageAttention2 detail page, Algorithm 1, with INT8 Q/K as the
 * source-analysis page's "Q/K 统一走 INT8"; smoothing Q is optional):
 *   1. Smooth K: subtract the per-channel mean of K over tokens
 *      (SageAttention synthesis page, Smooth K; Algorithm 1 preprocessing).
 *   2. Optionally smooth Q by the per-channel mean of each 128-token block
 *      (Algorithm 1's q_bar_i); the Delta S term q_bar_i . K_j adds the
 *      removed part back to the scores (sage_attn_fwd_smooth_q).
 *      Quantize Q (or Q - q_bar) per group of 128, 32 or 1 tokens and
 *      smoothed K per block of 64 tokens to INT8 with one FP32 scale per
 *      group: scale = amax / 127, code = round-half-even(x / scale)
 *      (deployment-guide page, quantization formula; block sizes b_q = 128,
 *      b_kv = 64 from the detail page's "Optimization Techniques" table; the
 *      finer Q groups are the per-warp / per-thread granularities, below).
 *   3. Quantize V per channel to FP8 E4M3 with one FP32 scale per channel:
 *      scale = amax / 448 (Algorithm 1's psi_V; source-analysis page: V is
 *      transposed, padded and permuted before the per-channel FP8 cast).
 *   4. Tiled online-softmax attention: S = (Q^ K^T) dQ dK sm_scale on INT8
 *      matrix cores, P~ = exp(S - m_running) scaled by 448 and cast to FP8
 *      E4M3, O accumulated in FP32 from FP8 P~ V products, final
 *      O = O / l / 448 * dV (Algorithm 1, the inner loop and the final
 *      rescale; online-softmax update on the source-analysis page).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors), caller-owned, contiguous, and must not alias each other.
 *     The library allocates nothing and keeps no state between calls; the
 *     entry points are re-entrant and thread-safe.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and returns without synchronizing.  Read outputs only after
 *     synchronizing the stream.
 *   - Arguments are validated on the host before anything is launched; the
 *     first violated rule is returned and nothing is enqueued.  Launch
 *     failures return SAGE_ERR_HIP.  Nothing throws across the ABI.
 *   - Layouts: Q, O are [B][H][N][d]; K, V are [B][H_kv][N][d] (the HND
 *     layout, source-analysis page, input checks); query head h reads kv
 *     head h / (H / H_kv) (GQA: H must be a multiple of H_kv).
 *   - d must be 64 or 128 (the pages' kernels cover head dims 64 and 128 and
 *     reject d > 128).  Inputs are fp16 or bf16 (the pages accept only these).
 *   - Size limits (else SAGE_ERR_SHAPE): B*H <= 65535; B*H*N*d < 2^40; and
 *     N rounded up to 128, times d, below 2^32 (one head's codes are
 *     addressed with 32-bit buffer ranges): N < 2^25 at d = 128.
 *   - Non-finite inputs are outside the method's domain (the pages do not
 *     treat NaN/Inf); results for them are unspecified.
 */
#ifndef SAGE_H_
#define SAGE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_ABI_VERSION 10

/* Q tokens per INT8 scale (default), K tokens per INT8 scale. */
#define SAGE_BLKQ 128
#define SAGE_BLKK 64

/*
 * Q scale granularity (`q_group`: consecutive Q tokens per scale).  The
 * SageAttention2 detail page quantizes Q per thread of the matrix-core
 * instruction (Figure 4; Table 6: per-thread is as accurate as per-token
 * and clearly better than per-block); the source-analysis page's
 * quantization module lists per-block, per-warp and per-thread Q scales.
 * Here a wave's matrix cores hold 32 queries, one per lane, so:
 *   SAGE_QGROUP_BLOCK (128): one scale per workgroup's 128 queries;
 *   SAGE_QGROUP_WAVE  (32):  one scale per wave's 32 queries (per-warp);
 *   SAGE_QGROUP_TOKEN (1):   one scale per query, the lane that holds it
 *                            (per-thread).
 * The attention kernel costs the same for all three.
 */
#define SAGE_QGROUP_BLOCK 128
#define SAGE_QGROUP_WAVE 32
#define SAGE_QGROUP_TOKEN 1
/* Keys per online-softmax step; also the padding unit of the FP8 V layout. */
#define SAGE_KV_TILE 128

typedef enum {
  SAGE_OK = 0,
  SAGE_ERR_NULL = 1,      /* a required pointer is NULL                        */
  SAGE_ERR_SHAPE = 2,     /* B, H, H_kv or N <= 0, or sizes overflow           */
  SAGE_ERR_HEADDIM = 3,   /* d not in {64, 128}                                */
  SAGE_ERR_GQA = 4,       /* H % H_kv != 0                                     */
  SAGE_ERR_DTYPE = 5,     /* dtype not SAGE_FP16 / SAGE_BF16                   */
  SAGE_ERR_ARG = 6,       /* sm_scale not finite or <= 0; bad flag or index    */
  SAGE_ERR_WORKSPACE = 7, /* workspace NULL or smaller than required           */
  SAGE_ERR_HIP = 8,       /* a HIP launch or runtime call failed               */
  SAGE_ERR_ALIGN = 9,     /* a pointer is not 16-byte aligned                  */
  SAGE_ERR_SCRATCH = 10   /* the shapes need more than the fixed scratch array */
} sage_status;

typedef enum { SAGE_FP16 = 0, SAGE_BF16 = 1 } sage_dtype;

/* Byte sizes of every buffer the entry points take, for given shapes. */
typedef struct {
  size_t q_i8;      /* int8  [B][H][N][d]                                       */
  size_t q_scale;   /* float [B][H][ceil(N/q_group)]                            */
  size_t k_i8;      /* int8  [B][H_kv][N][d]                                    */
  size_t k_scale;   /* float [B][H_kv][ceil(N/64)]                              */
  size_t k_mean;    /* float [B][H_kv][d]                                       */
  size_t v_f8;      /* uint8 [B][H_kv][ceil(N/128)*128*d], layout below         */
  size_t v_scale;   /* float [B][H_kv][d]                                       */
  size_t o;         /* fp16/bf16 [B][H][N][d]                                   */
  size_t ws_quant_qk; /* workspace bytes sage_quant_qk needs                    */
  size_t ws_quant_v;  /* workspace bytes sage_quant_v needs                     */
  size_t q_mean;    /* float [B][H][ceil(N/128)][d]   (smooth Q only)           */
  size_t ws_smooth_q; /* default workspace of sage_attn_fwd_smooth_q, float
                         [B][H][R][N]: the Delta S rows of R Q blocks (smooth
                         Q only; R in sage_attn_fwd_smooth_q's comment)       */
  size_t v_f4;      /* uint8 [B][H_kv][ceil(N/128)*64*d]  (MXFP4 V codes)       */
  size_t v_e8;      /* uint8 [B][H_kv][ceil(N/128)*512]   (MXFP4 V scales)      */
  size_t ws_quant_qkv; /* workspace bytes sage_quant_qkv needs (qk + v)        */
} sage_sizes;

/*
 * Layout of v_f8 (private to sage_quant_v / sage_attn_fwd, published so
 * callers and tests can decode it).  Per (b, kv head), V is cut into tiles
 * of 128 keys (keys >= N are zero codes).  A tile holds 128*d bytes as
 * 2 key halves (kb = 0, 1: keys kb*64 .. kb*64+63) x d/32 channel blocks
 * (cb) x 2 parts (p) x 64 lanes (L) x 16 bytes (i):
 *     offset = tile*128*d + ((kb*(d/32) + cb)*2 + p)*1024 + L*16 + i
 * holds the code of V[key][chan] with
 *     chan = cb*32 + (L % 32),    s = p*16 + i,    g = L / 32,
 *     key  = tile*128 + kb*64 + (s / 16)*32 + ((s % 16) / 4)*8 + g*4 + (s % 4).
 * (This is the transpose + pad + fixed permutation of the source-analysis
 * page's FP8 V preparation, chosen so one 32-byte row fragment per lane
 * feeds the FP8 matrix core with keys in the order the INT8 matrix core
 * leaves P in registers.)
 */

/* Fill *out with buffer sizes (q_group: see above; else SAGE_ERR_ARG).
 * Host only; touches no device. */
sage_status sage_buffer_sizes(int B, int H, int H_kv, int N, int d, int q_group,
                              sage_sizes* out);

/*
 * Steps 1-2: smooth K and quantize Q and K to INT8.
 *   q [B][H][N][d], k [B][H_kv][N][d] in `dtype` (read only).
 *   q_group: Q tokens per scale, SAGE_QGROUP_BLOCK / _WAVE / _TOKEN (else
 *     SAGE_ERR_ARG); q_scale holds ceil(N / q_group) scales per head, group
 *     i covering tokens i*q_group .. min(N, (i+1)*q_group) - 1.
 *   smooth_k: 1 = subtract the per-channel token mean of K before
 *     quantizing (the mean is the exact sum over all N tokens, divided by N
 *     and rounded to float32); 0 = no smoothing (k_mean is written as 0).
 *   smooth_q: 1 = write q_mean[b][h][i][c] = float32(exact sum / count) over
 *     the valid tokens of 128-token block i (Algorithm 1's q_bar_i, whatever
 *     q_group is) and quantize float32(q) - q_mean of the token's block;
 *     q_mean is then required.  0 = plain Q (q_mean may be NULL).
 *   Outputs: q_i8, q_scale, k_i8, k_scale, k_mean, q_mean (shapes in
 *     sage_sizes).
 *     scale = float32(amax / 127) with IEEE division over the block's valid
 *     tokens; code = RNE(float32(x / scale)) clamped to [-127, 127]; an
 *     all-zero block has scale 0 and codes 0.  Deterministic, bit-exact.
 *   workspace: >= sizes.ws_quant_qk bytes of device memory (scratch; its
 *     contents on entry do not matter).
 */
sage_status sage_quant_qk(const void* q, const void* k, sage_dtype dtype,
                          int B, int H, int H_kv, int N, int d, int q_group, int smooth_k,
                          int smooth_q, int8_t* q_i8, float* q_scale, int8_t* k_i8,
                          float* k_scale, float* k_mean, float* q_mean, void* workspace,
                          size_t ws_bytes, void* stream);

/*
 * Steps 1-3 in one call: sage_quant_qk and sage_quant_v on the same shapes,
 * with the same arguments, outputs and results (bit-identical), in three
 * launches instead of six: one pass reads K and V for the K column sums and
 * the V column maxima, one launch combines them into k_mean and v_scale, and
 * one launch quantizes Q, K and V (each workgroup one Q block, K block or V
 * tile).  workspace: >= sizes.ws_quant_qkv bytes (its contents on entry do
 * not matter).
 */
sage_status sage_quant_qkv(const void* q, const void* k, const void* v, sage_dtype dtype,
                           int B, int H, int H_kv, int N, int d, int q_group, int smooth_k,
                           int smooth_q, int8_t* q_i8, float* q_scale, int8_t* k_i8,
                           float* k_scale, float* k_mean, float* q_mean, uint8_t* v_f8,
                           float* v_scale, void* workspace, size_t ws_bytes, void* stream);

/*
 * Rows of the Delta S term of smooth Q (SageAttention2 detail page,
 * Algorithm 1: S_ij = dequant(Q^_i K^_j^T) + GEMV(q_bar_i, K_j^T); its
 * pipeline figure computes the GEMV before quantization, on the smoothed K):
 *   delta_s[b][h][r][j] = float32( sum_c q_mean[b][h][i0+r][c] *
 *                         (float32(k[b][h/(H/H_kv)][j][c]) - k_mean[b][h/(H/H_kv)][c])
 *                         * float32(sm_scale * log2(e)) )
 * for the 128-token Q blocks i0 .. i0 + nrows - 1 and every key j < N, in
 * the attention kernel's log2 score units.  The products are exact and the
 * sums are FP64 (FP64 matrix cores), rounded once: each entry is the
 * float32 rounding of the exact value up to the FP64 sum's rounding,
 * whatever the summation order.  sage_attn_fwd_smooth_q computes these rows
 * itself; this entry point exposes them for inspection.
 *   k: the original K in `dtype`; k_mean, q_mean: from sage_quant_qk
 *   (k_mean is zeros when K was not smoothed).  0 <= i0, 1 <= nrows,
 *   i0 + nrows <= ceil(N/128), else SAGE_ERR_ARG.
 *   delta_s: float [B][H][nrows][N], caller-owned.
 */
sage_status sage_delta_s(const void* k, sage_dtype dtype, const float* k_mean,
                         const float* q_mean, int B, int H, int H_kv, int N, int d,
                         float sm_scale, int i0, int nrows, float* delta_s, void* stream);

/*
 * Step 3: per-channel FP8 E4M3 quantization of V.
 *   v [B][H_kv][N][d] in `dtype`.
 *   Outputs: v_f8 (layout above) and v_scale [B][H_kv][d]:
 *     scale = float32(amax / 448) over all N tokens of the channel;
 *     code = E4M3_RNE(clamp(float32(v / scale), -448, 448)) (OCP E4M3,
 *     no infinities); zero channel -> scale 0, codes 0.
 *   workspace: >= sizes.ws_quant_v bytes.
 */
sage_status sage_quant_v(const void* v, sage_dtype dtype, int B, int H_kv, int N, int d,
                         uint8_t* v_f8, float* v_scale, void* workspace, size_t ws_bytes,
                         void* stream);

/*
 * Step 4: the attention kernel (Q not smoothed; see sage_attn_fwd_smooth_q).
 *   Inputs are the outputs of sage_quant_qk / sage_quant_v for the same
 *   shapes and q_group.  o [B][H][N][d] is written in `out_dtype` (round to
 *   nearest even).
 *   causal: 1 = key j visible to query i iff j <= i; fully masked key tiles
 *     are skipped.  sm_scale: the softmax scale (> 0, finite), commonly
 *     1/sqrt(d).
 *   Per 128-key tile, in float32 with every step rounded once (Algorithm 1's
 *   inner loop): x = S_int * float32(float32(dQ * dK) * float32(sm_scale *
 *   log2(e))), m = running max of x, P~ = exp2(x - m), code of P~ = E4M3 RNE
 *   of P~ * 448; l sums the unquantized P~.
 */
sage_status sage_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                          const float* k_scale, const uint8_t* v_f8, const float* v_scale,
                          void* o, sage_dtype out_dtype, int B, int H, int H_kv, int N, int d,
                          int q_group, int causal, float sm_scale, void* stream);

/*
 * Step 4 with the row log-sum-exp (the per-row softmax state a forward pass
 * keeps in place of P: the FlashAttention section of the source-analysis
 * page).  Same inputs, output and semantics as sage_attn_fwd, plus
 *   lse: float [B][H][N], required (caller-owned):
 *     lse[b][h][i] = ln sum_j exp(S_ij) + (lse_corr ? lse_corr[b][h][i] : 0)
 *     with S the dequantized scores the softmax used (sm_scale applied, the
 *     causal mask applied, K smoothed if sage_quant_qk smoothed it),
 *     computed as ln(2) * (m + log2 l) from the final running max m and sum l.
 *   lse_corr: float [B][H][N] or NULL.  With smoothed K, pass the output of
 *     sage_lse_correction to get the log-sum-exp of the unsmoothed logits
 *     sm_scale * q . k (smoothing removed sm_scale * q . mean(K) from every
 *     logit of a row; the source-analysis page, smooth_k and LSE correction).
 * Accuracy: each exponent is the float32 rounding of the score in log2
 * units, so lse carries a relative error of a few float32 ulps of |lse|
 * plus the float32 rounding of l's N-term sum.
 */
sage_status sage_attn_fwd_lse(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                              const float* k_scale, const uint8_t* v_f8, const float* v_scale,
                              void* o, sage_dtype out_dtype, float* lse, const float* lse_corr,
                              int B, int H, int H_kv, int N, int d, int q_group, int causal,
                              float sm_scale, void* stream);

/*
 * Step 4 for smoothed Q (sage_quant_qk with smooth_q = 1): the attention of
 * sage_attn_fwd / sage_attn_fwd_lse with the Delta S term of Algorithm 1
 * (SageAttention2 detail page) added to every score before the softmax:
 *   x = float32(S_int * c + g), rounded once, with c as in sage_attn_fwd and
 *   g the value sage_delta_s gives for the query's Q block and the key.
 * The Delta S rows are computed on the fly, a chunk at a time, into
 * `workspace`: each chunk's rows are written by the Delta S pass and consumed
 * by the attention of those query heads and Q blocks, so memory is a bounded
 * number of rows of N floats, never the whole B*H*ceil(N/128)*N table.
 * Results do not depend on the chunking (each row's arithmetic is the same).
 * With causal = 1 the pass may skip keys a Q block cannot attend (those at or
 * past (i + 1) * 128 for block i), about half the work of whole rows; the
 * skipped entries of the workspace keep whatever they held.
 *   k: the original K in k_dtype; k_mean, q_mean: from sage_quant_qk.
 *   lse: float [B][H][N] or NULL (then lse_corr must be NULL, else
 *     SAGE_ERR_ARG); meaning as in sage_attn_fwd_lse.
 *   workspace: device memory of ws_bytes, holding R = ws_bytes / (4*N) Delta S
 *     rows; R >= H/H_kv, else SAGE_ERR_WORKSPACE.  Its contents on entry do
 *     not matter.  With G = H/H_kv query heads per (b, kv head) group and
 *     M = ceil(N/128) Q blocks, a chunk is
 *       1. whole groups with all their Q blocks, g of them, when the largest
 *          multiple of 8 with g*G*M <= R is >= 8 and g*G*M is no less than
 *          the rows of a case-2 chunk (each (b, kv head) then stays on one
 *          XCD, and each Delta S pass reads the K of its groups once); g is
 *          evened out over the chunks;
 *       2. else, when R >= B*H, all B*H_kv groups with r = R / (B*H) Q
 *          blocks each;
 *       3. else one group with r = R / G Q blocks;
 *     r evened out over the chunks and rounded up to a multiple of 16 where
 *     that still fits.
 *   sizes.ws_smooth_q is the default: every head's rows of
 *     min(M, max(32, 16*ceil(ceil(2048/(B*H))/16))) Q blocks, which grows
 *     linearly with N.
 */
sage_status sage_attn_fwd_smooth_q(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                   const float* k_scale, const uint8_t* v_f8,
                                   const float* v_scale, const void* k, sage_dtype k_dtype,
                                   const float* k_mean, const float* q_mean, void* o,
                                   sage_dtype out_dtype, float* lse, const float* lse_corr,
                                   int B, int H, int H_kv, int N, int d, int q_group, int causal,
                                   float sm_scale, void* workspace, size_t ws_bytes,
                                   void* stream);

/*
 * corr[b][h][i] = sm_scale * sum_c q[b][h][i][c] * k_mean[b][h / (H/H_kv)][c]
 * in fp32 (fixed summation order), for sage_attn_fwd_lse.
 *   q [B][H][N][d] in `dtype` (the original, unquantized Q); k_mean
 *   [B][H_kv][d] from sage_quant_qk; corr float [B][H][N], caller-owned.
 */
sage_status sage_lse_correction(const void* q, sage_dtype dtype, const float* k_mean, int B, int H,
                                int H_kv, int N, int d, float sm_scale, float* corr,
                                void* stream);

/*
 * MXFP4 P V (the SageAttention3 synthesis page names MXFP4, the OCP
 * microscaling format, as the FP4 format of MI350-class GPUs): V and P~ in
 * E2M1 with one E8M0 scale 2^e per 32 consecutive keys, on the FP4 matrix
 * cores at twice the FP8 rate.  The format: e = floor(log2 amax) - 2
 * (clamped to [-127, 127]; an all-zero block takes -127), code =
 * RNE(x / 2^e) saturated to +-6.
 *
 * Step 3 in MXFP4: v [B][H_kv][N][d] in `dtype`.
 *   v_f4: per (b, kv head), 128-key tiles of 64*d bytes: 2 key halves (h:
 *     keys h*64 ..) x d/32 channel blocks (cb) x 64 lanes (L) x 16 bytes;
 *       offset = tile*64*d + ((h*(d/32) + cb)*64 + L)*16 + p/2
 *     holds in nibble p%2 (low first) the code of V[key][chan], chan = cb*32
 *     + L%32, key = tile*128 + h*64 + (L/32)*32 + 8*((p%16)/4) + 4*(p/16) +
 *     p%4 (the key order of P in the kernel's registers); keys >= N are 0.
 *   v_e8: per (b, kv head), 512 bytes per tile: byte (h*64 + L)*4 + cb is
 *     e + 127 for the 32 keys of chunk (tile, h, cb, L) (bytes cb >= d/32
 *     unused).  Deterministic, bit-exact.
 */
sage_status sage_quant_v_mxfp4(const void* v, sage_dtype dtype, int B, int H_kv, int N, int d,
                               uint8_t* v_f4, uint8_t* v_e8, void* stream);

/*
 * Step 4 with MXFP4 P V: as sage_attn_fwd_lse (lse may be NULL here), with V
 * from sage_quant_v_mxfp4 and, per tile and row, P~ quantized in blocks of
 * 32 consecutive keys: e = floor(log2 max P~) - 2, codes RNE(P~ / 2^e); l
 * sums the unquantized P~.  No Delta S (smoothed Q is not taken here).
 */
sage_status sage_attn_fwd_mxfp4(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                const float* k_scale, const uint8_t* v_f4, const uint8_t* v_e8,
                                void* o, sage_dtype out_dtype, float* lse, const float* lse_corr,
                                int B, int H, int H_kv, int N, int d, int q_group, int causal,
                                float sm_scale, void* stream);

/*
 * Diagnostic: the exact int32 dot products sum_c q_i8[b][h][i][c] *
 * k_i8[b][h/(H/H_kv)][j][c] of one query head, computed by the same INT8
 * matrix-core tile routine and K loader the attention kernel uses.
 *   s_out: int32 [N][N] (row = query i, column = key j), caller-owned.
 *   b in [0, B), h in [0, H), else SAGE_ERR_ARG.
 */
sage_status sage_qk_int32(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int H_kv,
                          int N, int d, int b, int h, int32_t* s_out, void* stream);

/*
 * Diagnostic for the roofline (not a step of the method): the dense MFMA rate
 * the device sustains and its shader clock meanwhile, against which the
 * attention kernel's fraction of peak can be stated besides the published
 * 2.4 GHz figure (the SageAttention2 detail page rates its kernels as a
 * fraction of the matrix cores' peak).  Each of nwg workgroups of 4 waves
 * issues, per wave, 4 * iters independent MFMAs back to back on register
 * operands whose bytes are all 1 (kind 0: v_mfma_i32_32x32x32_i8, the
 * instruction of S = Q K^T, 65536 ops each; kind 1: the scaled FP8 32x32x64
 * MFMA of P V with unit scales, operands E4M3 1.0, 131072 flops each).
 *   clocks: int64 [nwg*4][2], caller-owned device memory: per wave, the
 *     shader clocks (clock64) and the constant-rate clocks (wall_clock64) its
 *     loop took.
 *   sink: uint32 [nwg*256], caller-owned device memory: per lane, the sum of
 *     its 64 accumulator elements, 64 * 32 * iters (kind 0) or 64 * 64 * iters
 *     (kind 1), so a caller can check that every MFMA ran.
 *   wall_khz: host int, receives the constant-rate clock's frequency (kHz) of
 *     the current device.
 *   kind not 0 or 1, iters outside [1, 2^18] or nwg outside [1, 65536]:
 *   SAGE_ERR_ARG; clocks or sink not 16-byte aligned: SAGE_ERR_ALIGN; nothing
 *   launched either way.
 */
sage_status sage_mfma_peak(int kind, int iters, int nwg, int64_t* clocks, uint32_t* sink,
                           int* wall_khz, void* stream);

/*
 * sage_quant_qk without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments, outputs and results are those of
 * sage_quant_qk (bit-identical); the column-statistics scratch is instead a
 * fixed device array of SAGE_SCRATCH_BYTES inside the library, one per GPU,
 * held until the process ends.
 *   Limit: with smooth_k = 1 the shapes need sage_buffer_sizes().ws_quant_qk
 *     <= SAGE_SCRATCH_BYTES (B * H_kv * ceil(N/256) * d * 8 bytes), else
 *     SAGE_ERR_SCRATCH and nothing is launched.  smooth_k = 0 needs no scratch.
 *   The first call on a device looks the array's address up (no allocation);
 *     it runs on the device of `stream` (the current device for NULL).
 *   Every call on one GPU shares that GPU's array: calls that overlap in time
 *     on one GPU (other streams, other threads) race.  Calls serialized on a
 *     stream do not: each call writes every scratch byte it reads.
 */
#define SAGE_SCRATCH_BYTES (16u << 20)
sage_status sage_quant_qk_noalloc(const void* q, const void* k, sage_dtype dtype,
                                  int B, int H, int H_kv, int N, int d, int q_group,
                                  int smooth_k, int smooth_q, int8_t* q_i8, float* q_scale,
                                  int8_t* k_i8, float* k_scale, float* k_mean, float* q_mean,
                                  void* stream);

/* Static description of a status code. */
const char* sage_status_str(sage_status s);

/* SAGE_ABI_VERSION of the built library. */
int sage_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_H_ */
