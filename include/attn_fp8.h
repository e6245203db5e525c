/* attn_fp8.h -- C ABI of the MI355X (gfx950) FP8 fused attention forward library.
 *
 * The method is the fused running-softmax attention loop described on the page
 * "Fused attention kernel" (wikillm.com), sections "Overview" and
 * "Implementation sketch", fed by the 8-bit pre-processing of its section
 * "Variants / 8-bit forward pass (FP8, Hopper)": incoherent processing (Q and
 * K rotated by a random +-1 diagonal times a Hadamard matrix, an orthogonal
 * transform that leaves Q K^T unchanged) and e4m3 quantisation with a scale
 * chosen per block, separately for Q, K and V.  The problem page "FP8 attention that keeps FlashAttention-3 throughput at
 * BF16-level accuracy", section "How it gets verified", fixes the types: Q, K, V
 * in E4M3, FP32 softmax statistics, BF16 output; and measures the FP8 error
 * against the BF16 forward pass, exported here as attn_bf16_fwd.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers, allocated and owned by the caller;
 *     the library allocates no device memory and keeps no per-call state.
 *   - Layout is contiguous row-major [B][H][N][D] for Q, K, V, their codes and
 *     O; [B][H][N] for LSE; [B][H][ceil(N / scale_block)] for block descales.
 *   - Tensor pointers must be 16-byte aligned; descale and LSE pointers 4-byte.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it and the call returns without synchronising the host; no host copy
 *     of scales or sizes is made on the device path, so calls can be captured
 *     in a HIP graph.
 *   - Supported: D in {64, 128}; scale_block in {64, 128}; B, H, N >= 1;
 *     B * H * ceil(N / 128) < 2^31; N * D < 2^30.  Only gfx950 devices are
 *     supported.
 *   - Return value: ATTN_OK, or an attn_status error.  On ATTN_EINVAL and
 *     ATTN_EUNSUPPORTED nothing is launched and no output is written.
 *     attn_fp8_last_error() then describes the error (per calling thread).
 *   - Inputs must be finite.  Calls that overlap on one stream are ordered by
 *     the stream; outputs must not alias inputs.
 */
#ifndef ATTN_FP8_H
#define ATTN_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = 1,       /* bad argument (null/misaligned pointer, unsupported size) */
  ATTN_EUNSUPPORTED = 2, /* no gfx950 device is current */
  ATTN_EHIP = 3          /* a HIP runtime call or kernel launch failed */
} attn_status;

/* quantize_qkv_fp8 -- rotate + per-block scale + e4m3 encode of Q, K and V in
 * one launch ("Fused attention kernel", 8-bit forward pass: block quantisation
 * and incoherent processing; fused into one launch as in FLAMIA, 4.3 Ablation
 * Study).  V's block scales are powers of two (the attention applies them
 * exactly inside the matrix core); Q's and K's map the block maximum to 448.
 *   q, k, v        in : float32 [B][H][N][D].
 *   scale_block       : tokens per scale block (64 or 128); a block is
 *                       scale_block consecutive tokens of one (batch, head)
 *                       times all D channels; the last block may be short.
 *   hadamard          : nonzero -> Q and K rows become x * diag(sigma) * H_D
 *                       (unnormalised Sylvester Hadamard, butterfly stages in
 *                       ascending order, float32); V is never rotated.
 *   seed              : 64-bit seed of sigma: one Philox4x32-10 block with
 *                       counter 0 and key (seed low word, seed high word);
 *                       sigma_c = -1 when bit c of the 128-bit output is set.
 *   q8, k8, v8    out : e4m3 codes [B][H][N][D], code = e4m3_rne(clamp(y * inv, +-448))
 *   q/k_descale   out : float32 [B][H][ceil(N/scale_block)], descale = amax/448
 *                       (inv = 448/amax; 1 for an all-zero block).  A nonzero
 *                       block amax below 448 / FLT_MAX (about 1.3e-36) makes
 *                       inv overflow and is outside the contract of this rule
 *                       (the power-of-two rule of ATTN_FP8_MX covers it).
 *   v_descale     out : float32 [B][H][ceil(N/scale_block)], the smallest power
 *                       of two 2^e with amax <= 448 * 2^e (e clamped to
 *                       [-127, 127]; 2^0 for an all-zero block): an E8M0
 *                       scale, inv = 2^-e exactly, no code saturates.
 */
int quantize_qkv_fp8(const float* q, const float* k, const float* v,
                     int B, int H, int N, int D, int scale_block, int hadamard, uint64_t seed,
                     uint8_t* q8, uint8_t* k8, uint8_t* v8,
                     float* q_descale, float* k_descale, float* v_descale, void* stream);

/* Option flags of the *_opts entry points. */
#define ATTN_FP8_EXP2_SCHRAUDOLPH 1u  /* attn_fp8_fwd_opts only; see below */
/* ATTN_FP8_MX -- microscaling form of the block scales ("FLAMIA", 2 Background:
 * blocks of low-bit codes sharing one scale, which block-scaled matrix units
 * apply during accumulation).
 *   quantize_qkv_fp8_opts: each block's descale is the smallest power of two
 *     2^e with amax <= 448 * 2^e (e clamped to [-127, 127]; 2^0 for an
 *     all-zero block), i.e. an E8M0 scale; code = e4m3_rne(y * 2^-e), which
 *     never saturates.  Output layout as for quantize_qkv_fp8 (float32 2^e).
 *   attn_fp8_fwd_opts: the descales must be powers of two (as written by
 *     quantize_qkv_fp8_opts with ATTN_FP8_MX); their exponents are handed to
 *     the scaled FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4), which applies
 *     them to Q, K and V inside the matrix core; P enters with scale 2^0.
 *     Descales that are not powers of two give wrong results (only their
 *     exponent fields are read). */
#define ATTN_FP8_MX 2u
/* ATTN_FP8_MX32 -- the MX scales at their own granularity ("FLAMIA", 2
 * Background: MX formats share one E8M0 scale per block of 32 elements; 4.2
 * Numerical Accuracy evaluates per-32-element scaling): one power-of-two
 * scale per (scale_block tokens x 32 channels) of Q, K and V, applied by the
 * scaled FP8 MFMA per lane (the 32 channels one lane feeds to one product
 * share a scale).  Descales are [B][H][ceil(N / scale_block)][D / 32]
 * (float32 2^e, the smallest with the group's amax <= 448 * 2^e, e clamped to
 * [-127, 127], 2^0 for an all-zero group), written by quantize_qkv_fp8_opts
 * and read by attn_fp8_fwd_opts with this flag (alone or with
 * ATTN_FP8_EXP2_SCHRAUDOLPH; ATTN_FP8_MX is implied).  Dense layout only. */
#define ATTN_FP8_MX32 8u

/* quantize_qkv_fp8_opts -- quantize_qkv_fp8 with option flags (quantize_qkv_fp8
 * is this call with flags = 0).  flags: ATTN_FP8_MX, ATTN_FP8_MX32 or 0
 * (with both set, ATTN_FP8_MX32 applies); any other bit -> ATTN_EINVAL. */
int quantize_qkv_fp8_opts(const float* q, const float* k, const float* v,
                          int B, int H, int N, int D, int scale_block, int hadamard, uint64_t seed,
                          unsigned flags, uint8_t* q8, uint8_t* k8, uint8_t* v8,
                          float* q_descale, float* k_descale, float* v_descale, void* stream);

/* attn_fp8_fwd -- FP8 fused attention forward ("Fused attention kernel",
 * Implementation sketch: running max and sum, exp(old max - new max) rescale,
 * every key block scored; logsumexp output).
 *   q8, k8, v8, *_descale in : output of quantize_qkv_fp8 with the same
 *                       scale_block and hadamard flag (hadamard nonzero folds
 *                       the 1/D of the unnormalised rotation into the score
 *                       scale).  v_descale must hold powers of two: only
 *                       their exponent fields are read, as the E8M0 scale of
 *                       the P V product (v_mfma_scale_f32_32x32x64_f8f6f4).
 *   causal            : nonzero -> query i sees keys j <= i.
 *   o_bf16        out : bf16 bit patterns [B][H][N][D],
 *                       O = softmax(Q K^T / sqrt(D)) V of the dequantised inputs.
 *   lse           out : float32 [B][H][N], natural log of sum_j exp(q_i.k_j / sqrt(D)).
 * Arithmetic: e4m3 x e4m3 products with FP32 accumulation, FP32 statistics,
 * P re-quantised to e4m3 on chip (P = 2^(t - m) <= 2^8.8 ~ 445.7, inside
 * e4m3's range, against a per-row reference m in log2 units, which moves
 * only when a key block would exceed that, and then to 2 below that block's
 * maximum: the key that moved it gets P = 4).
 */
int attn_fp8_fwd(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                 const float* q_descale, const float* k_descale, const float* v_descale,
                 int B, int H, int N, int D, int scale_block, int hadamard, int causal,
                 uint16_t* o_bf16, float* lse, void* stream);

/* attn_fp8_fwd_opts -- attn_fp8_fwd with option flags (attn_fp8_fwd is this
 * call with flags = 0).
 *   flags             : any combination of ATTN_FP8_MX or ATTN_FP8_MX32
 *                       (above) and ATTN_FP8_EXP2_SCHRAUDOLPH.
 *                       ATTN_FP8_EXP2_SCHRAUDOLPH -> the probabilities use
 *                       Schraudolph's bit-level exponential (N. N. Schraudolph,
 *                       "A fast, compact approximation of the exponential
 *                       function", Neural Computation 11(4), 1999) in base 2:
 *                       the float32 bits of 2^x are floor(2^23 (x + 127 -
 *                       60801/2^20)), saturated at 0 below; relative error
 *                       -3.9% .. +2.0% per probability.  FLAMIA evaluates it
 *                       for inference ("FLAMIA", 4.4 Bit-Level Exponentials at
 *                       Inference).  The row sum uses the same approximated
 *                       values; the O rescale factor stays exact.
 *                       Any other bit -> ATTN_EINVAL.
 */
int attn_fp8_fwd_opts(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                      const float* q_descale, const float* k_descale, const float* v_descale,
                      int B, int H, int N, int D, int scale_block, int hadamard, int causal,
                      unsigned flags, uint16_t* o_bf16, float* lse, void* stream);

/* attn_bf16_fwd -- the same loop on BF16 inputs (BF16 products, FP32
 * accumulation and statistics, P in BF16), no rotation or quantisation: the
 * 16-bit yardstick of the problem statement ("What is asked").
 *   q, k, v      in : bf16 bit patterns [B][H][N][D].
 *   o_bf16, lse out : as for attn_fp8_fwd.
 */
int attn_bf16_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  int B, int H, int N, int D, int causal,
                  uint16_t* o_bf16, float* lse, void* stream);

/* ---- Packed variable-length documents ----------------------------------
 * "FLAMIA ..." (arXiv 2611.03344, Abstract and 4.1 Performance on Packed
 * Documents): documents of different lengths are packed one after another
 * with no padding and no repacking, every scale is local to one document, and
 * attention runs inside each document.  4.3 Ablation Study: causal work runs
 * longest first.  F. System Integration: scales and work lists stay on the
 * GPU (no host synchronisation; graph capture works).
 *
 * Layout: Q, K, V, their codes and O are [H][T][D] (heads outermost, the T
 * packed tokens of every head in document order); LSE is [H][T].
 * cu_seqlens: DEVICE int32 [ndoc + 1], document d = tokens cu[d] .. cu[d+1]-1;
 * it must start at 0, never decrease and end at T (empty documents are
 * allowed).  The host never reads it.
 * Scale blocks are document-local: the blocks of document d are its tokens in
 * groups of scale_block from its first token (the last may be short).  The
 * descale of block b of document d is entry cu[d] / scale_block + d + b of a
 * head's row: descales are [H][T / scale_block + ndoc] (integer division);
 * entries that belong to no block are not written.
 * Sizes: H, T, ndoc >= 1; T <= 2^20; ndoc <= 2^24; D, scale_block as above;
 * H * (T / scale_block + ndoc) < 2^31; H * ((T + 127 ndoc) / 128) < 2^31.
 */

/* Option flag of attn_fp8_fwd_varlen: schedule the work items in document
 * order (documents ascending, query tiles ascending) instead of longest
 * first.  It changes the order of the workgroups only, never a result: the
 * baseline of FLAMIA's longest-first ablation. */
#define ATTN_FP8_NATURAL_ORDER 4u

/* quantize_qkv_fp8_varlen -- quantize_qkv_fp8_opts on packed documents.
 *   q, k, v      in : float32 [H][T][D].
 *   cu_seqlens   in : device int32 [ndoc + 1] (see above).
 *   flags           : ATTN_FP8_MX or 0.
 *   q8, k8, v8  out : e4m3 codes [H][T][D] (the rule of quantize_qkv_fp8 per block).
 *   *_descale   out : float32 [H][T / scale_block + ndoc], slots as above.
 * cu_seqlens contents that break the rule above give unspecified codes and
 * descales; every access still stays inside the buffers (entries are clamped
 * to [0, T]).
 */
int quantize_qkv_fp8_varlen(const float* q, const float* k, const float* v,
                            const int32_t* cu_seqlens, int ndoc, int H, int T, int D,
                            int scale_block, int hadamard, uint64_t seed, unsigned flags,
                            uint8_t* q8, uint8_t* k8, uint8_t* v8,
                            float* q_descale, float* k_descale, float* v_descale, void* stream);

/* attn_fp8_varlen_workspace_bytes -- bytes of device workspace that
 * attn_fp8_fwd_varlen needs for T packed tokens in ndoc documents:
 * 16 + 8 * ((T + 127 ndoc) / 128).  0 for T < 1 or ndoc < 1. */
size_t attn_fp8_varlen_workspace_bytes(int T, int ndoc);

/* attn_fp8_fwd_varlen -- attn_fp8_fwd_opts on packed documents.  Two
 * launches on `stream`: one workgroup writes the work list (every (document,
 * query tile of 128) item, longest first: documents in non-increasing tile
 * count, each document's tiles together and from the last to the first, the
 * last seeing the most keys under a causal mask) into the workspace; then
 * the attention runs one workgroup per (item, head) in that order, the heads
 * of one item next to each other.
 *   q8 .. v_descale in : output of quantize_qkv_fp8_varlen with the same
 *                        cu_seqlens, scale_block and hadamard flag.
 *   causal             : nonzero -> query i of a document sees the keys of
 *                        its document up to position i.
 *   flags              : any combination of ATTN_FP8_EXP2_SCHRAUDOLPH,
 *                        ATTN_FP8_MX and ATTN_FP8_NATURAL_ORDER.
 *   workspace          : device memory, 16-byte aligned, at least
 *                        attn_fp8_varlen_workspace_bytes(T, ndoc) bytes,
 *                        owned by the caller; it holds the work list after
 *                        the call: int32 item count, int32 status (0 = ok,
 *                        1 = cu_seqlens broke the rule above), 8 unused bytes,
 *                        then (document, query tile) int32 pairs in launch
 *                        order.  Calls that share a workspace must not overlap.
 *   o_bf16, lse    out : [H][T][D] bf16 bit patterns and [H][T] float32; rows
 *                        of empty documents do not exist; with status 1 nothing
 *                        is written.
 */
int attn_fp8_fwd_varlen(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                        const float* q_descale, const float* k_descale, const float* v_descale,
                        const int32_t* cu_seqlens, int ndoc, int H, int T, int D,
                        int scale_block, int hadamard, int causal, unsigned flags,
                        void* workspace, size_t workspace_bytes,
                        uint16_t* o_bf16, float* lse, void* stream);

/* ---- Decode over an FP8 K/V cache ----------------------------------------
 * "FP8 attention that keeps FlashAttention-3 throughput at BF16-level
 * accuracy", Realistic applications: K and V stored in FP8 relieve the
 * bandwidth of the KV cache.  A decode step attends the Sq newest tokens of
 * each sequence to its cached keys; the cache moves one byte per element.
 *
 * Layout: cache codes k8, v8 [B][Hkv][Ncap][D] and descales
 * [B][Hkv][ceil(Ncap / scale_block)] as quantize_qkv_fp8 writes them for the
 * sequence (block b = tokens b*scale_block ..); sequence b uses its first
 * L_b = seqlens[b] tokens, the Sq new ones included.  Queries q8
 * [B][Hq][Sq][D] with q_descale [B][Hq] (quantize_qkv_fp8 on the new tokens:
 * one block, Sq <= scale_block; rotated with the cache's seed when hadamard
 * is set).  Query head h reads K/V head h / (Hq / Hkv) (grouped queries).
 * Query i of sequence b sits at position L_b - Sq + i; causal: it sees keys
 * up to that position.  Outputs o_bf16 [B][Hq][Sq][D], lse [B][Hq][Sq].
 *
 * The keys are cut into ranges; each range runs the loop of attn_fp8_fwd
 * (64-key tiles, lazy reference, P in e4m3, V's power-of-two block scale
 * inside the matrix core) and the ranges of one (sequence, K/V head) merge by
 * their log-sum-exp.  Two schedules:
 *   split = 0, B <= 512 (balanced shares): the 64-key tiles of every
 *     (sequence, K/V head), in the order sequence, K/V head, tile, are cut
 *     into W equal shares, one per wave, W = min(2048, B * Hkv *
 *     ceil(Ncap / 64)) rounded up to a multiple of 4: every wave streams the
 *     same number of tiles whatever the mix of lengths (the lengths are read
 *     on the device); a share that spans several sequences or heads makes one
 *     range per piece.
 *   split > 0 (or B > 512): fixed ranges of `split` keys per wave (a multiple
 *     of 64; for split = 0 the library's choice, attn_fp8_decode_split).
 * Sizes: (Hq / Hkv) * Sq <= 32 (so Sq <= scale_block), Ncap * D < 2^30,
 * B * Hkv <= 65535; fixed ranges: ceil(Ncap / (4 * split')) <= 65535.
 * seqlens: device int32 [B] with Sq <= L_b <= Ncap; other values give
 * unspecified rows of that sequence (L_b is clamped to [0, Ncap], so every
 * access stays in bounds).
 */

/* Keys per range of the fixed-range schedule for `split`, or 0 when the
 * balanced shares are used (split = 0 and B <= 512).  For split = 0 and
 * B > 512: the largest power of two in [64, 1024] that still gives 1024
 * workgroups of four ranges over Ncap. */
int attn_fp8_decode_split(int B, int Hkv, int Ncap, int split);

/* Bytes of device workspace attn_fp8_decode needs (the per-range partials):
 * balanced shares: 4 * (W + B * Hkv) * (Hq / Hkv) * Sq * (D + 2), W as above;
 * fixed ranges: 4 * B * Hkv * ceil(Ncap / (4 * split')) * (Hq / Hkv) * Sq * (D + 2),
 * split' = attn_fp8_decode_split(B, Hkv, Ncap, split); 0 for invalid sizes. */
size_t attn_fp8_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Ncap, int D, int split);

/* attn_fp8_decode -- FP8 attention of Sq new queries per sequence against an
 * FP8 K/V cache.  Two launches on `stream`: the range kernel (balanced
 * shares: W / 4 workgroups of four independent waves; fixed ranges: one
 * workgroup per 4 ranges of one (sequence, K/V head), grid (B * Hkv,
 * ranges / 4)) and the merge.
 *   workspace : device memory, 16-byte aligned, caller-owned, at least
 *               attn_fp8_decode_workspace_bytes(...) bytes; calls sharing a
 *               workspace must not overlap.
 * Other arguments as above; validation as for attn_fp8_fwd. */
int attn_fp8_decode(const uint8_t* q8, const float* q_descale,
                    const uint8_t* k8, const uint8_t* v8,
                    const float* k_descale, const float* v_descale,
                    const int32_t* seqlens, int B, int Hq, int Hkv, int Sq, int Ncap, int D,
                    int scale_block, int hadamard, int causal, int split,
                    void* workspace, size_t workspace_bytes,
                    uint16_t* o_bf16, float* lse, void* stream);

/* attn_fp8_decode_noalloc -- attn_fp8_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It takes no workspace: the per-range
 * partials live in a scratch array of ATTN_FP8_DECODE_NOALLOC_MAX_BYTES that
 * the library holds on every GPU it runs on until the process ends (a
 * file-scope __device__ array; no hipMalloc, hipFree or other allocation
 * happens in the call).  Sizes whose partials
 * (attn_fp8_decode_workspace_bytes(...)) exceed that limit -> ATTN_EINVAL,
 * nothing launched.  Every call on one GPU shares its array and leaves its
 * partials there (nothing in it needs clearing: each call writes every
 * partial it reads): calls that overlap on one GPU, on different streams or
 * threads, race and must not be made.  Other arguments, outputs and errors
 * as for attn_fp8_decode; the result is bitwise the same. */
#define ATTN_FP8_DECODE_NOALLOC_MAX_BYTES ((size_t)16 << 20)
int attn_fp8_decode_noalloc(const uint8_t* q8, const float* q_descale,
                            const uint8_t* k8, const uint8_t* v8,
                            const float* k_descale, const float* v_descale,
                            const int32_t* seqlens, int B, int Hq, int Hkv, int Sq, int Ncap, int D,
                            int scale_block, int hadamard, int causal, int split,
                            uint16_t* o_bf16, float* lse, void* stream);

/* Message for the last non-OK status returned on the calling thread ("" if none).
 * The string is owned by the library and valid until the next call on that thread. */
const char* attn_fp8_last_error(void);

/* ABI version of this header (incremented on incompatible changes). */
int attn_fp8_abi_version(void);

#define ATTN_FP8_ABI_VERSION 5

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FP8_H */
