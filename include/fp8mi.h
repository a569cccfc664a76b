/*
 * fp8mi.h — per-tensor-scaled FP8 matrix multiply with delayed scaling,
 * native to AMD Instinct MI355X (gfx950, CDNA4).  C ABI.
 *
 * The operations follow these pages:
 *   [TE]  "4.2 Hopper I — Transformer Engine·FP8" (aegloslab.com), §4.2.3–§4.2.6,
 *         §4.2.8 (formats, amax-based per-tensor scale, delayed scaling from an
 *         amax history, FP8 GEMM with FP32 accumulation and x(1/scale) restore,
 *         the HYBRID recipe with history length 16 and the "max" rule, OCP FP8).
 *   [FMT] "FP8 and low-precision formats" (aiunderstanding.org), "Deep dive" and
 *         "Technical insight" (E4M3/E5M2 bit splits, per-tensor or per-block
 *         scale factors, high-precision partial sums).
 *   [DG]  "#fp8" tag page (discuss.pytorch.kr), DeepGEMM entry (MoE grouped
 *         GEMM, two-level "promotion" of FP8 partial sums).
 *   [DG-talk] the same page, the discussion of FP8 LLM training ("automatic
 *         scaling" of gradients during the all-reduce); [FMT] use cases (E5M2
 *         for gradient communication).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named as device pointers must point to memory of the GPU that is
 *   current on the calling thread; all scalars (sizes, formats, flags) are host
 *   values.  Passing host memory where device memory is required is undefined.
 * - The caller allocates and owns every buffer.  No entry point allocates,
 *   frees or keeps device memory.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is
 *   asynchronous: results are valid after the caller synchronises the stream.
 *   Nothing synchronises the host.
 * - Argument errors are detected on the host before anything is launched and
 *   returned as a negative fp8mi_status; nothing is enqueued in that case.
 *   A failed launch returns FP8MI_ERR_LAUNCH.  Device faults surface at the
 *   caller's next synchronisation.  Numeric anomalies (NaN/Inf/zero amax) are
 *   not errors: see fp8_amax_update.  Nothing is thrown across the ABI.
 * - FP8 data is uint8 codes in the OCP 8-bit floating-point formats:
 *   E4M3 (bias 7, no Inf, NaN = S.1111.111, max 448) and E5M2 (bias 15,
 *   IEEE-like Inf/NaN, max 57344).
 * - Row-major everywhere; "[R x C]" means R rows of C contiguous elements.
 */
#ifndef FP8MI_H
#define FP8MI_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define FP8MI_API __attribute__((visibility("default")))
#else
#define FP8MI_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FP8MI_E4M3 = 0, FP8MI_E5M2 = 1 } fp8mi_format;
typedef enum { FP8MI_F32 = 0, FP8MI_BF16 = 1 } fp8mi_dtype;

/*
 * How the GEMMs contract FP8 operands (see fp8_gemm):
 *   FP8MI_ACCUM_EXACT     every product exact, sums in fp32: meets
 *                         |C - C_exact| <= 1e-5 * sum_k |a_k b_k| * sinv_a * sinv_b
 *                         for every input (FP8 widened exactly to bf16 in
 *                         registers, bf16 matrix cores, fp32 accumulators).
 *   FP8MI_ACCUM_MFMA_FP8  the native FP8 matrix-core instruction, twice the
 *                         peak rate.  On MI355X it sums each run of 8
 *                         consecutive K products in fixed point whose last bit
 *                         is 13 bits below the run's largest product
 *                         (truncating toward zero), then adds the runs in fp32.
 */
typedef enum { FP8MI_ACCUM_EXACT = 0, FP8MI_ACCUM_MFMA_FP8 = 1 } fp8mi_accum;

typedef enum {
  FP8MI_OK = 0,
  FP8MI_ERR_NULL = -1,    /* a required pointer is NULL                          */
  FP8MI_ERR_SHAPE = -2,   /* a size is negative, too large or inconsistent       */
  FP8MI_ERR_ALIGN = -3,   /* a pointer or leading size breaks the alignment rule */
  FP8MI_ERR_FORMAT = -4,  /* unknown fp8mi_format                                */
  FP8MI_ERR_DTYPE = -5,   /* unknown fp8mi_dtype                                 */
  FP8MI_ERR_LAUNCH = -6,  /* the HIP runtime rejected a kernel launch            */
  FP8MI_ERR_DEVICE = -7,  /* no usable gfx950 device is current                  */
  FP8MI_ERR_ACCUM = -8    /* unknown fp8mi_accum                                 */
} fp8mi_status;

/* Human-readable name of a status code (static storage; never NULL). */
FP8MI_API const char* fp8mi_status_string(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
FP8MI_API int fp8mi_version(void);

/*
 * fp8_quantize — fused amax reduction + scaled saturating cast ([TE] §4.2.4).
 *
 *   p      = fp32(x[i] * scale[0])                  (one fp32 multiply, RNE)
 *   code   = round_to_fp8(p): nearest, ties to even mantissa; |p| > max and
 *            +-Inf saturate to +-max; NaN -> sign|0x7F; sign always kept
 *   amax   = max_i |x[i]| of the UNSCALED input, taken as the largest
 *            (bits & 0x7FFFFFFF) — exact and order-free; NaN/Inf propagate
 *   sat    = #{ i : |p| > max }  (Inf counts, NaN does not)
 *
 * One read of x produces every output ([TE] §4.2.4: delayed scaling exists so
 * that the tensor is traversed once).
 *
 * x        device, [rows x cols] of xtype (fp32 or bf16 bit patterns); 16-B aligned.
 * scale    device, 1 fp32: the scale to apply (normally the delayed scale kept
 *          by fp8_amax_update).  May be NULL only when q and q_t are both NULL.
 * q        device, [rows x cols] uint8 codes, or NULL; 16-B aligned.
 * q_t      device, [cols x rows] uint8 codes of the transpose, or NULL
 *          ("cast-transpose": the K-contiguous layout fp8_gemm wants for an
 *          operand stored [K x N]).  When non-NULL, rows and cols must be
 *          multiples of 16.
 * amax     device, 1 fp32, overwritten (not accumulated), or NULL.
 * sat      device, 1 uint64, overwritten, or NULL.
 * workspace  device scratch owned by the caller, 16-B aligned, or NULL.  With
 *          one, each workgroup writes its partial amax / count into it and a
 *          small second kernel reduces them (no contended atomics); up to
 *          workspace_bytes / 16 workgroups are used, so FP8MI_QUANTIZE_WORKSPACE_BYTES
 *          lets the grid cover the device (the cast-transpose keeps up to 8
 *          workgroups per compute unit resident).  Contents on entry do not matter;
 *          two calls in flight at once must not share one workspace.  Without
 *          one, the outputs are cleared and then updated with atomics.
 * At least one of q, q_t, amax must be non-NULL.  rows*cols may be 0 (then
 * amax = 0 and sat = 0).
 */
#define FP8MI_QUANTIZE_WORKSPACE_BYTES 65536

FP8MI_API int fp8_quantize(const void* x, int xtype, int64_t rows, int64_t cols, int fmt,
                 const float* scale, uint8_t* q, uint8_t* q_t, float* amax,
                 unsigned long long* sat, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8_amax_update — delayed-scaling history step ([TE] §4.2.4 "delayed
 * scaling", §4.2.6 recipe: amax_history_len, amax_compute_algo = "max").
 *
 *   h = *head;  history[h] = *amax;  *head = (h + 1) % history_len;
 *   m = max(history[0 .. history_len-1])   (over fp32 bit patterns, so NaN > Inf)
 *   if (0 < m < Inf and s = fp32(MAX / m) is finite):
 *        *scale = s;  *scale_inv = fp32(1 / s)      (both correctly rounded)
 *   else: *scale and *scale_inv are left unchanged and bit 0 of *status is set.
 *
 * MAX is 448 for E4M3 and 57344 for E5M2.  The new scale is the one the NEXT
 * fp8_quantize of this tensor should use: the amax of the step just cast
 * never influences its own cast.
 *
 * history    device, history_len fp32 (caller-owned; zero it for a fresh tensor).
 * head       device, 1 int32 in [0, history_len).  An out-of-range value is
 *            treated as 0 and bit 1 of *status is set.
 * amax       device, 1 fp32 (e.g. fp8_quantize's amax output).
 * scale, scale_inv  device, 1 fp32 each (fresh tensor: 1.0 and 1.0).
 * status     device, 1 int32 of sticky flags, or NULL.
 * history_len in [1, 4096].
 */
FP8MI_API int fp8_amax_update(float* history, int32_t history_len, int32_t* head, const float* amax,
                    int fmt, float* scale, float* scale_inv, int32_t* status, void* stream);

/*
 * fp8_quantize_update — one delayed-scaling step of a tensor in one call
 * ([TE] §4.2.4, §4.2.6: cast with the scale predicted from the history, then
 * refresh the history and the scale for the next step): exactly
 *     fp8_quantize(x, xtype, rows, cols, fmt, scale, q, q_t, amax, sat, workspace, workspace_bytes)
 *     fp8_amax_update(history, history_len, head, amax, fmt, scale, scale_inv, status)
 * in that order.  The cast uses *scale as it is on entry; the new scale is
 * written after every element has been cast.  With a workspace, the history
 * step runs inside the launch that reduces the per-workgroup partials (two
 * launches in all instead of three).
 *
 * Arguments as for those two calls; amax is required here (it receives this
 * step's amax, which is also pushed into the history).
 * scale_inv_used  device, 1 fp32, or NULL: receives *scale_inv as it was on
 *         entry, i.e. the inverse of the scale this cast used.  A GEMM that
 *         consumes q must be given this value, not *scale_inv, which already
 *         belongs to the next step.
 */
FP8MI_API int fp8_quantize_update(const void* x, int xtype, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                        uint8_t* q_t, float* amax, unsigned long long* sat, void* workspace, size_t workspace_bytes,
                        float* history, int32_t history_len, int32_t* head, float* scale, float* scale_inv,
                        int32_t* status, float* scale_inv_used, void* stream);

/*
 * fp8_quantize_update_noalloc — fp8_quantize_update for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the per-workgroup partials go to a scratch
 * array the library holds on each GPU (FP8MI_NOALLOC_SCRATCH_BYTES, in the
 * library's device data, kept until the process ends) instead of a caller
 * workspace.  The call allocates nothing and frees nothing.
 *
 * Arguments, results and errors are those of fp8_quantize_update without
 * workspace / workspace_bytes; the outputs are bit for bit the same as
 * fp8_quantize_update with a workspace of FP8MI_QUANTIZE_WORKSPACE_BYTES.
 * The scratch holds 4096 partial slots, more than any cast grid uses, so no
 * tensor size is refused for want of scratch (sizes are limited as for
 * fp8_quantize_update).  FP8MI_ERR_DEVICE if the scratch's device address
 * cannot be found on the current device.
 *
 * All calls on one GPU share its scratch: two calls that may run at the same
 * time on one GPU (different streams without ordering between them) race on
 * it and must not be issued.  Calls ordered on one stream, or on streams that
 * are synchronised with each other, are safe; what a previous call left in the
 * scratch never affects the next one.
 */
#define FP8MI_NOALLOC_SCRATCH_BYTES 65536

FP8MI_API int fp8_quantize_update_noalloc(const void* x, int xtype, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                                uint8_t* q_t, float* amax, unsigned long long* sat, float* history,
                                int32_t history_len, int32_t* head, float* scale, float* scale_inv, int32_t* status,
                                float* scale_inv_used, void* stream);

/*
 * fp8_gemm — FP8 x FP8 GEMM with FP32 accumulation and the x(1/scale) restore
 * in the epilogue ([TE] §4.2.4; [FMT] "Technical insight").
 *
 *   C[m][n] = ( sum_k dec_fa(A[m][k]) * dec_fb(B_kn[k][n]) ) * sinv_a[0] * sinv_b[0]
 *
 * A       device, [M x K] uint8 codes of format fa (K contiguous), 16-B aligned.
 * B       device, uint8 codes of format fb, 16-B aligned:
 *           b_trans == 0: [N x K], K contiguous (B_kn[k][n] = B[n][k]; the layout
 *                         fp8_quantize's q_t writes for a weight stored [K x N]);
 *           b_trans != 0: [K x N], N contiguous (B_kn = B); N must be a multiple
 *                         of 16 and K * N < 2^31 (else FP8MI_ERR_ALIGN / _SHAPE).
 *         Both layouts give the same result bit for bit ([TE] §4.2.6: the
 *         forward and backward GEMMs of a layer take the weight in opposite
 *         orientations).
 * sinv_a, sinv_b  device, 1 fp32 each: the inverse scales of A and B.
 * C       device, [M x N] of ctype (fp32, or bf16 rounded to nearest even),
 *         16-B aligned.
 * accum   fp8mi_accum: FP8MI_ACCUM_EXACT (the FP32-accumulation contract above
 *         for every input) or FP8MI_ACCUM_MFMA_FP8 (native FP8 matrix cores; see
 *         the fp8mi_accum note for its arithmetic).
 * K must be a multiple of 16, 0 < K <= 2^23 (else FP8MI_ERR_ALIGN / _SHAPE);
 * M, N >= 0 (M or N == 0 is a no-op).
 * The order in which fp32 partial sums are added is not fixed.
 */
FP8MI_API int fp8_gemm(const uint8_t* A, int fa, const uint8_t* B, int fb, int b_trans, int64_t M, int64_t N,
             int64_t K, const float* sinv_a, const float* sinv_b, void* C, int ctype, int accum, void* stream);

/*
 * fp8_gemm_requant — fp8_gemm whose epilogue re-quantises the result to FP8
 * with the next consumer's scale ([TE] §4.2.4: the x(1/scale) restore
 * "combined with the next stage's scale"; each FP8 tensor's amax feeds its own
 * delayed-scaling history), so the result never makes an fp32 / bf16 round
 * trip through memory.
 *
 *   c[m][n]  = the fp32 value fp8_gemm stores for ctype = FP8MI_F32 (same
 *              accumulation, same x sinv_a[0] x sinv_b[0])
 *   Cq[m][n] = round_to_fp8(fp32(c[m][n] * out_scale[0]))  in out_fmt, exactly
 *              as fp8_quantize encodes (RNE, saturating, NaN -> sign|0x7F)
 *   amax     = max |c| over the M x N results, as the largest (bits & 0x7FFFFFFF)
 *   sat      = #{ (m, n) : |fp32(c * out_scale)| > MAX }  (Inf counts, NaN does not)
 * so the outputs equal fp8_gemm (fp32) followed by fp8_quantize of that result.
 *
 * A, B, fa, fb, sinv_a, sinv_b, M, N, K, accum  as for fp8_gemm.
 * out_fmt    fp8mi_format of Cq (E4M3 for a forward activation, E5M2 for a gradient).
 * out_scale  device, 1 fp32: normally the delayed scale of the output tensor's
 *            own state (fp8_amax_update).
 * Cq         device, [M x N] uint8 codes, 16-B aligned.
 * amax       device, 1 fp32, overwritten, or NULL.  Feed it to the output
 *            tensor's fp8_amax_update.
 * sat        device, 1 uint64, overwritten, or NULL.
 * M or N == 0 writes no codes (amax = 0, sat = 0).  A call clears amax and sat
 * with a small kernel before the GEMM, so two calls in flight at once must not
 * share them.
 */
FP8MI_API int fp8_gemm_requant(const uint8_t* A, int fa, const uint8_t* B, int fb, int64_t M, int64_t N, int64_t K,
                     const float* sinv_a, const float* sinv_b, int out_fmt, const float* out_scale,
                     uint8_t* Cq, float* amax, unsigned long long* sat, int accum, void* stream);

/*
 * fp8_shared_scale — the scale every rank of an FP8 gradient all-reduce casts
 * with ([FMT] use cases: E5M2 gradient communication; [DG-talk] "automatic
 * scaling" keeps gradients inside FP8's range during the all-reduce; [TE]
 * §4.2.4 scale = MAX / amax).
 *
 *   m = max over r < R of amaxes[r]   (bit patterns of |.|: NaN > Inf > finite)
 *   if 0 < m < Inf and s = fp32(MAX / m) is finite: *scale = s, *scale_inv = fp32(1 / s)
 *   else: *scale = *scale_inv = 1
 *
 * amaxes     device, R fp32: each rank's gradient amax after a MAX (or gather)
 *            exchange; on one GPU, the amaxes of the tensors that share a scale.
 * scale, scale_inv  device, 1 fp32 each, overwritten.
 * R in [1, 65536].
 */
FP8MI_API int fp8_shared_scale(const float* amaxes, int32_t R, int fmt, float* scale, float* scale_inv, void* stream);

/*
 * fp8_dequant_sum — the receiving side of an FP8 gradient all-reduce: the R
 * ranks' FP8 payloads of one chunk, summed in fp32 and restored.
 *
 *   out[i] = fp32( fp32( sum over r = 0, 1, ..., R-1 IN THAT ORDER of dec(q[r*stride + i]) ) * scale_inv[0] )
 *
 * (fp32 additions left to right; the first term is dec(q[i]) itself, so -0
 * stays -0.)  bf16 outputs are that value rounded to nearest even.
 *
 * q          device, R payloads of n codes of format fmt, payload r at q + r*stride;
 *            16-B aligned, stride a multiple of 16, stride >= n.
 * scale_inv  device, 1 fp32: the shared inverse scale (fp8_shared_scale).
 * out        device, n of otype (fp32 or bf16), 16-B aligned.
 * R in [1, 65536]; n may be 0.
 */
FP8MI_API int fp8_dequant_sum(const uint8_t* q, int32_t R, int64_t n, int64_t stride, int fmt, const float* scale_inv,
                    void* out, int otype, void* stream);

/*
 * fp8_quantize_mx — MXFP8 quantisation: one power-of-two scale per block of 32
 * consecutive values of a row ([FMT] "Deep dive": per-block scale factors,
 * shared micro-scaling blocks; [TE] §4.2.4: the scale fits the block's amax
 * to the format).  For every block b of a row:
 *   m = max |x| over the block (bit patterns);
 *   e = the smallest integer with m <= MAX * 2^e, clamped to [-127, 127]; e = 0
 *       when m is 0, Inf or NaN;
 *   scales[b] = e + 127   (the 8-bit exponent code: the scale is 2^(code - 127));
 *   q = round_to_fp8(fp32(x * 2^-e))  (as fp8_quantize: RNE, saturating, NaN -> sign|0x7F).
 * The block max lands in (MAX/2, MAX]: nothing saturates in a finite block.
 *
 * x       device, [rows x cols] of xtype, 16-B aligned; cols a multiple of 32.
 * q       device, [rows x cols] uint8 codes, 16-B aligned.
 * scales  device, [cols/32 x FP8MI_MX_SCALE_LD(rows)] uint8 exponent codes,
 *         K-block major with rows permuted inside groups of 64: the code of
 *         block b of row r at scales[b * ld + FP8MI_MX_SCALE_POS(r)] (the
 *         layout fp8_gemm_mx reads: one K block's codes of a 64-row group are
 *         contiguous, rows c, c+16, c+32, c+48 of a group share a dword).
 *         Positions of rows >= rows are not written.
 */
#define FP8MI_MX_SCALE_LD(rows) ((((int64_t)(rows)) + 63) / 64 * 64)
#define FP8MI_MX_SCALE_POS(r) \
  ((((int64_t)(r)) & ~(int64_t)63) | ((((int64_t)(r)) & 15) << 2) | ((((int64_t)(r)) >> 4) & 3))
FP8MI_API int fp8_quantize_mx(const void* x, int xtype, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                    uint8_t* scales, void* stream);

/*
 * fp8_gemm_mx — GEMM on MXFP8 operands:
 *   C[m][n] = sum_k dec_fa(A[m][k]) 2^(sa[m][k/32] - 127) * dec_fb(B[n][k]) 2^(sb[n][k/32] - 127)
 *
 * accum = FP8MI_ACCUM_EXACT: every product exact, sums in fp32 ([TE] §4.2.4:
 *   FP32 accumulation), i.e. within 1e-5 * sum_k |a_k b_k| of the exact sum.
 *   The codes of each row are widened to bf16 with the factor 2^(c - R) of
 *   their block (c the block's scale code, R the row's largest), contracted on
 *   the bf16 matrix cores, and the result multiplied by 2^(R_a - 127) and then
 *   2^(R_b - 127).  This requires every row of A and of B to have all its
 *   block scale codes within 47 of its largest (then every nonzero product is
 *   a normal fp32 number); outputs of a row or column outside that window are
 *   NaN.  (Data quantised from one tensor stays far inside it; an all-zero
 *   block carries code 127.)
 * accum = FP8MI_ACCUM_MFMA_FP8: the FP8 matrix cores with their per-block
 *   scaling (V_MFMA_SCALE_F32_16X16X128_F8F6F4), with the arithmetic of
 *   FP8MI_ACCUM_MFMA_FP8 (runs of 8 products in fixed point 13 bits below
 *   their largest, runs added in fp32); the scales of one 32-deep block are
 *   equal powers of two, so they do not change that model.
 *
 * A, B    device, [M x K] and [N x K] uint8 codes (K contiguous), 16-B aligned.
 * sa, sb  device, [K/32 x FP8MI_MX_SCALE_LD(M)] and [K/32 x FP8MI_MX_SCALE_LD(N)]
 *         exponent codes in fp8_quantize_mx's layout, 4-B aligned.  Code 255 (NaN) is not produced by the quantiser; its effect
 *         here is the instruction's.  The pad bytes only feed outputs that are
 *         not stored.
 * C       device, [M x N] fp32 or bf16, 16-B aligned.
 * K must be a multiple of 128, K <= 2^23, and each scale matrix must hold
 * fewer than 2^31 bytes (else FP8MI_ERR_SHAPE).
 */
FP8MI_API int fp8_gemm_mx(const uint8_t* A, int fa, const uint8_t* sa, const uint8_t* B, int fb, const uint8_t* sb,
                int64_t M, int64_t N, int64_t K, void* C, int ctype, int accum, void* stream);

/*
 * fp8_quantize_blockwise — current (not delayed) per-block scaling
 * ([FMT] "Deep dive": per-tensor or per-block scale factors; [DG]).
 *
 * Blocks are block_rows x 128 (block_rows = 1 for activations, 128 for
 * weights).  For every block b:  m_b = max |x| over the block (bit patterns);
 *   s_b = fp32(MAX / m_b) if 0 < m_b < Inf and the quotient is finite, else 1;
 *   q   = round_to_fp8(fp32(x * s_b))  (as fp8_quantize);
 *   scale_inv[b] = fp32(1 / s_b).
 *
 * x          device, [rows x cols] of xtype, 16-B aligned.
 * q          device, [rows x cols] uint8, 16-B aligned.
 * scale_inv  device, [ceil(rows/block_rows) x ceil(cols/128)] fp32.
 * cols must be a multiple of 16; block_rows is 1 or 128.
 */
FP8MI_API int fp8_quantize_blockwise(const void* x, int xtype, int64_t rows, int64_t cols, int32_t block_rows,
                           int fmt, uint8_t* q, float* scale_inv, void* stream);

/*
 * fp8_grouped_gemm — fine-grained-scaled grouped GEMM for MoE experts with
 * two-level accumulation ([DG]: grouped GEMM, "promotion" of FP8 partial sums).
 *
 * Expert g owns rows [m_offsets[g], m_offsets[g+1]) of A and C.  For each row
 * m of expert g and each 128-wide K block kb:
 *   P = sum_{k in kb} dec(A[m][k]) * dec(B[g][n][k])   (an FP32 MFMA partial)
 *   C[m][n] += sinv_a[m][kb] * sinv_b[g][n/128][kb] * P  (FP32 "promotion")
 *
 * A          device, [total_m x K] E4M3 codes.
 * sinv_a     device, [total_m x ceil(K/128)] fp32 (per 1x128 tile).
 * B          device, [G x N x K] E4M3 codes (each expert's weight, K contiguous).
 * sinv_b     device, [G x ceil(N/128) x ceil(K/128)] fp32 (per 128x128 block).
 * m_offsets  device, G+1 int32, non-decreasing, m_offsets[0] = 0,
 *            m_offsets[G] = total_m.  Each expert interval is clamped to
 *            [end of the previous interval, total_m]; rows outside every
 *            interval are left untouched.
 * C          device, [total_m x N] of ctype.
 * accum      fp8mi_accum, as for fp8_gemm (applies to each 128-deep partial P).
 * K must be a multiple of 16, K <= 2^22; G in [1, 1024]; all pointers 16-B aligned.
 */
FP8MI_API int fp8_grouped_gemm(const uint8_t* A, const float* sinv_a, const uint8_t* B, const float* sinv_b,
                     const int32_t* m_offsets, int32_t G, int64_t total_m, int64_t N, int64_t K,
                     void* C, int ctype, int accum, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8MI_H */
