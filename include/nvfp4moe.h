/*
 * nvfp4moe -- NVFP4 token-wise quantization and the W4A4 MoE grouped GEMM
 * path for one AMD MI355X (gfx950), behind a plain C ABI.
 *
 * Sources.  The pages this library follows are three news reports on the
 * miniTE technical report:
 *   [RU] "miniTE ускоряет RL в NVFP4 на B300: 1,39× к BF16 на Qwen3-30B-A3B"
 *        (hamidun.com; the Arabic page of the same address family is its twin)
 *   [JA] "miniTE報告、NVFP4強化学習の安定性を検証" (aib.vote)
 * [RU], key-facts list: native NVFP4 W4A4 (4-bit weights and activations).
 * [RU], section "Диагностика, выравнивание и быстрые ядра": the NVFP4
 *        kernels, the scaling scheme and grouped GEMMs over MoE experts
 *        carry the overhead that made naive FP4 slower than BF16.
 * [JA], fourth paragraph: the token-wise NVFP4 path is sped up with a
 *        contiguous data layout, device-side metadata, amax reuse, grouped
 *        GEMM and op fusion; quantization policy, linear layers and compute
 *        backend are kept apart (this library is the compute backend).
 * [JA], first paragraph: the backward pass runs in BF16.
 *
 * NVFP4 as defined by this library (the pages do not define it): per row,
 * 16 consecutive elements along K share one E4M3 (OCP E4M3FN) scale byte;
 * each element is a 4-bit E2M1 code (bit 3 = sign, magnitudes
 * 0,.5,1,1.5,2,3,4,6); one FP32 global decode scale g per tensor or per
 * row-group.  Value = e2m1(code) * e4m3(scale) * g.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers, owned by the caller.  The library
 *     never allocates, frees or synchronises; work is enqueued on `stream`
 *     (a hipStream_t; NULL = the default stream) and the call returns.
 *   - Row-major layouts; leading dimension = row length unless stated.
 *   - Errors the host can see (NULL pointer, negative size, bad enum, shape
 *     or alignment) are returned BEFORE any HIP call.  Then the current
 *     device is checked to be gfx950 (NVFP4MOE_EARCH otherwise).  Launch
 *     failures return NVFP4MOE_ELAUNCH.
 *   - Errors that depend on device data (an expert id outside [0, E)) never
 *     stop the host: they OR a bit into the optional device word `status`
 *     (int32, caller-zeroed, sticky) and the offending item is skipped.
 *   - Zero-sized work (rows == 0, T == 0, ...) is valid and launches nothing
 *     except what is needed to write well-defined outputs.
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* nvfp4moe_stream_t; /* == hipStream_t */

/* status codes */
#define NVFP4MOE_OK 0
#define NVFP4MOE_EINVAL (-1)     /* NULL pointer, negative size, bad enum */
#define NVFP4MOE_ESHAPE (-2)     /* shape or alignment not supported */
#define NVFP4MOE_EARCH (-3)      /* current device is not gfx950 */
#define NVFP4MOE_ELAUNCH (-4)    /* a kernel launch failed */
#define NVFP4MOE_EWORKSPACE (-5) /* workspace missing or too small */

/* device status bits */
#define NVFP4MOE_STATUS_BAD_EXPERT 1 /* a routing id was outside [0, E) */

/* dtype enum */
#define NVFP4MOE_F32 0
#define NVFP4MOE_BF16 1
#define NVFP4MOE_U8 2

/* GEMM layouts for nvfp4moe_grouped_gemm_bf16 */
#define NVFP4MOE_NT 0 /* C[M,N]   = A[M,K] . B_e[N,K]^T  (forward, baseline) */
#define NVFP4MOE_NN 1 /* C[M,N]   = A[M,K] . B_e[K,N]    (data gradient)     */
#define NVFP4MOE_TN 2 /* C_e[K,N] = A_e[M_e,K]^T . B_e[M_e,N] (weight grad)  */

/* MX element formats for mx_quantize (the W4A8 variant) */
#define NVFP4MOE_MX_E4M3 0 /* MXFP8: E4M3 elements, one byte each */
#define NVFP4MOE_MX_E2M1 1 /* MXFP4: E2M1 elements, two per byte */

/* W4A4 GEMM epilogues */
#define NVFP4MOE_EPI_NONE 0
#define NVFP4MOE_EPI_SILU_GATE 1 /* c receives H = silu(gate) * up, see below */

/* ABI version of this header; returned by nvfp4moe_abi_version(). */
#define NVFP4MOE_ABI_VERSION 2

int nvfp4moe_abi_version(void);
/* Static string for a status code (never NULL). */
const char* nvfp4moe_status_string(int status);

/*
 * nvfp4_quantize -- NVFP4 quantization of `rows` x `K` values (steps of the
 * scaling scheme, [RU] fast-kernels section; amax reuse, [JA] fourth
 * paragraph).  The rows form `groups` equal consecutive row-groups; each
 * group has its own global scale (groups = 1 for an activation tensor,
 * groups = E for a stacked [E*N, K] expert weight).
 *
 *   x        [rows][K] of x_dtype (NVFP4MOE_F32 or NVFP4MOE_BF16), 16-byte
 *            aligned.  Finite values.
 *   amax_in  [groups] fp32 or NULL.  When given, it is the amax used for the
 *            global scale (amax reuse; a stale value saturates, it is not an
 *            error).  When NULL, the amax of each group is computed and
 *            written to amax_out (which must then be non-NULL) and used.
 *   amax_out [groups] fp32 or NULL; written only when amax_in is NULL.
 *   q        [rows][K/2] bytes out: two E2M1 codes per byte, element 2j in
 *            the low nibble; 8-byte aligned.
 *   scales   [rows][K/16] bytes out: E4M3 scale per block, row-major,
 *            unswizzled.
 *   gscale   [groups] fp32 out: g = amax / 2688 (1 when amax == 0).
 *   status   unused (may be NULL); kept for a uniform signature.
 * Per 16-block with amax a: t = a/6, u = t/g, S = E4M3_RNE_satfinite(u),
 * s = decode(S), d = s*g; code = sign(x) | E2M1_RNE_satfinite(|x|/d)
 * (magnitude 0 when d == 0).  All steps IEEE fp32, correctly rounded;
 * results are bit-exact and independent of launch shape.
 * Errors: EINVAL (NULL, negative, bad dtype, groups < 1, amax_in and
 * amax_out both NULL), ESHAPE (K % 16 != 0, rows % groups != 0, alignment).
 */
int nvfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t K, int64_t groups,
                   const float* amax_in, float* amax_out, uint8_t* q, uint8_t* scales,
                   float* gscale, int32_t* status, nvfp4moe_stream_t stream);

/*
 * nvfp4_quantize_onepass -- nvfp4_quantize with the amax computed
 * (amax_in = NULL), reading x once instead of twice: the same outputs, bit
 * for bit.  Meant for stacked expert weights (groups = E), which are
 * quantized once per optimizer step (scaling scheme and amax reuse: [RU]
 * fast-kernels section, [JA] fourth paragraph).
 *
 * Each group is cut into slices of 1024 blocks of 16.  The workgroups of a
 * group's slices keep their slice in registers and publish its amax in a
 * slot of `workspace`; once every slot of the group is filled they encode
 * with the group's amax.  A workgroup that finds the group incomplete after
 * a bounded wait reads the whole group for its amax instead, so the results
 * never depend on scheduling (the environment variable
 * NVFP4MOE_ONEPASS_POLL_LIMIT, read at each call, overrides the bound; 0
 * takes that path at once, for tests).  Groups larger than what the device
 * holds in flight at once (about 16 M elements on MI355X) take the two-pass
 * path inside the call, with the same results.
 *
 *   x, x_dtype, rows, K, groups, q, scales, gscale: as for nvfp4_quantize.
 *   amax_out  [groups] fp32 out (required): the amax of each group.
 *   workspace device scratch of nvfp4_quantize_onepass_workspace_size(rows,
 *             K, groups) bytes (4-byte aligned; may be NULL when that size
 *             is 0).  Its contents on entry do not matter; calls that share
 *             one workspace must not overlap.
 * Errors: as nvfp4_quantize; EWORKSPACE when the workspace is missing or
 * too small.
 */
size_t nvfp4_quantize_onepass_workspace_size(int64_t rows, int64_t K, int64_t groups);
int nvfp4_quantize_onepass(const void* x, int x_dtype, int64_t rows, int64_t K, int64_t groups, float* amax_out,
                           uint8_t* q, uint8_t* scales, float* gscale, void* workspace, size_t workspace_bytes,
                           nvfp4moe_stream_t stream);

/*
 * moe_permute -- routing metadata for the contiguous per-expert layout and
 * (optionally) the row gather into it, with the amax of the gathered rows
 * fused in (contiguous layout, device-side metadata, amax reuse: [JA],
 * fourth paragraph).
 *
 * Assignment i = t*k + j (token t, slot j) with expert topk_ids[t][j] goes
 * to permuted row dest[i]; rows of expert e are [offsets[e], offsets[e+1]);
 * inside a segment rows keep assignment order (a stable counting sort,
 * deterministic).  src[dest[i]] = i.  offsets[E] = number of valid
 * assignments (T*k unless some id is out of range: such an assignment gets
 * dest = -1, is not placed, and sets NVFP4MOE_STATUS_BAD_EXPERT).
 *
 *   topk_ids  [T][k] int32 (device).            T >= 0, 1 <= k, 1 <= E <= 4096
 *   x         [T][row_elems] of x_dtype, or NULL (metadata only).  16-byte
 *             aligned; row bytes a multiple of 16.
 *   x_perm    [T*k][row_elems] out (ignored when x is NULL).
 *   offsets   [E+1] int32 out; dest, src [T*k] int32 out (src entries past
 *             offsets[E] are -1).
 *   amax_out  fp32 [1] or NULL: max |x| over the gathered rows (F32/BF16
 *             payloads only; 0 for an empty gather).
 *   workspace device scratch of moe_permute_workspace_size(T, k, E) bytes
 *             (per-chunk expert histograms; moe_permute_nvfp4 also keeps the
 *             parts of its activation amax there).
 */
size_t moe_permute_workspace_size(int64_t T, int k, int E);
int moe_permute(const int32_t* topk_ids, int64_t T, int k, int E, const void* x, int x_dtype,
                int64_t row_elems, void* x_perm, int32_t* offsets, int32_t* dest, int32_t* src,
                float* amax_out, void* workspace, size_t ws_bytes, int32_t* status,
                nvfp4moe_stream_t stream);

/*
 * moe_permute_nvfp4 -- moe_permute fused with the NVFP4 quantization of the
 * gathered rows (token-wise path with contiguous layout, device-side
 * metadata, amax reuse and op fusion: [JA], fourth paragraph).  Computes the
 * same offsets/dest/src as moe_permute, optionally the bf16 rows x_perm, and
 * q/scales/gscale equal to nvfp4_quantize(x_perm, groups = 1, amax_in =
 * amax) -- bit for bit -- without reading x_perm back: each row of x is
 * encoded once and its codes and scales (and bf16 copy) are written to its
 * k permuted rows.
 *   x        [T][D] bf16, 16-byte aligned; D % 16 == 0.
 *   x_perm   [T*k][D] bf16 out, or NULL when only the NVFP4 rows are needed.
 *   amax_in  fp32 [1] or NULL.  When NULL, amax = max |x| over all T rows of
 *            x is computed first and written to amax_out (then non-NULL).
 *            With every id valid it equals max |x_perm| (each token is
 *            routed); a token whose ids are all invalid has no permuted row
 *            but still counts (0 when D == 0).
 *   q        [T*k][D/2], scales [T*k][D/16], gscale [1] out (see
 *            nvfp4_quantize).  Rows past offsets[E] (invalid ids) are zeros.
 *   offsets, dest, src, workspace, status: as for moe_permute.
 * Errors: EINVAL (NULL, negative sizes, amax_in and amax_out both NULL),
 * ESHAPE (D % 16, alignment, E > 4096, k > 64), EWORKSPACE.
 */
int moe_permute_nvfp4(const int32_t* topk_ids, int64_t T, int k, int E, const void* x, int64_t D,
                      void* x_perm, const float* amax_in, float* amax_out, uint8_t* q, uint8_t* scales,
                      float* gscale, int32_t* offsets, int32_t* dest, int32_t* src, void* workspace,
                      size_t ws_bytes, int32_t* status, nvfp4moe_stream_t stream);

/*
 * moe_permute_nvfp4_noalloc -- moe_permute_nvfp4 for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same arguments without the
 * workspace, the same results bit for bit.  The histograms and amax parts
 * live in a library-owned device array of NVFP4MOE_NOALLOC_SCRATCH_BYTES
 * per GPU, kept until the process ends; no allocation of any kind happens
 * in the call.  Calls whose moe_permute_workspace_size(T, k, E) exceeds it
 * return NVFP4MOE_EWORKSPACE before any HIP call.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two threads) race and must be ordered by the caller.  Nothing in
 * the array needs clearing between calls.  Errors otherwise as
 * moe_permute_nvfp4.
 */
#define NVFP4MOE_NOALLOC_SCRATCH_BYTES (2u << 20)
int moe_permute_nvfp4_noalloc(const int32_t* topk_ids, int64_t T, int k, int E, const void* x, int64_t D,
                              void* x_perm, const float* amax_in, float* amax_out, uint8_t* q,
                              uint8_t* scales, float* gscale, int32_t* offsets, int32_t* dest, int32_t* src,
                              int32_t* status, nvfp4moe_stream_t stream);

/*
 * moe_permute_mx -- moe_permute's routing metadata with the MXFP8
 * quantization of X fused into the permutation (the W4A8 variant's
 * activations, [JA] third paragraph; contiguous layout and op fusion, [JA]
 * fourth paragraph): each row of X is read once, quantized once (E4M3
 * elements, one E8M0 scale per 32, the rule of mx_quantize) and its codes
 * and scales are written to the token's k permuted rows.  Rows past
 * offsets[E] (skipped assignments) are zeros.  The results equal, bit for
 * bit, mx_quantize(x, NVFP4MOE_MX_E4M3) followed by the row gather of the
 * codes and of the scales through src.
 *   topk_ids, T, k, E, offsets, dest, src, workspace, ws_bytes, status: as
 *             moe_permute (workspace of moe_permute_workspace_size bytes).
 *   x         [T][D] of x_dtype (NVFP4MOE_BF16 or NVFP4MOE_F32), 16-byte
 *             aligned; D % 32 == 0.
 *   q         [T*k][D] E4M3 codes out (16-byte aligned).
 *   scales    [T*k][D/32] E8M0 scale bytes out.
 * Errors: EINVAL (NULL, negative, bad dtype), ESHAPE (D % 32, alignment,
 * E > 4096, k > 64, T*k >= 2^31), EWORKSPACE.
 */
int moe_permute_mx(const int32_t* topk_ids, int64_t T, int k, int E, const void* x, int x_dtype, int64_t D,
                   uint8_t* q, uint8_t* scales, int32_t* offsets, int32_t* dest, int32_t* src, void* workspace,
                   size_t ws_bytes, int32_t* status, nvfp4moe_stream_t stream);

/*
 * moe_gather -- out[p] = w[src[p]] * x[src[p] / k] for p < R (w = 1 when
 * topk_w is NULL); rows with src[p] < 0 are written as zeros.  With
 * topk_w == NULL any dtype is copied verbatim (NVFP4MOE_U8 row payloads,
 * e.g. packed NVFP4 codes or scales); with weights the payload must be
 * F32/BF16 and is scaled in fp32 and rounded to out_dtype (RNE).  This is
 * the backward of the unpermute-combine ([JA] first and fourth paragraphs).
 *   x [T][row_elems], src [R], out [R][row_elems]; 16-byte aligned rows.
 */
int moe_gather(const void* x, int x_dtype, int64_t row_elems, const int32_t* src,
               const float* topk_w, int k, int64_t R, void* out, int out_dtype,
               nvfp4moe_stream_t stream);

/*
 * moe_scatter -- the same rows as moe_gather with weights, written from the
 * token side: out[dest[t*k+j]] = w[t*k+j] * x[t] (w = 1 when topk_w is NULL),
 * scaled in fp32 and rounded to out_dtype (RNE); assignments with dest < 0
 * are skipped and rows of out past offsets[E] are written as zeros.  Equal,
 * bit for bit, to moe_gather(x, src, topk_w) for the src and dest of one
 * permutation; each row of x is read once.  Row i of the backward's
 * dY2[dest] = w * dY ([JA] first paragraph: the BF16 backward).
 *   x [T][row_elems] F32/BF16, dest [T*k], topk_w [T*k] fp32 or NULL,
 *   offsets [E+1] (device), out [T*k][row_elems]; 16-byte aligned rows,
 *   row_elems % 8 == 0.
 *   amax_out fp32 [1] or NULL: max |out| over the stored values, for the
 *   NVFP4 quantization of out that follows (amax reuse, [JA] fourth
 *   paragraph); 0 when nothing is written.
 * Errors: EINVAL (NULL, negative sizes, bad dtype), ESHAPE (row_elems % 8,
 * alignment, T*k >= 2^31).
 */
int moe_scatter(const void* x, int x_dtype, int64_t row_elems, const int32_t* dest,
                const float* topk_w, const int32_t* offsets, int E, int64_t T, int k, void* out,
                int out_dtype, float* amax_out, nvfp4moe_stream_t stream);

/*
 * moe_unpermute -- out[t] = sum_{j=0..k-1} w[t][j] * y_perm[dest[t*k+j]]
 * (w = 1 when topk_w is NULL: the gradient of the row gather), accumulated
 * in fp32 in ascending j with fused multiply-add, then rounded to out_dtype
 * (RNE).  Entries with dest < 0 contribute nothing.  ([JA] fourth paragraph:
 * contiguous layout.)
 *   y_perm [*][D] of y_dtype (F32/BF16), dest [T*k], topk_w [T][k] fp32 or
 *   NULL, out [T][D] of out_dtype (F32/BF16).  D % 8 == 0, 16-byte aligned.
 */
int moe_unpermute(const void* y_perm, int y_dtype, const int32_t* dest, const float* topk_w,
                  int64_t T, int k, int64_t D, void* out, int out_dtype, nvfp4moe_stream_t stream);

/*
 * grouped_gemm_w4a4 -- the grouped NVFP4 x NVFP4 GEMM over the contiguous
 * per-expert layout ([RU] fast-kernels section; [JA] fourth paragraph):
 *   C[r][n] = a_g * b_g[e] * sum_k deq(A)[r][k] * deq(B_e)[n][k]
 * for rows r in [offsets[e], offsets[e+1]).  deq = e2m1 * e4m3 scale
 * (exact); products accumulate in fp32.  Rows >= offsets[E] are not written.
 *   a_q [M_total][K/2], a_s [M_total][K/16], a_g [1]      (activations)
 *   b_q [E][N][K/2],    b_s [E][N][K/16],    b_g [E]      (expert weights)
 *   offsets [E+1] int32 on the device (never read by the host)
 *   c [M_total][N] of c_dtype (F32/BF16)
 * K % 64 == 0 (every 64-element step holds whole 16-blocks and 4-byte
 * aligned scale words), N % 32 == 0; a_q, b_q, c 16-byte aligned, a_s, b_s
 * 4-byte aligned.  workspace may be NULL (none needed).
 * epilogue NVFP4MOE_EPI_NONE: c as above.
 * epilogue NVFP4MOE_EPI_SILU_GATE (the gate+up projection, B_e = [gate rows
 * 0..F-1; up rows F..2F-1] with N = 2F): c receives only H [M_total][F]
 * bf16 (c_dtype must be BF16), the SiLU gate of the bf16-rounded C exactly as
 * silu_gate_fwd computes it, and amax_out[0] (may be NULL) = max |H|
 * ([JA] fourth paragraph: op fusion, amax reuse).  N % 256 == 0.
 * M_total, N, K < 2^31.  Errors: EINVAL (NULL, negative, bad enum), ESHAPE
 * (the shape and alignment rules above).
 */
int grouped_gemm_w4a4(const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
                      const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
                      const int32_t* expert_offsets, int E, int64_t M_total, int64_t N, int64_t K,
                      void* c, int c_dtype, int epilogue, float* amax_out, void* workspace,
                      size_t ws_bytes, nvfp4moe_stream_t stream);

/*
 * grouped_gemm_w4a4_scaled_mfma -- the same product as grouped_gemm_w4a4
 * (NVFP4MOE_EPI_NONE) computed the other way open on gfx950 ([RU] fast-kernels
 * section: the scaling scheme's cost): NVFP4's E4M3 block scales are not
 * E8M0, so the scaled fp4 MFMA runs one 16-element block per instruction
 * with unit E8M0 scales and the other K slots zero, and each block's exact
 * partial sums are multiplied by sA * sB and accumulated in fp32.  Kept to
 * measure this design against the shipped one (exact fp16 expansion on the
 * 16-bit MFMA, grouped_gemm_w4a4), which it loses to: the per-element fp32
 * rescale and the 4x zero padding of the MFMA's K.  Arguments, layouts and
 * errors as grouped_gemm_w4a4.
 */
int grouped_gemm_w4a4_scaled_mfma(const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
                                  const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
                                  const int32_t* expert_offsets, int E, int64_t M_total, int64_t N, int64_t K,
                                  void* c, int c_dtype, nvfp4moe_stream_t stream);

/*
 * grouped_gemm_w4a4_silu_gate -- the gate+up W4A4 GEMM with the SiLU gate
 * and the amax of its output in the epilogue ([JA] fourth paragraph: op
 * fusion, amax reuse): the result equals grouped_gemm_w4a4 (N = 2F, bf16 C)
 * followed by silu_gate_fwd, bit for bit, without re-reading Y1.
 *   operands as grouped_gemm_w4a4 with N = 2F (B_e = [gate; up] rows)
 *   y1 [M_total][2F] bf16 or NULL: Y1 is stored only when given (the BF16
 *      backward needs it)
 *   h  [M_total][F] bf16: H = silu(G) * U of the bf16 Y1, fp32 math
 *   amax_out [1] fp32 or NULL: max |H| over the stored bf16 values
 * F % 128 == 0, K % 64 == 0; y1, h 16-byte aligned.  Errors as
 * grouped_gemm_w4a4.
 */
int grouped_gemm_w4a4_silu_gate(const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
                                const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
                                const int32_t* expert_offsets, int E, int64_t M_total, int64_t F,
                                int64_t K, void* y1, void* h, float* amax_out,
                                nvfp4moe_stream_t stream);

/*
 * grouped_gemm_w4a4_silu_gate_nvfp4 -- grouped_gemm_w4a4_silu_gate with the
 * NVFP4 requantization of H in the same epilogue ([JA], fourth paragraph:
 * op fusion and amax reuse), for a caller that hands in the amax of H (a
 * delayed amax, e.g. the previous step's, or one agreed otherwise): q_h,
 * s_h and g_h equal nvfp4_quantize(H, groups = 1, amax_in = amax_h_in) bit
 * for bit, H being the bf16 SiLU gate that h would receive, so neither Y1
 * nor H needs to be stored or re-read.  A stale amax saturates, as in
 * nvfp4_quantize.
 *   operands, F, K, y1 (nullable) as grouped_gemm_w4a4_silu_gate
 *   h         [M_total][F] bf16 or NULL (not stored)
 *   amax_out  [1] fp32 or NULL: max |H| of this call (the next step's
 *             delayed amax); must not alias amax_h_in
 *   amax_h_in [1] fp32, device: the amax used for H's global scale
 *   q_h [M_total][F/2], s_h [M_total][F/16], g_h [1] out (4-byte aligned)
 * Errors as grouped_gemm_w4a4_silu_gate; EINVAL also for a NULL q_h, s_h,
 * g_h or amax_h_in, or amax_out == amax_h_in.
 */
int grouped_gemm_w4a4_silu_gate_nvfp4(const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
                                      const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
                                      const int32_t* expert_offsets, int E, int64_t M_total, int64_t F,
                                      int64_t K, void* y1, void* h, float* amax_out,
                                      const float* amax_h_in, uint8_t* q_h, uint8_t* s_h, float* g_h,
                                      nvfp4moe_stream_t stream);

/*
 * The NVFP4 backward variant.  The learner backward of [JA] (first
 * paragraph) is BF16 (grouped_gemm_bf16 below); the headline learner speed-up
 * of [RU] (intro, key-facts list) is read as possibly including quantized
 * backward GEMMs.  This variant keeps the BF16 backward's dataflow and runs
 * its four grouped GEMMs as W4A4:
 *   dH = dY2 . Wdn_e, dX_perm = dY1 . Wgu_e   grouped_gemm_w4a4 with the
 *        gradient quantized by nvfp4_quantize (along its columns) and the
 *        weights by nvfp4_quantize_transposed;
 *   dWdn_e = dY2_e^T . H_e, dWgu_e = dY1_e^T . X_perm_e   grouped_gemm_w4a4_wgrad
 *        on operands quantized by nvfp4_quantize_colwise.
 * Gradients are rounded like every NVFP4 tensor (RNE; the pages do not say).
 *
 * nvfp4_quantize_colwise -- column-wise NVFP4 of a row-grouped bf16 tensor:
 * within each expert's row segment [offsets[e], offsets[e+1]), 16
 * consecutive rows of one column form a block (E4M3 scale, E2M1 codes, the
 * steps of nvfp4_quantize); the segment's tail is zero-padded.  Stored
 * transposed: column n of x becomes row n of q_t / s_t, expert e's segment
 * starting at column poff_e = 64 * (floor(offsets[e] / 64) + e), padded with
 * zero blocks to a multiple of 64 (it never reaches poff_{e+1}).  One global
 * scale g = amax_in[0] / 2688 (amax reuse: the tensor's amax, e.g. from its
 * row-wise quantization; 1 when 0).
 *   x        [M_total][N] bf16, 16-byte aligned; N % 8 == 0.
 *   offsets  [E+1] int32 on the device (as produced by moe_permute).
 *   q_t      [N][Kp/2] out (16-byte aligned), s_t [N][Kp/16] out (4-byte
 *            aligned); columns outside the padded segments are not written.
 *   Kp       row length of q_t/s_t: Kp % 64 == 0, Kp >= 64*(M_total/64 + E).
 *   gscale   [1] out.
 * Errors: EINVAL (NULL, negative, dtype other than BF16), ESHAPE (N % 8,
 * Kp, alignment, q_t of 2 GiB or more).
 */
int nvfp4_quantize_colwise(const void* x, int x_dtype, int64_t M_total, int64_t N,
                           const int32_t* expert_offsets, int E, const float* amax_in, uint8_t* q_t,
                           uint8_t* s_t, float* gscale, int64_t Kp, nvfp4moe_stream_t stream);

/*
 * nvfp4_quantize_transposed -- NVFP4 of stacked bf16 matrices quantized
 * along their rows' index: x [groups][L][N] gives the codes of each
 * transposed matrix, q_t [groups][N][L/2], s_t [groups][N][L/16], blocks of
 * 16 consecutive rows of one column, one global scale per group (for the
 * expert weights of the data-gradient GEMMs: W^T_e, whose amax is that of
 * W_e, so amax_in may be the forward weights' amax).  amax_in [groups] or
 * NULL (then computed into amax_out).  L % 64 == 0, N % 8 == 0; x, q_t
 * 16-byte aligned; q_t under 2 GiB.  Errors as nvfp4_quantize (ESHAPE for
 * q_t of 2 GiB or more).
 */
int nvfp4_quantize_transposed(const void* x, int x_dtype, int64_t groups, int64_t L, int64_t N,
                              const float* amax_in, float* amax_out, uint8_t* q_t, uint8_t* s_t,
                              float* gscale, nvfp4moe_stream_t stream);

/*
 * grouped_gemm_w4a4_wgrad -- the NVFP4 weight gradient over the contiguous
 * per-expert layout:
 *   C_e[i][j] = a_g * b_g * sum over rows r of expert e of deq(A)[r][i] * deq(B)[r][j]
 * with A and B given column-wise (nvfp4_quantize_colwise with the same
 * offsets and Kp): a_q [N1][Kp/2], a_s [N1][Kp/16], a_g [1]; b_q [N2][Kp/2],
 * b_s [N2][Kp/16], b_g [1].  c [E][N1][N2] F32 (or BF16); an empty expert
 * gives zeros.  fp32 accumulation.  N1 % 32 == 0, N2 % 32 == 0, Kp as for
 * nvfp4_quantize_colwise; N1*Kp/2 and N2*Kp/2 < 2^31.  Errors: EINVAL,
 * ESHAPE.
 */
int grouped_gemm_w4a4_wgrad(const uint8_t* a_q, const uint8_t* a_s, const float* a_g, const uint8_t* b_q,
                            const uint8_t* b_s, const float* b_g, const int32_t* expert_offsets, int E,
                            int64_t M_total, int64_t Kp, int64_t N1, int64_t N2, void* c, int c_dtype,
                            nvfp4moe_stream_t stream);

/*
 * mx_quantize -- MX quantization for the W4A8 variant, whose activations are
 * MXFP8 ([JA], third paragraph: the activation-precision comparison of
 * W4A16, W4A8 with MXFP8 activations, and W4A4).  The pages do not define MX;
 * the library follows the published microscaling rule: every 32 consecutive
 * elements of a row along K share one E8M0 scale byte S (value 2^(S-127));
 * for a block with amax a > 0, S - 127 = floor(log2 a) - emax (emax 8 for
 * E4M3, 2 for E2M1) clamped to [-127, 127], and S = 0 for an all-zero block.
 * Element = (V / 2^(S-127)) rounded to nearest even and saturated to 448
 * (E4M3) or 6 (E2M1); its sign bit is the sign of V (also for -0).  No global
 * scale, no amax pass: each block is encoded from its own values.
 *   x       [rows][K] F32 or BF16, 16-byte aligned, finite.
 *   elem    NVFP4MOE_MX_E4M3: q [rows][K] bytes (16-byte aligned);
 *           NVFP4MOE_MX_E2M1: q [rows][K/2] bytes, element 2j in the low
 *           nibble (8-byte aligned).
 *   scales  [rows][K/32] bytes out, row-major, unswizzled.
 * Bit-exact and independent of launch shape.  Errors: EINVAL (NULL,
 * negative, bad dtype or elem), ESHAPE (K % 32 != 0, alignment).
 */
int mx_quantize(const void* x, int x_dtype, int64_t rows, int64_t K, int elem, uint8_t* q,
                uint8_t* scales, nvfp4moe_stream_t stream);

/*
 * grouped_gemm_w4a8 -- the grouped GEMM of the W4A8 variant ([JA], third
 * paragraph): MXFP8 activations (E4M3 elements) times MXFP4 expert weights
 * (E2M1 elements), both with E8M0 scales per 32 along K, over the contiguous
 * per-expert layout ([JA], fourth paragraph):
 *   C[r][n] = sum_k deq(A)[r][k] * deq(B_e)[n][k],  r in [offsets[e], offsets[e+1])
 * with deq = element * 2^(S-127).  The scales are powers of two, so gfx950's
 * scaled MFMA takes them natively (no operand expansion); accumulation in
 * fp32.  Rows >= offsets[E] are not written.
 *   a_q [M_total][K], a_s [M_total][K/32]     (mx_quantize E4M3)
 *   b_q [E][N][K/2],  b_s [E][N][K/32]        (mx_quantize E2M1)
 *   offsets [E+1] int32 on the device; c [M_total][N] F32 or BF16.
 * K % 128 == 0, N % 32 == 0; a_q, b_q, c 16-byte aligned, a_s, b_s 4-byte
 * aligned; M_total, N, K < 2^31.  Errors: EINVAL (NULL, negative, bad
 * dtype), ESHAPE (shape and alignment rules).
 */
int grouped_gemm_w4a8(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                      const int32_t* expert_offsets, int E, int64_t M_total, int64_t N, int64_t K, void* c,
                      int c_dtype, nvfp4moe_stream_t stream);

/*
 * grouped_gemm_w4a8_silu_gate -- the W4A8 gate+up GEMM with the SiLU gate
 * and the amax of its output in the epilogue, as grouped_gemm_w4a4_silu_gate
 * ([JA], fourth paragraph: op fusion): equal, bit for bit, to
 * grouped_gemm_w4a8 (N = 2F, bf16 C) followed by silu_gate_fwd.
 *   operands as grouped_gemm_w4a8 with N = 2F (B_e = [gate; up] rows)
 *   y1 [M_total][2F] bf16 or NULL, h [M_total][F] bf16, amax_out [1] or NULL.
 * F % 128 == 0, K % 128 == 0.  Errors as grouped_gemm_w4a8.
 */
int grouped_gemm_w4a8_silu_gate(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q,
                                const uint8_t* b_s, const int32_t* expert_offsets, int E, int64_t M_total,
                                int64_t F, int64_t K, void* y1, void* h, float* amax_out,
                                nvfp4moe_stream_t stream);

/*
 * grouped_gemm_w4a8_silu_gate_mx -- grouped_gemm_w4a8_silu_gate that also
 * quantizes H to MXFP8 in the epilogue ([JA], fourth paragraph: op fusion;
 * the W4A8 variant, third paragraph), ready for the down GEMM: q_h and s_h
 * equal, bit for bit, mx_quantize(H, NVFP4MOE_MX_E4M3) of the bf16 H the
 * epilogue computes.  MX has no global scale, so no amax is needed first.
 *   operands, y1, amax_out as grouped_gemm_w4a8_silu_gate; h may be NULL
 *   (H is then not stored in bf16).
 *   q_h [M_total][F] E4M3 codes (8-byte aligned), s_h [M_total][F/32] E8M0
 *   scale bytes; rows >= offsets[E] are not written.
 * Errors as grouped_gemm_w4a8 (EINVAL for q_h or s_h NULL).
 */
int grouped_gemm_w4a8_silu_gate_mx(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q,
                                   const uint8_t* b_s, const int32_t* expert_offsets, int E, int64_t M_total,
                                   int64_t F, int64_t K, void* y1, void* h, float* amax_out, uint8_t* q_h,
                                   uint8_t* s_h, nvfp4moe_stream_t stream);

/*
 * grouped_gemm_bf16 -- grouped BF16 GEMM, fp32 accumulation (the BF16
 * backward, [JA] first paragraph; also the BF16 baseline of the forward).
 *   NVFP4MOE_NT: a [M_total][K], b [E][N][K] -> c [M_total][N]
 *   NVFP4MOE_NN: a [M_total][K], b [E][K][N] -> c [M_total][N]
 *   NVFP4MOE_TN: a [M_total][K], b [M_total][N] -> c [E][K][N],
 *                c_e = sum over rows r of expert e of a[r]^T b[r]
 *                (an empty expert gives zeros, or leaves c_e unchanged
 *                when accumulating)
 * accumulate = 1 adds into c (F32 output only); 0 overwrites.  Rows of c
 * beyond offsets[E] are not written (NT/NN).  K % 32 == 0 and N % 32 == 0
 * (TN: K % 32 == 0, N % 32 == 0; M_e arbitrary); 16-byte aligned pointers.
 * Operands are read through 32-bit buffer offsets: NN needs K*N*2 < 2^31,
 * TN needs M_total*K*2 and M_total*N*2 < 2^31; M_total, N, K < 2^31 (else
 * ESHAPE).
 * workspace may be NULL.
 */
int grouped_gemm_bf16(int layout, const void* a, const void* b, const int32_t* expert_offsets,
                      int E, int64_t M_total, int64_t N, int64_t K, void* c, int c_dtype,
                      int accumulate, void* workspace, size_t ws_bytes, nvfp4moe_stream_t stream);

/*
 * grouped_gemm_bf16_tn_gather -- the NVFP4MOE_TN weight gradient with B's
 * rows gathered from the unpermuted tokens, so that the permuted copy of
 * the activations (contiguous layout, [JA] fourth paragraph) need not be
 * kept for the BF16 backward ([JA] first paragraph):
 *   c_e = sum over rows r of expert e of a[r]^T b[b_src[r] / k]
 * (rows with b_src[r] < 0 contribute nothing).  With b_src = the src array
 * of moe_permute and b = the [T][N] tokens, this equals NVFP4MOE_TN on the
 * permuted rows bit for bit.
 *   a      [M_total][K] bf16 (permuted rows, e.g. the gradient of Y1).
 *   b      [b_rows][N] bf16 (e.g. the T unpermuted tokens).
 *   b_src  [M_total] int32, device; k >= 1.  b_src[r] / k must be < b_rows
 *          (a larger index reads zeros or other rows of b; never outside it).
 *   c      [E][K][N], F32 or BF16; accumulate as for grouped_gemm_bf16.
 * K % 32 == 0, N % 32 == 0; 16-byte aligned a, b, c; 4-byte aligned b_src;
 * M_total*K*2 and b_rows*N*2 < 2^31 (else ESHAPE).  EINVAL for NULL
 * pointers with work to do, k < 1, negative sizes or a bad dtype.
 */
int grouped_gemm_bf16_tn_gather(const void* a, const void* b, const int32_t* b_src, int k,
                                int64_t b_rows, const int32_t* expert_offsets, int E, int64_t M_total,
                                int64_t N, int64_t K, void* c, int c_dtype, int accumulate,
                                nvfp4moe_stream_t stream);

/*
 * silu_gate_fwd -- H[r][f] = silu(Y1[r][f]) * Y1[r][F+f] (gate half first),
 * fp32 math, bf16 out (RNE), and amax_out[0] = max |H| over the stored bf16
 * values, ready for amax reuse by the next quantization ([JA] fourth
 * paragraph: op fusion, amax reuse).  y1 [R][2F] bf16, h [R][F] bf16,
 * F % 8 == 0.  amax_out may be NULL.
 */
int silu_gate_fwd(const void* y1, int64_t R, int64_t F, void* h, float* amax_out,
                  nvfp4moe_stream_t stream);

/*
 * silu_gate_bwd -- dY1 = [dH*U*silu'(G) | dH*silu(G)], fp32 math, bf16 out.
 * y1 [R][2F] bf16, dh [R][F] bf16, dy1 [R][2F] bf16; F % 8 == 0.
 * amax_out fp32 [1] or NULL: max |dY1| over the stored bf16 values, for the
 * NVFP4 quantization of dY1 that follows (amax reuse, [JA] fourth paragraph).
 */
int silu_gate_bwd(const void* y1, const void* dh, int64_t R, int64_t F, void* dy1, float* amax_out,
                  nvfp4moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4MOE_H */
