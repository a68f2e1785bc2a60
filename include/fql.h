/*
 * fql.h - C ABI of the MI355X (gfx950) NVFP4 W4A4 quantized linear library.
 *
 * The layer (vLLM write-ups "TorchNvFp4LinearKernel", "QUTLASS NVFP4 online
 * transforms", "B12X CuTe-DSL linear backends"): bf16 activations are
 * quantized on the fly to NVFP4 (E2M1 codes, one E4M3 scale per 16 elements
 * along K, one float32 global scale), optionally after a block-diagonal
 * Hadamard rotation; a block-scaled GEMM multiplies them with a pre-packed
 * NVFP4 weight; alpha (the product of the two global dequant scales) and an
 * optional bias are applied and the result is cast to bf16.
 *
 * Conventions shared by every call:
 *  - All tensor pointers are DEVICE pointers unless stated otherwise, owned by
 *    the caller. Outputs are caller-allocated and written in place; no call
 *    allocates device memory (the write-ups' in-place quantize op takes
 *    preallocated outputs for the same reason).
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream). Every
 *    call is stream-ordered and asynchronous: it only enqueues kernels.
 *  - Sizes are element counts; leading dimensions (ld*) are in elements.
 *  - Return value: FQL_OK (0) or a negative FQL_ERR_* code. On error nothing
 *    is launched and fql_last_error() returns a message for the calling
 *    thread. Validation is cheap and host-side only.
 *  - Layouts: activations x [M][ldx] bf16 row-major (ldx >= K, any row
 *    stride: a non-contiguous row slice is consumed without a copy, as the
 *    B12X NVFP4 path requires); codes [rows][K/2] bytes with the even-index
 *    element in the low nibble; scales [rows][K/16] E4M3 bytes, row-major
 *    (the canonical layout; the GEMM's own layout is internal to the packed
 *    weight); y [M][ldy] bf16 row-major, exactly N columns written.
 *  - Numerics of the quantizer: a = max|v| over the 16-block,
 *    s = E4M3_RNE_satfinite(fl32(fl32(a/6)*g)), r = fl32(g/s) (0 if s == 0),
 *    q = E2M1_RNE_satfinite(fl32(v*r)) with the sign of v kept. Codes and
 *    scales are bit-identical to the CPU oracle.
 */
#ifndef FQL_H
#define FQL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FQL_OK 0
#define FQL_ERR_INVALID -1     /* bad argument: shape, stride, pointer, value */
#define FQL_ERR_UNSUPPORTED -2 /* device or configuration not supported */
#define FQL_ERR_HIP -3         /* a HIP runtime call failed */
#define FQL_ERR_WORKSPACE -4   /* workspace too small */

/* Weight/activation formats (fql_can_implement). */
#define FQL_FMT_NVFP4 1
#define FQL_FMT_MXFP4 2
#define FQL_FMT_MXFP8 3
#define FQL_FMT_FP8 4       /* per-tensor FP8 */
#define FQL_FMT_FP8_BLOCK 5 /* block FP8: 1 x 128 activation, 128 x 128 weight groups */

/* Library version (major*10000 + minor*100 + patch). */
int fql_version(void);

/* Message for the last error returned on the calling thread ("" if none). */
const char* fql_last_error(void);

/*
 * Availability check, in the spirit of the write-ups' is_supported(): returns
 * 1 if `device` is a gfx950 GPU this library was built for, else 0, and
 * writes the reason into `reason` (may be NULL) when it is not. Negative on
 * a HIP error.
 */
int fql_is_supported(int device, char* reason, size_t reason_len);

/*
 * Format-level constraints, in the spirit of can_implement(): returns 1 if a
 * layer with these sizes can run, else 0 with the reason. NVFP4 needs
 * K % 16 == 0, N >= 1, K >= 16, and hadamard_block in {0, 16, 32, 64, 128}
 * with K % hadamard_block == 0. MXFP4, MXFP8 and per-tensor FP8 need
 * K % 32 == 0, N >= 1, K >= 32 and hadamard_block == 0. Block FP8 needs N and
 * K multiples of 128 (the B12X write-up's can_implement: activation group
 * (1, 128), weight group (128, 128), 128-aligned features) and
 * hadamard_block == 0. N and K are at most 2^24.
 */
int fql_can_implement(int format, int64_t N, int64_t K, int hadamard_block, char* reason,
                      size_t reason_len);

/*
 * max |v| over x [M][K] (bf16, row stride ldx) after the optional
 * block-diagonal Hadamard rotation (hadamard_block 0 = none), written as one
 * float to `amax_out` (device). The calibration value for the global scale
 * g = 448*6/amax (QUTLASS write-up: the rotation is applied before
 * quantization, so the calibration sees rotated values).
 */
int fql_amax_bf16(const void* x, int64_t M, int64_t K, int64_t ldx, int hadamard_block,
                  float* amax_out, void* stream);

/* Same for float32 input (weights before packing). */
int fql_amax_f32(const float* w, int64_t N, int64_t K, int64_t ldw, int hadamard_block,
                 float* amax_out, void* stream);

/*
 * Activation quantizer (TorchNvFp4LinearKernel apply_weights: the activation
 * is quantized with the layer's input global scale into packed FP4 bytes and
 * block scales; QUTLASS write-up: fused block-diagonal Hadamard + NVFP4
 * quantize into caller-provided code and scale tensors).
 *   x       [M][ldx] bf16, ldx >= K; 16-byte aligned rows are fastest but not
 *           required.
 *   global_scale  g > 0 and finite (the reciprocal of the global dequant scale).
 *   hadamard_block 0 (none) or 16/32/64/128: per b-element chunk of each row,
 *           v = H_b v / sqrt(b) with Sylvester H_b, as a float32 FWHT with
 *           strides 1, 2, ..., b/2 and one multiply by fl32(1/sqrt(b)).
 *   codes   [M][K/2] bytes out; scales [M][K/16] E4M3 bytes out.
 */
int fql_quant_nvfp4(const void* x, int64_t M, int64_t K, int64_t ldx, float global_scale,
                    int hadamard_block, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * Weight quantizer: as fql_quant_nvfp4 but for float32 input w [N][ldw]. With
 * hadamard_block > 0 the weight rows are rotated by the same transform, so
 * x' w'^T = x w^T (the rotation is orthogonal).
 */
int fql_quant_nvfp4_f32(const float* w, int64_t N, int64_t K, int64_t ldw, float global_scale,
                        int hadamard_block, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * Size in bytes of the packed weight for an [N][K] NVFP4 weight (host-side,
 * no device work). The packed blob pads N to a multiple of 16 and K to a
 * multiple of 128 with zeros.
 */
int fql_packed_nvfp4_bytes(int64_t N, int64_t K, size_t* bytes);

/*
 * Weight packer (process_weights_after_loading in the write-ups, which
 * re-lays block scales and pads the weight for their GEMM): re-lays canonical
 * codes [N][K/2] and scales [N][K/16] into the GEMM's operand order. Writes
 * into the caller's buffer `packed` (packed_bytes from
 * fql_packed_nvfp4_bytes), so re-packing a reloaded weight keeps its address
 * (the B12X write-up reuses packed storage so captured graphs stay valid).
 */
int fql_pack_weight_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                          void* packed, size_t packed_bytes, void* stream);

/* Inverse of fql_pack_weight_nvfp4 (packed -> canonical codes and scales). */
int fql_unpack_weight_nvfp4(const void* packed, int64_t N, int64_t K, uint8_t* codes,
                            uint8_t* scales, void* stream);

/*
 * Workspace bytes fql_linear_nvfp4 needs for this shape (host-side). The
 * workspace holds arrival counters (its first 64 KiB), the dequantized
 * activation operand (M > 32) and, for split-K launches, float32 partial
 * sums. The counters must be zero before a workspace's first use (allocate it
 * zero-filled); every call leaves them zero again. Calls that run at the same
 * time (other streams) must not share a workspace.
 */
int fql_linear_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes);

/*
 * Diagnostics: writes a one-line description of the launch plan
 * fql_linear_nvfp4 uses for this shape into `buf` (kernel name, template
 * parameters, grid, splits), e.g. for attributing profiler time. `aligned`
 * is a bit set: bit 0 says whether x rows will be 16-byte aligned; bit 1
 * describes the plan of fql_linear_nvfp4_transform instead (the unaligned
 * plan, with the transform kernel as its quantizer; the dynamic-scale call
 * without a transform plans like an unaligned plain call); bit 2 says that
 * the call rotates the activation (hadamard_block > 0), which can change the
 * column tiles per workgroup of the fused small-M kernel. Host-side only.
 */
int fql_linear_nvfp4_describe(int64_t M, int64_t N, int64_t K, int aligned, char* buf,
                              size_t buf_len);

/*
 * The NVFP4 W4A4 linear layer (TorchNvFp4LinearKernel / B12X NVFP4
 * apply_weights): y = bf16(alpha * (x_q @ w_q^T) + bias), where x_q is x
 * quantized exactly as fql_quant_nvfp4 does with (input_global_scale,
 * hadamard_block), w_q the packed weight, and the sum is accumulated in
 * float32 over exactly dequantized products.
 *   x        [M][ldx] bf16, M >= 1 (M = product of the leading dims).
 *   w_packed from fql_pack_weight_nvfp4 for an [N][K] weight (rotated with
 *            the same hadamard_block if it is > 0).
 *   alpha    float32 scalar: 1 / (g_x * g_w).
 *   bias     [N] bf16 or NULL.
 *   y        [M][ldy] bf16 out, ldy >= N.
 *   workspace/workspace_bytes  device scratch of at least
 *            fql_linear_nvfp4_workspace_bytes(M, N, K).
 */
int fql_linear_nvfp4(const void* x, int64_t M, int64_t K, int64_t ldx, float input_global_scale,
                     int hadamard_block, const void* w_packed, int64_t N, float alpha,
                     const void* bias, void* y, int64_t ldy, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * fql_linear_nvfp4 with alpha read from device memory (one float32 at
 * alpha_dev, 4-byte aligned) instead of passed by value. A layer that keeps
 * its alpha in device memory can re-pack new weights with a different
 * weight global scale into the same storage, update that float in stream
 * order, and replay HIP graphs captured before (the B12X write-up,
 * Implementation: packed weight storage is reused in place so that captured
 * graphs stay valid). Other arguments, the workspace and errors as
 * fql_linear_nvfp4.
 */
int fql_linear_nvfp4_dev_alpha(const void* x, int64_t M, int64_t K, int64_t ldx,
                               float input_global_scale, int hadamard_block, const void* w_packed,
                               int64_t N, const float* alpha_dev, const void* bias, void* y,
                               int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Diagnostics: the two halves of fql_linear_nvfp4, for launch plans that
 * quantize the activation in a pass of their own (every plan but the
 * one-launch small-M kernel and the opt-in in-GEMM quantization; those
 * return FQL_ERR_UNSUPPORTED). fql_linear_nvfp4_quantize writes the GEMM's
 * activation operand into the workspace exactly as fql_linear_nvfp4 does:
 * at byte offset 65536 (after the arrival counters), either x_hat, the
 * exactly dequantized values e2m1(q) * s as float16 in MFMA A-fragment order
 * [Mp/16][Kp/32][64 lanes][8] (lane = kq*16 + m holds row m of the 16-row
 * tile, k = 32*step + 8*kq + 0..7), or the packed activation (the packed
 * weight layout of fql_pack_weight_nvfp4 with Mp rows); Mp and Kp are the
 * row count and K padded with zeros (fql_linear_nvfp4_describe names the
 * form: "xhat" or "apack"). fql_linear_nvfp4_gemm then runs the block-scaled
 * GEMM and the epilogue on that operand; x_aligned says whether x had
 * 16-byte aligned rows (pointer and stride), which selects the same plan.
 * Called in this order on one stream and workspace, the pair computes
 * exactly what one fql_linear_nvfp4 call computes.
 */
int fql_linear_nvfp4_quantize(const void* x, int64_t M, int64_t K, int64_t ldx,
                              float input_global_scale, int hadamard_block, int64_t N,
                              void* workspace, size_t workspace_bytes, void* stream);
int fql_linear_nvfp4_gemm(int64_t M, int64_t K, int x_aligned, const void* w_packed, int64_t N,
                          float alpha, const void* bias, void* y, int64_t ldy, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * The NVFP4 linear layer for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): fql_linear_nvfp4 without a workspace argument. The scratch the
 * call needs (arrival counters, the quantized activation operand, split-K
 * partial sums) lives in a file-scope device array of
 * FQL_NOALLOC_SCRATCH_BYTES bytes on each device, held until the process
 * ends; a call whose launch plan needs more returns FQL_ERR_WORKSPACE and
 * launches nothing. The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine). Every call on a device shares that device's
 * array: calls that overlap in time on one device (other streams, other
 * threads) race; calls in order on one stream do not. Same arguments,
 * launch plan, numerics and errors as fql_linear_nvfp4 otherwise.
 */
#define FQL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fql_linear_nvfp4_noalloc(const void* x, int64_t M, int64_t K, int64_t ldx,
                             float input_global_scale, int hadamard_block, const void* w_packed,
                             int64_t N, float alpha, const void* bias, void* y, int64_t ldy,
                             void* stream);

/* ---------------------------------------------------------------------------
 * Host-side scalars of the layer (no device work, callable without a GPU).
 * ------------------------------------------------------------------------- */

/* NVFP4 activation or weight global scale from a calibration amax
 * (TorchNvFp4LinearKernel: the input global scale is the inverse of the
 * global dequant scale): g = fl32(448 * 6 / amax) (a correctly rounded
 * float32 division), 1 when amax = 0, at most 2^118 (so g divided by the
 * smallest nonzero E4M3 scale 2^-9 stays finite). amax must be finite and
 * >= 0. */
int fql_nvfp4_global_scale(float amax, float* global_scale);

/* NVFP4 alpha, the product of the two global dequant scales
 * (TorchNvFp4LinearKernel apply_weights): fl32((1/g_x) * (1/g_w)) evaluated
 * in double precision and rounded once. Both scales finite and > 0. */
int fql_nvfp4_alpha(float input_global_scale, float weight_global_scale, float* alpha);

/* Per-tensor FP8 calibration scale: fl32(amax / 448), or 1 when that is 0
 * (an all-zero tensor). amax finite and >= 0. */
int fql_fp8_scale(float amax, float* scale);

/* Per-tensor FP8 output scale (B12X write-up: the input and weight scales are
 * merged into one output scale): fl32(input_scale * weight_scale), both
 * finite and > 0. */
int fql_fp8_output_scale(float input_scale, float weight_scale, float* alpha);

/* Benchmarking aid: replace a launch-plan override. which: FQL_PLAN_NVFP4
 * ("kind=K,waves=W,nt=N,st=S,splits=Z,tail=T,..."), FQL_PLAN_SC_GEMM
 * ("wm,wn,mtw,ntw,st[,splits[,tail]]") or FQL_PLAN_SC_GEMV ("W,NT,D[,FQ]",
 * or "0" for no GEMV); spec NULL or "" removes it. tail: 1 keeps the last
 * round of tiles whole, 2..4 splits its tiles that many ways along K. The initial values are the
 * environment variables FQL_PLAN, FQL_SC_PLAN and FQL_SC_GEMV, read once.
 * An override changes which kernel configuration runs, so results may differ
 * in the float32 summation order over K, never otherwise; configurations
 * that are not built are ignored. Host-side only. */
#define FQL_PLAN_NVFP4 0
#define FQL_PLAN_SC_GEMM 1
#define FQL_PLAN_SC_GEMV 2
int fql_set_plan_override(int which, const char* spec);

/* ---------------------------------------------------------------------------
 * General block-diagonal transform and dynamic global scale ("QUTLASS NVFP4
 * online transforms" write-up: the fused quantizer accepts any
 * block-diagonal transform, not only a fixed Hadamard matrix; the matrix is
 * one b x b partition of the layer's input-transform weight with the
 * 1/sqrt(n) normalisation already folded in, b in {16, 32, 64, 128}; its
 * dense branch applies it as a linear layer, v = x @ T^T per chunk).
 *   T   bf16 [b][b] row-major device matrix, 16-byte aligned; K % b == 0.
 *   v[c*b + i] = sum_j T[i][j] * x[c*b + j]  per row, per b-chunk c,
 *       accumulated in float32 on the matrix cores (the products are exact;
 *       the sum's rounding order is the hardware's, so v may differ from the
 *       exactly rounded sum in the last bits, and codes or scales from an
 *       exact evaluation only at near-ties). An exactly zero sum is +0.
 * Then the NVFP4 quantizer of fql_quant_nvfp4 on v. The dynamic variants
 * compute g = fl32(2688 / amax) over the whole transformed activation on
 * the device (1 when amax = 0, at most 2^118, which keeps g / s finite for
 * every nonzero E4M3 scale s), so no host synchronisation is needed.
 * ------------------------------------------------------------------------- */

/* The transform alone: bf16 x [M][ldx] -> float32 v [M][ldv] (16-byte
 * aligned, ldv >= K, ldv % 4 == 0). */
int fql_transform_bf16(const void* x, int64_t M, int64_t K, int64_t ldx, const void* T, int b,
                       float* v, int64_t ldv, void* stream);

/* Transform + NVFP4 quantize with a static global scale: codes [M][K/2]
 * (8-byte aligned), scales [M][K/16] E4M3, as fql_quant_nvfp4. */
int fql_quant_nvfp4_transform(const void* x, int64_t M, int64_t K, int64_t ldx,
                              float global_scale, const void* T, int b, uint8_t* codes,
                              uint8_t* scales, void* stream);

/* NVFP4 quantize with the dynamic global scale. T may be NULL: then b is a
 * Hadamard block (0 = no rotation) as in fql_quant_nvfp4. scalars: device
 * float32 [FQL_DYNAMIC_SCALARS] (4-byte aligned); words 0..63 are partial
 * maxima (scratch), word 64 receives amax and word 65 g. Four kernels on the
 * stream (clear, amax, scale, quantize); a call on the same buffer before
 * the previous one has finished races. */
#define FQL_DYNAMIC_SCALARS 68
int fql_quant_nvfp4_dynamic(const void* x, int64_t M, int64_t K, int64_t ldx, const void* T, int b,
                            float* scalars, uint8_t* codes, uint8_t* scales, void* stream);

/* fql_linear_nvfp4 with the transform T (b x b) in place of the Hadamard
 * rotation; the packed weight must come from a weight transformed alike.
 * Same arguments, layouts and workspace as fql_linear_nvfp4. */
int fql_linear_nvfp4_transform(const void* x, int64_t M, int64_t K, int64_t ldx,
                               float input_global_scale, const void* T, int b,
                               const void* w_packed, int64_t N, float alpha, const void* bias,
                               void* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                               void* stream);

/* fql_linear_nvfp4 with the dynamic activation global scale: g_x from this
 * call's activation (after T, or the Hadamard block b when T is NULL) and
 * alpha = fl32((1/g_x) * (1/weight_global_scale)) in float64, both on the
 * device (kept in the workspace's reserved scalar slots, so concurrent calls
 * need separate workspaces, as for every linear call). */
int fql_linear_nvfp4_dynamic(const void* x, int64_t M, int64_t K, int64_t ldx, const void* T,
                             int b, const void* w_packed, int64_t N, float weight_global_scale,
                             const void* bias, void* y, int64_t ldy, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * MXFP4 (B12X write-up, Implementation: the MXFP4 linear kernel accepts only a
 * dynamically quantized activation; element and scale formats per OCP
 * Microscaling v1.0): E2M1 codes with one E8M0 scale byte per 32 consecutive
 * elements along K, no global scale, no rotation.
 * Quantizer numerics, per 32-block: a = max|v|; E = floor(log2 a) - 2
 * clamped to [-127, 127] (a = 0 gives -127); scale byte E + 127;
 * q = E2M1_RNE_satfinite(fl32(v * 2^-E)) with the sign of v kept. The block
 * maximum lands in [4, 8), so values in (6, 8) * 2^E saturate to 6 * 2^E.
 * Codes [rows][K/2] (even element in the low nibble) and scales [rows][K/32]
 * are bit-identical to the CPU oracle.
 * ------------------------------------------------------------------------- */

/* Activation quantizer: bf16 x [M][ldx] (ldx >= K, K % 32 == 0) -> codes
 * [M][K/2] (4-byte aligned) and scales [M][K/32]. */
int fql_quant_mxfp4(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                    uint8_t* scales, void* stream);

/* Same for float32 input (weights before packing). */
int fql_quant_mxfp4_f32(const float* w, int64_t N, int64_t K, int64_t ldw, uint8_t* codes,
                        uint8_t* scales, void* stream);

/* Size in bytes of the packed MXFP4 weight for [N][K] (host-side). The blob
 * pads N to a multiple of 16 and K to a multiple of 128 with zero codes and
 * zero scale bytes. */
int fql_packed_mxfp4_bytes(int64_t N, int64_t K, size_t* bytes);

/* Weight packer (process_weights_after_loading): canonical codes [N][K/2]
 * (16-byte aligned) and scales [N][K/32] -> the scaled-MFMA operand order, in
 * the caller's 16-byte aligned buffer of at least fql_packed_mxfp4_bytes. */
int fql_pack_weight_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                          void* packed, size_t packed_bytes, void* stream);

/* Workspace bytes fql_linear_mxfp4 needs (host-side): arrival counters (first
 * 64 KiB, zero before first use and left zero by every call), the quantized
 * activation operand and split-K partial sums. */
int fql_linear_mxfp4_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes);

/* One-line description of the launch plan of fql_linear_mxfp4 (host-side). */
int fql_linear_mxfp4_describe(int64_t M, int64_t N, int64_t K, char* buf, size_t buf_len);

/*
 * The MXFP4 W4A4 linear layer (B12X MXFP4 apply_weights: dynamic activation
 * quantize, then the block-scaled GEMM): y = bf16(alpha * (x_q @ w_q^T) + bias)
 * with x_q quantized exactly as fql_quant_mxfp4 does and the products of
 * dequantized values accumulated in float32 by the scaled matrix cores.
 *   x        [M][ldx] bf16 (any alignment), K % 32 == 0.
 *   w_packed from fql_pack_weight_mxfp4 for [N][K].
 *   alpha    float32 output scale (1 for a plain MXFP4 layer).
 *   bias     [N] bf16 or NULL.   y [M][ldy] bf16 out, ldy >= N.
 *   workspace  at least fql_linear_mxfp4_workspace_bytes(M, N, K), 256-byte
 *            aligned; one workspace per stream at a time.
 */
int fql_linear_mxfp4(const void* x, int64_t M, int64_t K, int64_t ldx, const void* w_packed,
                     int64_t N, float alpha, const void* bias, void* y, int64_t ldy,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * MXFP8 (B12X write-up, Implementation: the MXFP8 linear kernel; OCP
 * Microscaling v1.0): E4M3 codes with one E8M0 scale byte per 32 elements
 * along K. Quantizer per 32-block: E = floor(log2 max|v|) - 8 clamped to
 * [-127, 127] (all-zero block: -127), scale byte E + 127,
 * q = E4M3_RNE_satfinite(fl32(v * 2^-E)). Codes [rows][K] (one byte per
 * element), scales [rows][K/32]. Same conventions as the MXFP4 calls.
 * ------------------------------------------------------------------------- */
int fql_quant_mxfp8(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                    uint8_t* scales, void* stream);
int fql_quant_mxfp8_f32(const float* w, int64_t N, int64_t K, int64_t ldw, uint8_t* codes,
                        uint8_t* scales, void* stream);
int fql_packed_mxfp8_bytes(int64_t N, int64_t K, size_t* bytes);
int fql_pack_weight_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                          void* packed, size_t packed_bytes, void* stream);
int fql_linear_mxfp8_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes);
int fql_linear_mxfp8_describe(int64_t M, int64_t N, int64_t K, char* buf, size_t buf_len);
/* y = bf16(alpha * (x_q @ w_q^T) + bias) with x quantized as fql_quant_mxfp8;
 * arguments as fql_linear_mxfp4. */
int fql_linear_mxfp8(const void* x, int64_t M, int64_t K, int64_t ldx, const void* w_packed,
                     int64_t N, float alpha, const void* bias, void* y, int64_t ldy,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Per-tensor FP8 (B12X write-up, Implementation: the per-tensor FP8 kernel
 * quantizes the activation with a static per-tensor scale, packs the weight
 * ahead of time and merges the input and weight scales into one output
 * scale). q = E4M3_RNE_satfinite(fl32(v * fl32(1 / scale))), scale > 0
 * (calibration: fl32(amax / 448), amax from fql_amax_bf16 / fql_amax_f32).
 * Codes [rows][K], K % 32 == 0.
 * ------------------------------------------------------------------------- */
int fql_quant_fp8(const void* x, int64_t M, int64_t K, int64_t ldx, float scale, uint8_t* codes,
                  void* stream);
int fql_quant_fp8_f32(const float* w, int64_t N, int64_t K, int64_t ldw, float scale,
                      uint8_t* codes, void* stream);
int fql_packed_fp8_bytes(int64_t N, int64_t K, size_t* bytes);
/* codes [N][K] (16-byte aligned) -> packed operand order. */
int fql_pack_weight_fp8(const uint8_t* codes, int64_t N, int64_t K, void* packed,
                        size_t packed_bytes, void* stream);
int fql_linear_fp8_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes);
int fql_linear_fp8_describe(int64_t M, int64_t N, int64_t K, char* buf, size_t buf_len);
/* y = bf16(alpha * (x_q @ w_q^T) + bias): x_q = fql_quant_fp8(x, input_scale),
 * alpha = fl32(input_scale * weight_scale) (the merged output scale). */
int fql_linear_fp8(const void* x, int64_t M, int64_t K, int64_t ldx, float input_scale,
                   const void* w_packed, int64_t N, float alpha, const void* bias, void* y,
                   int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);
/* fql_linear_fp8 with the output scale read from device memory (one float32
 * at alpha_dev, 4-byte aligned), so a weight re-packed with a new weight
 * scale only updates that float and captured graphs stay valid. */
int fql_linear_fp8_dev_alpha(const void* x, int64_t M, int64_t K, int64_t ldx, float input_scale,
                             const void* w_packed, int64_t N, const float* alpha_dev,
                             const void* bias, void* y, int64_t ldy, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Block FP8 (B12X write-up, Implementation: the block FP8 kernel: activation
 * group (1, 128), weight group (128, 128), 128-aligned features, float32
 * scales; UE8M0 weight scales are widened to float32 by the caller).
 * Per group: s = fl32(max|v| / 448), q = E4M3_RNE_satfinite(fl32(v * fl32(1/s)))
 * (s = 0: q = 0). Activation: codes [M][K], scales float [M][K/128].
 * Weight: codes [N][K], scales float [N/128][K/128]. The GEMM adds every
 * 128-deep partial product times s_x[m][kb] * s_w[nb][kb] in float32.
 * ------------------------------------------------------------------------- */
int fql_quant_fp8_block(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                        float* scales, void* stream);
int fql_quant_fp8_block_weight_f32(const float* w, int64_t N, int64_t K, int64_t ldw,
                                   uint8_t* codes, float* scales, void* stream);
int fql_packed_fp8_block_bytes(int64_t N, int64_t K, size_t* bytes);
int fql_pack_weight_fp8_block(const uint8_t* codes, const float* scales, int64_t N, int64_t K,
                              void* packed, size_t packed_bytes, void* stream);
int fql_linear_fp8_block_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes);
int fql_linear_fp8_block_describe(int64_t M, int64_t N, int64_t K, char* buf, size_t buf_len);
/* y = bf16(alpha * sum_kb s_x s_w (x_q @ w_q^T)_kb + bias), alpha normally 1. */
int fql_linear_fp8_block(const void* x, int64_t M, int64_t K, int64_t ldx, const void* w_packed,
                         int64_t N, float alpha, const void* bias, void* y, int64_t ldy,
                         void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FQL_H */
