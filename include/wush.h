/*
 * wush.h -- C ABI of the WUSH online activation path on AMD Instinct MI355X
 * (gfx950).
 *
 * The operation comes from "WUSH: Near-Optimal Adaptive Transforms for LLM
 * Quantization" (arXiv 2512.00956).  Each token's activation row is cut into
 * blocks of G contiguous channels.  Each block is multiplied by its own G x G
 * matrix T_wush(c) = H S^-1/2 U^T W'^T, built offline (Eq. 8; deep dive,
 * section 3.4.4).  The result is quantized round-to-nearest with an AbsMax
 * scale per group of G (deep dive, sections 3.4.6 and 3.4.7; Eq. 10).  The
 * transform and the quantization run in one kernel pass, so the transformed
 * activations never go to memory (deep dive, section 3.4.7, "QuTLASS
 * baseline" paragraph).
 *
 * Conventions for every entry point:
 *   - Every buffer is a DEVICE pointer on the current HIP device, allocated
 *     and owned by the caller.  The library allocates no memory, keeps no
 *     state that changes between calls, and is thread-safe.
 *   - Work is enqueued on `stream` (0 = the null stream) and the call
 *     returns without synchronizing.  Results are visible to later work on
 *     that stream.
 *   - Arguments are validated before any HIP call.  If validation fails,
 *     nothing is launched and the matching error code is returned;
 *     wush_last_error() then holds a message, per thread.
 *   - M == 0 is a valid no-op that returns WUSH_OK.
 *   - Inputs must be finite.  NaN and Inf inputs are outside the contract.
 *   - Device faults surface at the caller's next synchronization, not here.
 *
 * Layouts (all row-major):
 *   X       bf16 [M][K].  Token m, channel k at X[m*K + k].  16-byte aligned.
 *   T       bf16 [K/G][G][G].  T[c][i][j] multiplies x_(cG+j) into output i of
 *           block c, so block c's matrix is one contiguous G*G slice.
 *           16-byte aligned.
 *   codes   uint8 [M][K/2].  Element 2j in bits 3:0 of byte j, element 2j+1
 *           in bits 7:4.  16-byte aligned.
 *   scales  one per (token, block), [M][K/G].  The format decides the type
 *           and the alignment (8 bytes for MXFP4, 16 for NVFP4 and INT4).
 *   The kernels write codes and scales with 16- and 8-byte vector stores,
 *   which these alignments keep on natural boundaries.
 *
 * Pre-quantization values: y = fp32 rounding of the exact sum
 * sum_j T[c][i][j] * x_j.  The kernels use fp32 matrix-core accumulation,
 * which can differ from the exact sum by an error bounded by the sum of
 * |T x| terms.  Any group whose scale decision falls within that bound of
 * a rounding boundary gets its exact AbsMax: each output that can hold the
 * maximum (within twice the bound of the largest matrix-core value) is
 * recomputed from its G products (each exact in float64), summed in
 * float64 and rounded once to fp32.  That sum is exact when the products
 * span at most 32 binary octaves; beyond that its error stays below 2^-47
 * of the sum of |T x| terms, so the recomputed y can differ from the
 * exactly rounded one only if the exact sum lies that close to an fp32
 * rounding midpoint.  With that proviso every scale equals the one
 * computed from the exactly rounded y.  An element code may still differ
 * by one level where the scaled value sits within the accumulation bound
 * of a rounding midpoint.
 */
#ifndef WUSH_H_
#define WUSH_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WUSH_ABI_VERSION 2

typedef enum wush_status {
  WUSH_OK = 0,
  WUSH_EINVAL = 1,       /* bad size, null pointer or overlapping buffers   */
  WUSH_EALIGN = 2,       /* a pointer does not meet its alignment           */
  WUSH_EUNSUPPORTED = 3, /* current device is not gfx950, or bad G/format   */
  WUSH_EHIP = 4          /* HIP runtime error (launch or device query)      */
} wush_status;

/* MXFP4 (G = 32).  E2M1 codes, rounded to nearest even with saturation at 6.
 * One E8M0 scale byte per 32: code = e + 127, where e = floor(log2 amax) - 2
 * clamped to [-127, 127], and amax = 0 gives code 0.  Elements are y * 2^-e.
 * MXFP4 is E2M1 elements with a shared 8-bit scale per 32 (deep dive,
 * section 2, "New block-level floating-point formats"; OCP MX v1.0).
 * scales: uint8 [M][K/32], 8-byte aligned.  K must be a multiple of 32. */
wush_status wush_quant_mxfp4(const void* X, const void* T, int64_t M, int64_t K,
                             void* codes, void* scales, hipStream_t stream);

/* wush_quant_mxfp4 with its codes and scales written in the packed operand
 * layout of wush_gemm_mxfp4_packed (the layout wush_gemm_pack_b describes,
 * over M rows): per 128-row tile and 256-element K step, 16 KB of codes and
 * 1 KB of scales in the order the GEMM kernel stages them.  The same codes
 * and scales, bit for bit, only placed differently; each workgroup's 32 rows
 * become 4 KB and 256 B of contiguous memory.  Rows past M in the last tile
 * are not written (the GEMM computes them but never stores them).  An
 * interface of this library: the pages leave the layout open.
 * K must be a multiple of 256.  packed_codes: Mp * K/2 bytes, 16-byte
 * aligned; packed_scales: Mp * K/32 bytes, 8-byte aligned; Mp = M rounded up
 * to a multiple of 128. */
wush_status wush_quant_mxfp4_packed(const void* X, const void* T, int64_t M, int64_t K,
                                    void* packed_codes, void* packed_scales, hipStream_t stream);

/* NVFP4 (G = 16).  E2M1 codes.  One OCP E4M3FN scale byte per 16, relative to
 * a per-tensor fp32 scale g read from device memory at `global_scale`:
 *   code = E4M3_rne_sat(fp32(fp32(amax/6) / g)),  eff = E4M3(code) * g,
 *   elements = y * fp32(1/eff).
 * If g == 0 or eff == 0, the group's codes are all zero.  Pass the g from
 * wush_nvfp4_global_scale (dynamic) or a calibrated constant (static).  g
 * must be 0 or at least 2^-100.  NVFP4 is E2M1 with an FP8 scale per 16 (deep
 * dive, section 2).  The pages do not say how g is chosen; this interface
 * takes it from device memory, so it can be dynamic or calibrated.
 * scales: uint8 [M][K/16], 16-byte aligned.  K must be a multiple of 16. */
wush_status wush_quant_nvfp4(const void* X, const void* T, int64_t M, int64_t K,
                             const float* global_scale, void* codes, void* scales,
                             hipStream_t stream);

/* INT4 (G = 32).  Symmetric levels -7..7, stored as two's-complement nibbles.
 * One IEEE fp16 scale per 32: s = fp16(fp32(amax / 7)).  Elements are
 * rne(clamp(y * fp32(1/s), -7, 7)), and s == 0 gives zero codes.  This is
 * the AbsMax INT quantizer (deep dive, section 3.4.5).
 * scales: fp16 bits [M][K/32], 16-byte aligned.  K must be a multiple of 32. */
wush_status wush_quant_int4(const void* X, const void* T, int64_t M, int64_t K,
                            void* codes, void* scales, hipStream_t stream);

/* Generic form of the three entry points above (an interface of this
 * library; the pages define no API).
 * fmt: 0 = MXFP4, 1 = NVFP4, 2 = INT4.
 * global_scale: used only for NVFP4.
 * n_exact: if non-null, a device uint32 to which the kernel atomically adds
 * the number of token panels (32 channels of one token: one group, or two
 * for NVFP4) with a group that took the exact step.  The caller zeroes it. */
wush_status wush_quant(int fmt, const void* X, const void* T, int64_t M, int64_t K,
                       const float* global_scale, void* codes, void* scales,
                       uint32_t* n_exact, hipStream_t stream);

/* Output element type of wush_gemm_mxfp4. */
typedef enum { WUSH_OUT_F32 = 0, WUSH_OUT_BF16 = 1 } wush_out_type;

/* MXFP4 GEMM: the FP4 matrix multiplication of the inference forward pass
 * ("WUSH: Near-Optimal Adaptive Transforms for LLM Quantization", deep dive,
 * section 3.4.6, Eq. 10).  With a and b the values that wush_quant_mxfp4
 * encodes (E2M1 codes times the block's E8M0 scale),
 *     C[m][n] = sum_k a[m][k] * b[n][k],
 * accumulated in fp32 on the matrix cores.
 *   a_codes:  u8 [M][K/2], a_scales: u8 [M][K/32]   (activations, e.g. the
 *             quantized transform of a token batch)
 *   b_codes:  u8 [N][K/2], b_scales: u8 [N][K/32]   (weights, quantized
 *             offline with the weight-side transform)
 *   C:        [M][N], fp32 or bf16 (round to nearest even), row-major.
 * Requires K > 0 and K % 256 == 0; M, N >= 0 (0 is a no-op).  All pointers
 * are device pointers owned by the caller; codes must be 16-byte aligned,
 * scales 8-byte aligned, C 4-byte aligned, and C must not overlap an input.
 * Errors as for wush_quant. */
wush_status wush_gemm_mxfp4(const void* a_codes, const void* a_scales, const void* b_codes,
                            const void* b_scales, int64_t M, int64_t N, int64_t K, void* C,
                            int out_type, hipStream_t stream);

/* Packed weights for wush_gemm_mxfp4_packed.  The pages pre-quantize the
 * weights offline (deep dive, section 3.4.6, Eq. 10); this library's GEMM can
 * also take them re-laid once, offline, in the order its kernel stages them,
 * so that every weight copy of the GEMM reads whole contiguous blocks.  The
 * pages define no such layout; it is an interface of this library.
 *   in:  b_codes u8 [N][K/2] (16-byte aligned), b_scales u8 [N][K/32]
 *        (8-byte aligned): the wush_quant_mxfp4 layout.
 *   out: packed_codes, Np * K/2 bytes (16-byte aligned), and packed_scales,
 *        Np * K/32 bytes (8-byte aligned), with Np = N rounded up to a
 *        multiple of 128.  Per 128-row tile t and 256-element K step s, in
 *        order of t then s: 16 KB of codes (row r, 16-byte chunk c at byte
 *        1024 (r / 8) + 16 (8 (r % 8) + (c ^ ((r / 2) % 8)))) and then, in
 *        the scale buffer, 1 KB of scales (row r at byte 8 r).  Rows past N
 *        repeat row N - 1.
 * K must be a positive multiple of 256; N >= 0 (0 is a no-op).  The outputs
 * must not overlap the inputs or each other.  Errors as for wush_quant. */
wush_status wush_gemm_pack_b(const void* b_codes, const void* b_scales, int64_t N, int64_t K,
                             void* packed_codes, void* packed_scales, hipStream_t stream);

/* wush_gemm_mxfp4 with B in the wush_gemm_pack_b layout (N the unpadded row
 * count).  a_packed = 0: A as wush_quant_mxfp4 writes it; a_packed = 1: A in
 * the same packed layout over M rows, as wush_quant_mxfp4_packed writes it
 * (buffers of Mp * K/2 and Mp * K/32 bytes, Mp = M rounded up to 128).
 * Otherwise the same arguments, requirements and result, bit for bit. */
wush_status wush_gemm_mxfp4_packed(const void* a_codes, const void* a_scales, int a_packed,
                                   const void* b_packed_codes, const void* b_packed_scales, int64_t M, int64_t N,
                                   int64_t K, void* C, int out_type, hipStream_t stream);

/* Dequantization: out[m][k] = the value code k of row m stands for,
 *   MXFP4  e2m1(code) * 2^(scale - 127)                  (G = 32)
 *   NVFP4  e2m1(code) * fp32(E4M3(scale) * g)            (G = 16)
 *   INT4   code * fp16(scale)                            (G = 32)
 * with codes and scales in the layouts the quantizers write.  This gives
 * the quantized operands of the layerwise loss of Eq. 5 ("WUSH", deep dive,
 * section 3.4.1): (d_out d_batch)^-1 ||q(T_W W)^T q(T_X X) - W^T X||_F^2.
 *   fmt: 0 = MXFP4, 1 = NVFP4, 2 = INT4.  global_scale: device fp32, NVFP4 only.
 *   out: fp32 [M][K], 16-byte aligned, must not overlap the inputs.
 * K must be a positive multiple of 32 (MXFP4, INT4) or 16 (NVFP4); codes
 * 8-byte aligned.  Errors as for wush_quant. */
wush_status wush_dequant(int fmt, const void* codes, const void* scales, const float* global_scale, int64_t M,
                         int64_t K, float* out, hipStream_t stream);

/* Offline construction of the transforms, on the GPU in float64 ("WUSH",
 * Eq. 7 and Eq. 8; deep dive, sections 3.2 and 3.4.2-3.4.4).  For every
 * block c of G input channels:
 *   Sigma_w = W_c^T W_c / d_out,  Sigma_x = X_c^T X_c / n_cal   (uncentered)
 *   each + damp * mean(diag) * I;  W', X' = lower Cholesky factors
 *   W'^T X' = U S V^T (singular values descending; each (u_k, v_k) signed so
 *   that v_k's largest-magnitude entry is positive, ties to the lowest index)
 *   T_wush = H S^-1/2 U^T W'^T,  T_xvsh = H S^-1/2 V^T X'^T
 * with H the Sylvester Hadamard matrix / sqrt(G) (use_hadamard = 1) or I
 * (use_hadamard = 0, the WUS variant).
 *   W: bf16 [d_out][d_in] (nn.Linear order); Xcal: bf16 [n_cal][d_in];
 *   both 16-byte aligned.  G is 16 or 32 and divides d_in; d_out, n_cal >= 1.
 *   T_wush, T_xvsh: float64 [d_in/G][G][G], 8-byte aligned.
 *   T_wush_bf16, T_xvsh_bf16: optional (may be NULL) bf16(fp32(T)) copies in
 *   the kernel layout, 2-byte aligned.
 *   damp: the relative damping (>= 0; 1e-6 is the reading used elsewhere).
 * A block whose damped moments are not positive definite (for example all
 * zero with damp = 0) yields NaN entries.  Errors as for wush_quant. */
wush_status wush_build_transforms(const void* W, int64_t d_out, const void* Xcal, int64_t n_cal, int64_t d_in,
                                  int G, double damp, int use_hadamard, double* T_wush, double* T_xvsh,
                                  void* T_wush_bf16, void* T_xvsh_bf16, hipStream_t stream);

/* Intra-block GPTQ step of GPTQ-WUSH ("WUSH", deep dive, section 3.4.6,
 * Algorithm 1, the GPTQ branch).  One block of transformed weights,
 *   Wbar: float64 [G][d_out]   (row j = transformed input coordinate j)
 *   R:    float64 [G][G], the upper Cholesky factor of the inverse block
 *         Hessian (H S H^T)^-1 (R = I gives round-to-nearest),
 * is quantized column by column: each output channel o is one group of G
 * values whose scale comes from their AbsMax (MXFP4: E8M0 code
 * floor(log2 amax) - 2 + 127; INT4: fp16(fp32(amax) / 7)); for j = 0..G-1,
 * w_j is quantized at that scale (E2M1 nearest even with saturation, or
 * INT4 nearest even clamped to +-7) and the error err = (w_j - q_j) / R[j][j]
 * is spread as w_k -= R[j][k] err for k > j.
 *   fmt: 0 = MXFP4, 2 = INT4.  G: 16 or 32.
 *   Q: float64 [G][d_out], the dequantized values.
 *   codes: row o (G/2 bytes, element 2j in the low nibble) at codes + o *
 *          codes_stride bytes; 4-byte aligned rows.
 *   scales: E8M0 byte (MXFP4) or fp16 bits (INT4) of row o at element
 *           o * scales_stride.
 * Wbar, R, Q 8-byte aligned; outputs must not overlap inputs.  Errors as for
 * wush_quant. */
wush_status wush_gptq_block(int fmt, const double* Wbar, const double* R, int G, int64_t d_out, double* Q,
                            void* codes, int64_t codes_stride, void* scales, int64_t scales_stride,
                            hipStream_t stream);

/* GPTQ-WUSH, the whole of Algorithm 1 for one layer ("WUSH", deep dive,
 * section 3.4.6, "GPTQ Integration (Algorithm 1)"), in float64 on the device:
 *   1. Hx = Xcal^T Xcal / n_cal + damp * mean(diag) * I;  X' = its lower
 *      Cholesky factor.
 *   2. Y = W X'.
 *   3. For blocks b = d_in/G - 1 down to 0 (columns [bG, bG + G)):
 *        Y_b = U S V^T (thin SVD; singular values descending; each (u_k, v_k)
 *        signed so that v_k's largest-magnitude entry is positive, ties to
 *        the lowest index);  S <- S / sqrt(d_out);
 *        T_x[b] = H S^1/2 V^T X'[b,b]^-1           (activation transform);
 *        Wbar   = sqrt(d_out) H S^1/2 U^T            ([G][d_out]);
 *        each output channel's G values of Wbar are one group, quantized
 *        as in wush_gptq_block with R the upper Cholesky factor of
 *        (H S H^T)^-1 (use_gptq != 0) or R = I (round-to-nearest);
 *        Y[:, < bG] -= Wsub^T T_x[b] X'[b, < bG], Wsub = the quantized
 *        block (GPTQ) or Wbar (round-to-nearest).
 *      H is the Sylvester Hadamard matrix / sqrt(G).
 *   fmt: 0 = MXFP4, 2 = INT4.  G: 16 or 32, dividing d_in.  d_out >= G,
 *   n_cal >= 1.  damp >= 0 (the relative damping; 0.01 is GPTQ's customary
 *   value).
 *   Inputs:  W float64 [d_out][d_in] (nn.Linear order); Xcal float64
 *            [n_cal][d_in].
 *   Outputs: Xp  float64 [d_in][d_in], the lower factor X' (zero above the
 *                diagonal);
 *            Y   float64 [d_out][d_in], column block b = the target block b
 *                was fitted to (W X' less the updates of blocks above b);
 *            T_x float64 [d_in/G][G][G]; Wq float64 [d_out][d_in], the
 *                dequantized weights (block b in columns b);
 *            codes u8 [d_out][d_in/2] (4-byte aligned), scales [d_out][d_in/G]
 *                (E8M0 bytes, or fp16 bits 2-byte aligned): the layout
 *                wush_gemm_mxfp4 and wush_dequant read.
 *   Float64 arrays 8-byte aligned; outputs must not overlap inputs or each
 *   other.  A Hessian that is not positive definite after damping, or (with
 *   use_gptq) a block whose target Y_b has a zero singular value, yields
 *   NaN.  Errors as for wush_quant. */
wush_status wush_gptq_wush(int fmt, const double* W, const double* Xcal, int64_t d_out, int64_t n_cal, int64_t d_in,
                           int G, double damp, int use_gptq, double* Xp, double* Y, double* T_x, double* Wq,
                           void* codes, void* scales, hipStream_t stream);

/* Transform only: Y[m][cG+i] = sum_j T[c][i][j] x_(cG+j), in fp32 from the
 * matrix cores, without rounding fix-up.  G is 16 or 32.  Use it to check
 * values before quantization, or when the transformed activations are wanted
 * in fp32.  The product is the block transform of Eq. 8 applied to the
 * activations (deep dive, section 3.4.4); the pages define no such entry,
 * since their kernel never writes the transformed values out.
 * Y: fp32 [M][K], 16-byte aligned. */
wush_status wush_transform_f32(const void* X, const void* T, int64_t M, int64_t K, int G,
                               float* Y, hipStream_t stream);

/* Largest |y| over the whole transformed tensor, where y is the exactly
 * rounded fp32 value of each output (the same y the quantizers' scales
 * use).  The pass bounds every matrix-core value by its accumulation
 * error and recomputes, in float64, only the tokens that can hold the
 * maximum, so the result is the maximum of the recomputed values.
 * The pages do not define this entry: it serves the NVFP4 per-tensor scale,
 * which they leave open (see wush_nvfp4_global_scale).
 * *amax is overwritten, not accumulated: the call enqueues a fill of *amax
 * with 0, then the pass, which folds each workgroup's maximum in with an
 * atomic max.  Two calls that share `amax` on different streams race.
 * G is 16 or 32.  amax: device fp32, 4-byte aligned. */
wush_status wush_absmax_transformed(const void* X, const void* T, int64_t M, int64_t K, int G,
                                    float* amax, hipStream_t stream);

/* NVFP4 per-tensor scale: *global_scale = fp32(absmax(T x) / 2688), with
 * 2688 = 6 * 448 and absmax from wush_absmax_transformed (G = 16).  The
 * block holding the tensor maximum then gets the largest E4M3 scale.  The
 * pages name NVFP4's FP8 block scale but not its tensor scale; this
 * dynamic AbsMax rule is this library's reading. */
wush_status wush_nvfp4_global_scale(const void* X, const void* T, int64_t M, int64_t K,
                                    float* global_scale, hipStream_t stream);

/* The E2M1 element rounding the kernels use, exposed for exhaustive testing:
 * codes[i] = E2M1_rne_sat(v[i]), one 4-bit code per byte, sign in bit 3.
 * n >= 0.  v is fp32, 4-byte aligned.  A test interface of this library:
 * the pages name the E2M1 element format (deep dive, section 2) but define
 * no entry point. */
wush_status wush_e2m1_encode(const float* v, int64_t n, uint8_t* codes, hipStream_t stream);

/* Fixed transform banks, the data-agnostic comparators the pages evaluate
 * through the same quantizer (deep dive, section 5: RTN with no transform,
 * and RTN-H, the blockwise Hadamard transform):
 *   kind 0: T[c] = I;  kind 1: T[c] = H / sqrt(G), H the Sylvester Hadamard
 *   matrix (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]), for c < C.
 * G is 16 or 32; C >= 0 (0 is a no-op).  Outputs (either may be NULL, not
 * both): T float64 [C][G][G], 8-byte aligned; T_bf16 bf16 [C][G][G] in the
 * kernel layout (bf16 of fp32 of the value), 16-byte aligned. */
wush_status wush_fixed_transforms(int kind, int64_t C, int G, double* T, void* T_bf16, hipStream_t stream);

/* The kernel layout of a float64 transform bank: dst[i] = bf16(fp32(src[i]))
 * (both roundings to nearest even), the 16-bit storage of T the pages
 * describe (ai.info summary: transforms kept in 16 bits; deep dive,
 * section 3.4.7: BF16 or FP16 transform matrices).  n >= 0; src 8-byte
 * aligned, dst 2-byte aligned; they must not overlap. */
wush_status wush_f64_to_bf16(const double* src, int64_t n, void* dst, hipStream_t stream);

/* Status text, and the detail of the last failure on this thread.  Library
 * interfaces; nothing on the pages corresponds. */
const char* wush_status_string(wush_status status);
const char* wush_last_error(void);
int wush_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WUSH_H_ */
