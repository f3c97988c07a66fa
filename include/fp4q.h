/*
 * fp4q.h -- C ABI of libfp4q: block-scaled 4-bit (NVFP4 / MXFP4) W4A4 linear
 * layer and looped Sigma-Delta weight re-quantization on AMD Instinct MI355X
 * (gfx950, CDNA4).
 *
 * Sources (page titles; the section, box or step that defines each call is
 * named at the call):
 *   [LQ]   "Looped Transformer quantization: error propagation, NVFP4 and
 *          Sigma-Delta modulation" (mer.dev, loopquant-fp4)
 *   [GDN]  "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for the
 *          Recurrent Half of a Hybrid 27B LLM" (paper 2609.04098)
 *   [MQ]   "MACaQ: Fast, Model Agnostic Calibrated Quantization for
 *          Low-Precision Weights and Activations" (paper 2611.10649)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every data pointer is a DEVICE pointer (memory of the current HIP
 *    device) unless the comment says "host".  `stream` is a hipStream_t
 *    passed as void* (NULL = the default stream).
 *  - The caller owns and allocates every buffer; the library never
 *    allocates, frees or synchronizes.  Every call validates its arguments
 *    on the host, then enqueues its kernels on `stream` and returns; results
 *    are valid once the stream has reached that point.
 *  - Matrices are row-major with the reduction / block axis (cols, K)
 *    contiguous.  `ld*` arguments are row strides in ELEMENTS of the input
 *    type.  Outputs written by the library are dense: packed codes are
 *    [rows][cols/2] bytes, element 2j in the low nibble of byte j and
 *    element 2j+1 in the high nibble; NVFP4 block scales are [rows][cols/16]
 *    E4M3 bytes; MXFP4 block scales are [rows][cols/32] E8M0 bytes.
 *  - Weights are stored [N][K] (out features x in features); GEMMs compute
 *    Y[M][N] = A[M][K] * B[N][K]^T with fp32 accumulation and fp32 output.
 *  - Non-finite inputs are outside the contract (results unspecified, no
 *    fault).
 *  - Return value: FP4Q_OK or an error status; on error nothing was
 *    enqueued.  fp4q_last_error() returns a thread-local description of the
 *    most recent failure on the calling thread.
 *  - Calls on the same stream are ordered; calls that share output buffers
 *    on different streams race.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4Q_ABI_VERSION 1

enum fp4q_status {
  FP4Q_OK = 0,
  FP4Q_ERR_NULL_PTR = 1,    /* a required pointer is NULL                         */
  FP4Q_ERR_BAD_SHAPE = 2,   /* sizes <= 0, cols not a multiple of the block, ld < cols, ... */
  FP4Q_ERR_BAD_ALIGN = 3,   /* a pointer or row stride breaks the 16-byte alignment rule */
  FP4Q_ERR_BAD_DTYPE = 4,   /* unknown element type / format enum                  */
  FP4Q_ERR_BAD_ARG = 5,     /* any other invalid argument                          */
  FP4Q_ERR_DEVICE = 6,      /* current device is not gfx950, or no device          */
  FP4Q_ERR_LAUNCH = 7       /* the HIP runtime rejected a launch                   */
};

enum fp4q_dtype { FP4Q_F32 = 0, FP4Q_BF16 = 1 };
enum fp4q_format { FP4Q_NVFP4 = 0, FP4Q_MXFP4 = 1 };

/* ABI version of the loaded library (FP4Q_ABI_VERSION at build time). */
int fp4q_abi_version(void);
/* Static name of a status code. */
const char* fp4q_status_str(int status);
/* Thread-local text of the last failure on this thread ("" if none). */
const char* fp4q_last_error(void);

/*
 * NVFP4 quantization.  [LQ] section 0.2 (E2M1 elements, 16-element blocks,
 * E4M3 block scale, FP32 tensor scale) and section 2.2 (default tensor scale
 * max|W|/(6*256); the candidate E4M3 block scale is rounded up); [GDN]
 * background box "NVFP4 and W4A4" (block scale = block max / 6).
 * Arithmetic, every step one IEEE binary32 operation (round to nearest even):
 *     s_t = A / 1536 with A = max|x| (or the caller's s_t)
 *     s_b = ceil_E4M3(a_b / (6 * s_t)),  a_b = max|x| of the block
 *     rho = 1 / (s_t * s_b);  code = nearest E2M1 of x * rho (ties to even
 *     mantissa, saturating at +-6, sign bit = sign of x * rho)
 *   A block with a_b == 0, or a tensor with s_t == 0, gets scale 0 and codes 0.
 * x:       [rows][ldx] elements of type x_dtype (FP4Q_F32 or FP4Q_BF16);
 *          16-byte aligned, ldx*sizeof(elem) a multiple of 16, ldx >= cols.
 * cols:    multiple of 16.
 * codes:   [rows][cols/2] bytes, 16-byte aligned (output).
 * scales:  [rows][cols/16] E4M3 bytes (output).  With
 *          tensor_scale_is_input == 0 the call first uses this buffer as
 *          scratch for per-workgroup partial maxima (no allocation), then
 *          overwrites it with the block scales; it must then be 4-byte
 *          aligned (FP4Q_ERR_BAD_ALIGN).
 * tensor_scale: one fp32.  tensor_scale_is_input == 0: the library computes
 *          A over the whole tensor on the stream and writes s_t here (the
 *          location is also used as the reduction cell while the call runs);
 *          == 1: s_t is read from here (must be finite and >= +0).  In
 *          both modes the cell must not lie inside the scales buffer
 *          (FP4Q_ERR_BAD_ARG).
 */
int fp4q_quantize_nvfp4(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                        uint8_t* codes, uint8_t* scales, float* tensor_scale,
                        int tensor_scale_is_input, void* stream);

/*
 * NVFP4 quantization with 4/6 block scales.  [LQ] section 2.2 (paragraph
 * applying the residue bound to the signed E2M1 code book: the 4/6 block
 * scaling keeps |x / s| <= 6 whether the rounded-up E4M3 candidate maps the
 * block maximum to 6 or to 4) and the section 2.5 listing (block_scale_46).
 * Per 16-block both candidates are encoded exactly as in
 * fp4q_quantize_nvfp4, with 6 * s_t replaced by 4 * s_t for the second:
 *     s_b(c) = ceil_E4M3(a_b / (c * s_t)),  c in {6, 4}
 * and the block keeps candidate 4 only if its squared error is strictly
 * smaller, both in binary32 in this fixed order:
 *     d_i = x_i - (s(c) * value(code_i)),  e_i = d_i * d_i
 *     E = [((e0+e1)+(e2+e3))+((e4+e5)+(e6+e7))] + [same over elements 8..15]
 * Arguments, buffers, scratch use and errors as for fp4q_quantize_nvfp4;
 * the outputs feed every NVFP4 consumer (GEMMs, Sigma-Delta) unchanged.
 */
int fp4q_quantize_nvfp4_46(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t* codes, uint8_t* scales, float* tensor_scale,
                           int tensor_scale_is_input, void* stream);

/*
 * MXFP4 quantization with the optional online transform.  [MQ] background
 * box "MXFP4 micro-scaling format" (OCP MXFP4: 32-element blocks, E8M0
 * power-of-two scale, E2M1 elements) and "Method steps" 1-3 (activations
 * times the per-channel balance scale t, then the block-32 Hadamard
 * rotation; scaling before rotation; exponent derived from the block max).
 * Arithmetic (binary32, one operation at a time):
 *     z = x * chan_scale[col]                    (skipped if chan_scale == NULL)
 *     z' = FWHT32(z) in Sylvester order, stages h = 1,2,4,8,16, then times
 *          fl32(1/sqrt(32))                      (only if hadamard32 == 1)
 *     e = floor(log2 max|z'| over the block) - 2, clamped to [-127, 127];
 *     byte = e + 127 (0 for an all-zero block); code = nearest E2M1 of z'*2^-e
 * x:          as for fp4q_quantize_nvfp4; cols a multiple of 32.
 * chan_scale: [cols] fp32 or NULL.
 * codes:      [rows][cols/2] (output, 16-byte aligned).
 * scales:     [rows][cols/32] E8M0 bytes (output).
 */
int fp4q_quantize_mxfp4(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                        const float* chan_scale, int hadamard32,
                        uint8_t* codes, uint8_t* scales, void* stream);

/*
 * Standalone balance scale + block-32 Hadamard rotation to fp32, the
 * weight-side transform W' = (W / t) B of [MQ] "Method steps" step 2 (pass
 * chan_scale = 1/t).  Same arithmetic as the transform inside
 * fp4q_quantize_mxfp4, so quantizing y with hadamard32 = 0 gives the same
 * codes as the fused call.
 * y: [rows][ldy] fp32 output, 16-byte aligned, ldy >= cols, ldy % 4 == 0.
 */
int fp4q_hadamard32_scale(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                          const float* chan_scale, float* y, int64_t ldy, void* stream);

/*
 * Per-channel balance scale (calibration statistic; [MQ] "Core method" step
 * (i)): t_j = sigma_j^alpha / rms_j^(1-alpha), sigma_j the population
 * standard deviation of column j of W [N][K], rms_j the root mean square of
 * column j of the calibration activations X [M][K]; each factor floored at
 * 1e-12, t clamped to [2^-16, 2^16]; computed in fp64 on the device.
 * Writes t_out[j] = fl32(t_j) (activation side) and u_out[j] = fl32(1/t_j)
 * (weight side).  w, x: bf16 or fp32, row strides ldw, ldx (elements).
 */
int fp4q_balance_scale(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ldw,
                       const void* x, int x_dtype, int64_t M, int64_t ldx,
                       double alpha, float* t_out, float* u_out, void* stream);

/*
 * One linear of the looped core for first-order Sigma-Delta re-quantization.
 * The ARRAY of segments lives in HOST memory; the pointers inside it are
 * device pointers.
 *   w:            [rows][cols] fp32 master weight (dense)
 *   scales:       [rows][cols/16] E4M3 block scales and
 *   tensor_scale: one fp32 s_t -- the FIXED NVFP4 scale of this weight,
 *                 e.g. from fp4q_quantize_nvfp4(w, ...)
 *   residue:      [rows][cols] fp32 Sigma-Delta state r, read and written;
 *                 the caller zeroes it before the first step of a forward
 *   codes:        output code bank(s), [rows][cols/2] bytes each, 16-byte aligned
 */
typedef struct fp4q_sd_segment {
  const float* w;
  const uint8_t* scales;
  const float* tensor_scale;
  float* residue;
  uint8_t* codes;
  int64_t rows;
  int64_t cols;
} fp4q_sd_segment;

/*
 * First-order Sigma-Delta re-quantization over nseg weights in one launch.
 * [LQ] section 2.1 (fixed scale s, r_0 = 0, v_k = x + r_{k-1},
 * q_k = Q(v_k), r_k = v_k - q_k), section 2.2 (saturating nearest quantizer,
 * x inside the hull [-6, 6]) and the STE listing of section 2.5 (x = W / s,
 * q = nearest E2M1 code, r zeroed every forward).
 * Per element, binary32:  x = clamp(w * rho, -6, 6) with rho = 1/(s_t*s_b)
 * (0 in a zero-scale block);  for each step: v = x + r; code = nearest E2M1
 * of v; r = v - value(code) (exact).
 * steps >= 1 consecutive steps are run with r kept on chip; step j writes its
 * codes at segs[i].codes + j * bank_stride_bytes (bank_stride_bytes is
 * ignored when steps == 1 and otherwise must be >= rows*cols/2 and a
 * multiple of 16).  r is written back once, after the last step.
 * nseg in [1, 64]; every segment: rows >= 1, cols a multiple of 16.
 */
int fp4q_sigma_delta_requant(const fp4q_sd_segment* segs, int nseg, int steps,
                             int64_t bank_stride_bytes, void* stream);

/*
 * Code banks for n_rtn + n_tail loop accesses with the reverse-order tail.
 * [LQ] section 2.3 (partial summation and the reverse-order tail): the
 * first n_rtn accesses use the plain nearest code; the last n_tail run a
 * fresh chain from r_0 = 0 and use its codes in reverse, tail access j
 * taking the chain's code n_tail - j + 1, so the last access gets the
 * nearest code and the chain's final residue meets the tail's first
 * access.  Same per-element arithmetic as fp4q_sigma_delta_requant; one
 * launch; the residue field of the segments is not used (may be NULL).
 * Access b (0-based) is written at segs[i].codes + b * bank_stride_bytes
 * (ignored when n_rtn + n_tail == 1, else >= rows*cols/2 and a multiple of
 * 16).  n_rtn in [0, 4096], n_tail in [1, 4096], nseg in [1, 64].
 */
int fp4q_sigma_delta_schedule(const fp4q_sd_segment* segs, int nseg, int n_rtn, int n_tail,
                              int64_t bank_stride_bytes, void* stream);

/*
 * Stochastic-rounding code banks for the looped core, the comparison the
 * loopquant page runs against Sigma-Delta.  [LQ] section 2 (a fresh random
 * code per access whose expectation equals the weight) and the experiments
 * that use one fixed seed for the whole weight trajectory.  Same fixed
 * scale and x = clamp(w / s, -6, 6) as fp4q_sigma_delta_requant; per
 * element, lo = the largest E2M1 value <= x, hi = the next one,
 * u = (word >> 8) * 2^-24: the code is hi exactly when lo + u (hi - lo) < x
 * (decided exactly, in integers), so P(hi) = (x - lo) / (hi - lo) up to 2^-24; values
 * on the grid are kept; a zero value keeps the sign bit of x; zero-scale
 * blocks give code 0.
 * Random words: Philox4x32-10 (Salmon et al., SC'11) with key
 * (seed mod 2^32, seed >> 32); element e (row-major within segment i) at
 * access k takes output word e mod 4 of counter
 * (g mod 2^32, g >> 32, step0 + k, i), g = e / 4.
 * Access k is written at segs[i].codes + k * bank_stride_bytes (ignored when
 * steps == 1, else >= rows*cols/2 and a multiple of 16).  The residue field
 * is not used.  steps in [1, 4096], nseg in [1, 64].
 */
int fp4q_stochastic_round_requant(const fp4q_sd_segment* segs, int nseg, int steps, int64_t bank_stride_bytes,
                                  uint64_t seed, uint32_t step0, void* stream);

/*
 * Code banks of the stateless two-point chain (F4b) for the looped core.
 * [LQ] section 2.2 (the bound proof covers the recursive chain, not the
 * "two-point closed-form difference" of the code-generation benchmark) and
 * section 4's benchmark; the page gives no formula, and the reading taken:
 * with the same fixed scale and x = clamp(w / s, -6, 6) as
 * fp4q_sigma_delta_requant, lo = the largest E2M1 value <= x, hi = the next
 * one and p = (x - lo) / (hi - lo), access k (k >= 1) takes hi exactly when
 * floor(k p) - floor((k - 1) p) = 1, else lo (exact; values on the grid are
 * kept; a zero keeps the sign bit of x; zero-scale blocks give code 0).  No
 * state: any access is computed directly.  Bank j holds access step0 + j + 1
 * at segs[i].codes + j * bank_stride_bytes (rules as for
 * fp4q_stochastic_round_requant); the residue field is not used.
 * steps in [1, 4096], step0 + steps < 2^24, nseg in [1, 64].
 */
int fp4q_two_point_requant(const fp4q_sd_segment* segs, int nseg, int steps, int64_t bank_stride_bytes,
                           uint32_t step0, void* stream);

/*
 * One member of a fused NVFP4 GEMM (weights quantized separately and
 * concatenated along N).  The ARRAY of members lives in HOST memory; the
 * pointers inside it are device pointers.
 *   scales:       [rows][cols/16] E4M3 block scales of this member, dense,
 *                 rewritten in place; any alignment
 *   tensor_scale: one fp32 s_t of this member (finite, >= 0), read, then
 *                 overwritten with the shared scale
 */
typedef struct fp4q_nv_member {
  uint8_t* scales;
  float* tensor_scale;
  int64_t rows;
  int64_t cols;
} fp4q_nv_member;

/*
 * Shared tensor scale for the members of a fused NVFP4 GEMM.  [GDN]
 * background box on fused GEMMs and the global-scale mismatch, and step (2)
 * of its pipeline: the fused GEMM applies ONE tensor scale, the largest
 * member scale; each member's ratio is folded into its E4M3 block scales
 * (codes unchanged), which re-rounds each block scale by at most half an
 * E4M3 step (1/16 relative for normal results).  Binary32, per member i:
 *   s_t = max_i s_t,i;  r_i = s_t,i / s_t (1 when s_t == 0);
 *   s_b' = E4M3 value nearest to fl(s_b * r_i), ties to the even byte.
 * Bytes with the sign bit set or NaN (0x7F, 0xFF) are left unchanged.
 * Afterwards every members[i].tensor_scale and *shared_tensor_scale hold s_t
 * (shared_tensor_scale may be one of the member cells), so a second call is
 * the identity.  Two kernels on `stream`; nothing is allocated.
 * n_members in [1, 16]; every member: rows >= 1, cols a multiple of 16; the
 * members' scale ranges must not overlap each other or any scale cell
 * (FP4Q_ERR_BAD_ARG).
 */
int fp4q_harmonize_nvfp4(const fp4q_nv_member* members, int n_members,
                         float* shared_tensor_scale, void* stream);

/*
 * Calibration Hessian for the MXFP4 weight refinement.  [MQ] "Method steps"
 * 0 (H = sum over calibration chunks of X^T X, accumulated chunk by chunk)
 * and "Core method" (iii)-(iv) (H taken in the domain of the transformed
 * weight: pass X' = (X * t) B, e.g. from fp4q_hadamard32_scale).
 *   x: [T][ldx] fp32 calibration rows (device), ldx >= n
 *   h: [n][n] fp64 (device), read and written: h_jk += sum_t x_tj * x_tk,
 *      float64, tokens in order (products of two floats are exact), so
 *      chunks passed in order equal one call on their concatenation.  The
 *      caller zeroes h before the first chunk.
 * T >= 1, 1 <= n <= 65536.
 */
int fp4q_hessian_accumulate(const float* x, int64_t T, int64_t n, int64_t ldx, double* h, void* stream);

/*
 * Bytes of device workspace fp4q_macaq_refine needs for an m x n weight:
 * 8 * (32 + n + m * n).
 */
int64_t fp4q_macaq_workspace_bytes(int64_t m, int64_t n);

/*
 * MACaQ weight-side refinement of an MXFP4 weight.  [MQ] "Core method"
 * (iii) and (iv), "Method steps" 3 and 4 (equation 12, Algorithm 1):
 *   H_f = H + lambda * mean(diag H) * I;
 *   per row and 32-block, among the standard exponent e0 (block maximum, as
 *   fp4q_quantize_mxfp4 takes it), e0 + 1 and e0 - 1 keep the one with the
 *   least sum_j (H_f)_jj (w_j - What_j(e))^2 (What: nearest codes at 2^e);
 *   then up to k_iters rounds of Flip-Refinement per row: the move of one
 *   code to an adjacent E2M1 value with the largest positive
 *   gain = 2 D g_ij - D^2 (H_f)_jj is taken and g_i -= D (H_f)_j, with
 *   g_i = (w_i - What_i) H_f; a row stops when no gain is positive.
 * float64, every sum in a fixed sequential order; ties keep e0 (then try
 * e0 + 1 before e0 - 1) and take the smallest j, the move down first.  A
 * zero value is code 0x8 when w is negative (sign bit); an all-zero block
 * keeps scale byte 0 and codes 0.
 *   w:         [m][ldw] fp32 transformed weight W' (device, 16-byte aligned,
 *              ldw >= n, ldw % 4 == 0)
 *   h:         [n][n] fp64 calibration Hessian (symmetric), not modified
 *   lambda:    ridge factor (finite, >= 0; the page uses 1.0)
 *   k_iters:   maximum flips per row (the page uses 128); 0 = screen only
 *   codes:     [m][n/2] packed E2M1 codes (output, 16-byte aligned)
 *   scales:    [m][n/32] E8M0 bytes (output)
 *   flips:     [m] int32 flips taken per row (output) or NULL
 *   workspace: >= fp4q_macaq_workspace_bytes(m, n) bytes of device memory,
 *              8-byte aligned, contents destroyed
 * n % 32 == 0, 32 <= n <= 16384, m >= 1.  Four kernels on `stream`.
 */
int fp4q_macaq_refine(const float* w, int64_t m, int64_t n, int64_t ldw, const double* h, double lambda,
                      int k_iters, uint8_t* codes, uint8_t* scales, int32_t* flips, void* workspace,
                      int64_t workspace_bytes, void* stream);

/*
 * fp4q_macaq_refine for callers that cannot allocate device memory (code
 * under stream capture, serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, and the same output bytes.
 * The workspace is a static array of 16 MiB per device, loaded with the
 * library's code object and held until the process ends; this call makes
 * no allocation.  Rows pass through it in chunks of
 * (2^21 - 32 - n) / n rows (510 at n = 4096, 126 at n = 16384), each chunk
 * on the same four kernels, so every m is accepted; n above 16384 (as for
 * fp4q_macaq_refine) is rejected with FP4Q_ERR_BAD_SHAPE.
 * Nothing in the array needs to start at zero: each call writes what it
 * reads.  Every call on one device shares that device's array and leaves
 * its contents behind: calls that overlap on one device (two streams, two
 * threads) race and give undefined results; serialise them.
 */
int fp4q_macaq_refine_noalloc(const float* w, int64_t m, int64_t n, int64_t ldw, const double* h, double lambda,
                              int k_iters, uint8_t* codes, uint8_t* scales, int32_t* flips, void* stream);

/*
 * W4A4 GEMM over quantized operands: Y = dequant(A) * dequant(B)^T, fp32
 * accumulate, fp32 out.  [MQ] "Core method" (y = [(x*t)B]_MXFP4 W'^T_MXFP4)
 * and [GDN] "NVFP4 and W4A4" (both operands NVFP4, GEMM on the 4-bit data).
 * fmt == FP4Q_MXFP4: a_scales [M][K/32], b_scales [N][K/32] E8M0;
 *                    a_tscale, b_tscale ignored (may be NULL).
 * fmt == FP4Q_NVFP4: a_scales [M][K/16], b_scales [N][K/16] E4M3;
 *                    a_tscale, b_tscale point to one fp32 each.
 * a_codes [M][K/2], b_codes [N][K/2] (16-byte aligned); scales 8-byte
 * aligned; K a multiple of 32 (one MXFP4 block; [MQ] MXFP4 box);
 * y [M][ldy] fp32 (4-byte aligned), ldy >= N.  Shapes with K % 128 != 0
 * run on register-staged kernels that zero the partial last K stage.
 */
int fp4q_gemm_w4a4(int fmt, const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tscale,
                   const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tscale,
                   int64_t M, int64_t N, int64_t K, float* y, int64_t ldy, void* stream);

/*
 * W4A16 GEMM: Y = A_bf16 * dequant(B_nvfp4)^T, fp32 accumulate and output.
 * The matrix product the looped core runs on each step's re-quantized weight
 * ([LQ] section 4: the core-linear microbenchmark with online NVFP4 codes).
 * a: [M][lda] bf16, 16-byte aligned, lda % 8 == 0.  B as for NVFP4 above.
 * K a multiple of 32.
 */
int fp4q_gemm_w4a16(const void* a_bf16, int64_t lda,
                    const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tscale,
                    int64_t M, int64_t N, int64_t K, float* y, int64_t ldy, void* stream);

/*
 * One W4A16 problem for fp4q_gemm_w4a16_grouped: the arguments of
 * fp4q_gemm_w4a16 (same meaning, layout and alignment rules).  The ARRAY
 * lives in HOST memory; the pointers inside it are device pointers.
 */
typedef struct fp4q_w4a16_problem {
  const void* a_bf16;
  int64_t lda;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* b_tscale;
  int64_t M, N, K;
  float* y;
  int64_t ldy;
} fp4q_w4a16_problem;

/*
 * n independent W4A16 GEMMs (the linears of one loop step of the looped
 * core, [LQ] section 4's W4A16 forward), each exactly as
 * fp4q_gemm_w4a16 computes it (bit-identical results), in as few launches
 * as the shapes allow: problems of up to 16 at a time share one launch, so
 * small GEMMs do not each leave the chip idle at their tail.  Outputs must
 * not overlap each other or any input.  n in [1, 64]; each problem is
 * validated as fp4q_gemm_w4a16 validates it (the status names the first
 * bad problem in fp4q_last_error).
 */
int fp4q_gemm_w4a16_grouped(const fp4q_w4a16_problem* probs, int n, void* stream);

/*
 * Decode-shaped NVFP4 W4A4 linear with the activation quantization fused
 * into the GEMM ([GDN] "Limitations": decode was slowed by the small-batch
 * NVFP4 activation-quantization kernel).  Quantizes A (bf16) exactly as
 * fp4q_quantize_nvfp4 does and multiplies by the NVFP4 weight B;
 * Y is bit-identical to fp4q_quantize_nvfp4 followed by fp4q_gemm_w4a4.
 * M in [1, 16]; K a multiple of 32 and at most 7168 (A is held on chip).
 * a_tscale: one fp32, same in/out rule as fp4q_quantize_nvfp4's
 * tensor_scale (with a_tscale_is_input == 0 every workgroup derives s_t
 * from the exact amax of A, so s_t equals fp4q_quantize_nvfp4's).
 * lda: row stride of a in elements, a multiple of 8, >= K; a 16-byte
 * aligned.  b_scales 8-byte aligned; y [M][ldy] fp32, ldy >= N.
 */
int fp4q_linear_w4a4(const void* a_bf16, int64_t lda, float* a_tscale, int a_tscale_is_input,
                     const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tscale,
                     int64_t M, int64_t N, int64_t K, float* y, int64_t ldy, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4Q_H */
