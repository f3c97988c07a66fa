// internal.h -- launchers shared between the kernel translation units and the
// C ABI layer (api.cpp).  Every launcher enqueues on `s` and returns the HIP
// status of its launches; argument validation happens in api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp4q.h"

namespace fp4q {

// Compute units of the current device (cached per device; 256 if the query
// fails).
int device_cus();

// four_six != 0: the 4/6 block scales (block maximum to 6 or to 4, whichever
// gives the smaller block squared error)
hipError_t launch_quant_nvfp4(const void* x, int bf16, int64_t rows, int64_t cols, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, float* ts, int ts_is_input,
                              int four_six, hipStream_t s);
// Writes the tensor maximum A = max|x| into the tensor-scale cell: with one
// workgroup as flag | A (amax encoding), after per-workgroup partial maxima
// (in scratch, when it is large enough; may be NULL with scratch_bytes ==
// 0; its contents are destroyed) as s_t = fl(A / 1536) itself.  The NVFP4
// quantizer reads either form.
hipError_t launch_amax_to_cell(const void* x, int bf16, int64_t rows, int64_t cols, int64_t ldx,
                               float* cell, uint8_t* scratch, int64_t scratch_bytes, hipStream_t s);
hipError_t launch_quant_mxfp4(const void* x, int bf16, int64_t rows, int64_t cols, int64_t ldx,
                              const float* chan_scale, int hadamard, uint8_t* codes,
                              uint8_t* scales, hipStream_t s);
hipError_t launch_hadamard32_scale(const void* x, int bf16, int64_t rows, int64_t cols,
                                   int64_t ldx, const float* chan_scale, float* y, int64_t ldy,
                                   hipStream_t s);
hipError_t launch_balance_scale(const void* w, int w_bf16, int64_t N, int64_t K, int64_t ldw,
                                const void* x, int x_bf16, int64_t M, int64_t ldx, double alpha,
                                float* t_out, float* u_out, hipStream_t s);
// sched != 0: the reverse-order tail schedule (n_rtn nearest-code banks,
// then `steps` chain codes in reverse; no residue buffer)
hipError_t launch_sigma_delta(const fp4q_sd_segment* segs, int nseg, int steps,
                              int64_t bank_stride, int sched, int n_rtn, hipStream_t s);
// two_point != 0: the stateless two-point chain instead (seed unused)
hipError_t launch_stochastic_round(const fp4q_sd_segment* segs, int nseg, int steps, int64_t bank_stride,
                                   uint64_t seed, uint32_t step0, int two_point, hipStream_t s);
hipError_t launch_harmonize_nvfp4(const fp4q_nv_member* mem, int n, float* shared, hipStream_t s);
hipError_t launch_hessian(const float* x, int64_t T, int64_t n, int64_t ldx, double* h, hipStream_t s);
hipError_t launch_macaq_refine(const float* w, int64_t m, int64_t n, int64_t ldw, const double* h, double lam,
                               int k_iters, uint8_t* codes, uint8_t* scales, int32_t* flips, double* ws,
                               hipStream_t s);
// The same refinement with the workspace in a static per-device array of
// kMacaqScratchDoubles float64 (16 MiB): the ridge once, then the rows in
// passes of macaq_scratch_rows(n) rows.  Calls that overlap on one device
// race on that array.
constexpr int64_t kMacaqScratchDoubles = int64_t(1) << 21;
int64_t macaq_scratch_rows(int64_t n);
hipError_t launch_macaq_refine_static(const float* w, int64_t m, int64_t n, int64_t ldw, const double* h,
                                      double lam, int k_iters, uint8_t* codes, uint8_t* scales, int32_t* flips,
                                      hipStream_t s);

hipError_t launch_gemm_mxfp4(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                             const uint8_t* bs, int64_t M, int64_t N, int64_t K, float* y,
                             int64_t ldy, hipStream_t s);
// Register-staged MXFP4 kernel for shapes the direct-load kernel does not take.
hipError_t launch_gemm_mxfp4_staged(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                                    const uint8_t* bs, int64_t M, int64_t N, int64_t K, float* y,
                                    int64_t ldy, hipStream_t s);
hipError_t launch_gemm_nvfp4_staged(const uint8_t* a, const uint8_t* as, const float* ats,
                                    const uint8_t* b, const uint8_t* bs, const float* bts, int64_t M,
                                    int64_t N, int64_t K, float* y, int64_t ldy, hipStream_t s);
hipError_t launch_gemm_nvfp4(const uint8_t* a, const uint8_t* as, const float* ats,
                             const uint8_t* b, const uint8_t* bs, const float* bts, int64_t M,
                             int64_t N, int64_t K, float* y, int64_t ldy, hipStream_t s);
// W4A16 on the direct-load pipeline (gemm_mx.hip), when the shape allows it
bool w4a16_direct_supported(int64_t lda, int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_w4a16_direct(const void* a, int64_t lda, const uint8_t* b, const uint8_t* bs,
                                    const float* bts, int64_t M, int64_t N, int64_t K, float* y, int64_t ldy,
                                    hipStream_t s);
hipError_t launch_gemm_w4a16(const void* a, int64_t lda, const uint8_t* b, const uint8_t* bs,
                             const float* bts, int64_t M, int64_t N, int64_t K, float* y,
                             int64_t ldy, hipStream_t s);
// Several W4A16 problems; those the direct-load kernel takes share launches
// of up to 16 problems (n <= 64).
hipError_t launch_gemm_w4a16_grouped(const fp4q_w4a16_problem* probs, int n, hipStream_t s);
// Largest K the skinny kernel holds in LDS.
bool skinny_supported(int64_t K);
// Skinny NVFP4 GEMM for M <= 16.  If a_bf16 != NULL the activation is
// quantized inside the kernel (a_codes / a_scales ignored; a_ts is the
// tensor-scale cell in the same state encoding fp4q_quantize_nvfp4 uses).
hipError_t launch_gemm_nvfp4_skinny(const void* a_bf16, int64_t lda, const uint8_t* a_codes,
                                    const uint8_t* a_scales, const float* a_ts, int a_dynamic,
                                    const uint8_t* b, const uint8_t* bs, const float* bts,
                                    int64_t M, int64_t N, int64_t K, float* y, int64_t ldy,
                                    hipStream_t s);

}  // namespace fp4q
