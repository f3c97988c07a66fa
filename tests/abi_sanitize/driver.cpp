// Walks the refusal paths of every C-ABI entry point with fake, never
// dereferenced device pointers (validation fails first) and real host
// structs, under host AddressSanitizer and UndefinedBehaviorSanitizer.
// Prints "ok <n>" and returns 0 when every status matches.  Test
// infrastructure only.
#include <cstdio>
#include <cstring>
#include <cstdint>
#include "../../include/fp4q.h"

static int fails = 0, n = 0;
#define CHECK(expr, want)                                                                          \
  do {                                                                                             \
    ++n;                                                                                           \
    const int got_ = (expr);                                                                       \
    const char* msg_ = fp4q_last_error();                                                          \
    if (got_ != (want) || (got_ != 0 && (!msg_ || !msg_[0]))) {                                    \
      std::printf("FAIL line %d: %s -> %d (want %d) '%s'\n", __LINE__, #expr, got_, (int)(want),   \
                  msg_ ? msg_ : "(null)");                                                         \
      ++fails;                                                                                     \
    }                                                                                              \
  } while (0)

int main() {
  void* f16 = reinterpret_cast<void*>(0x10000);
  void* f4 = reinterpret_cast<void*>(0x10004);
  uint8_t* u16 = static_cast<uint8_t*>(f16);
  float* fl = static_cast<float*>(f16);
  double* db = static_cast<double*>(f16);
  CHECK(fp4q_abi_version() == 1 ? 0 : 1, 0);
  for (int s = 0; s <= 8; ++s) if (!fp4q_status_str(s)) ++fails;
  // quantizers
  CHECK(fp4q_quantize_nvfp4(nullptr, FP4Q_BF16, 4, 32, 32, u16, u16, fl, 0, nullptr), FP4Q_ERR_NULL_PTR);
  CHECK(fp4q_quantize_nvfp4(f16, FP4Q_BF16, 4, 24, 24, u16, u16, fl, 0, nullptr), FP4Q_ERR_BAD_SHAPE);
  CHECK(fp4q_quantize_nvfp4(f16, FP4Q_BF16, 4, 32, 16, u16, u16, fl, 0, nullptr), FP4Q_ERR_BAD_SHAPE);
  CHECK(fp4q_quantize_nvfp4(f4, FP4Q_BF16, 4, 32, 32, u16, u16, fl, 0, nullptr), FP4Q_ERR_BAD_ALIGN);
  CHECK(fp4q_quantize_nvfp4(f16, 7, 4, 32, 32, u16, u16, fl, 0, nullptr), FP4Q_ERR_BAD_DTYPE);
  CHECK(fp4q_quantize_nvfp4(f16, FP4Q_BF16, 0, 32, 32, u16, u16, fl, 0, nullptr), FP4Q_ERR_BAD_SHAPE);
  CHECK(fp4q_quantize_nvfp4(f16, FP4Q_BF16, int64_t(1) << 40, 32, 32, u16, u16, fl, 0, nullptr), FP4Q_ERR_BAD_SHAPE);
  CHECK(fp4q_quantize_nvfp4_46(f16, FP4Q_F32, 4, 32, 32, u16, reinterpret_cast<uint8_t*>(0x10001),
                               reinterpret_cast<float*>(0x20000), 0, nullptr), FP4Q_ERR_BAD_ALIGN);
  CHECK(fp4q_quantize_mxfp4(f16, FP4Q_BF16, 4, 48, 48, nullptr, 0, u16, u16, nullptr), FP4Q_ERR_BAD_SHAPE);
  CHECK(fp4q_quantize_mxfp4(f16, FP4Q_BF16, 4, 64, 64, nullptr, 2, u16, u16, nullptr), FP4Q_ERR_BAD_ARG);
  CHECK(fp4q_quantize_mxfp4(f16, FP4Q_BF16, 4, 64, 64, fl + 1, 1, u16, u16, nullptr), FP4Q_ERR_BAD_ALIGN);
  CHECK(fp4q_hadamard32_scale(f16, FP4Q_BF16, 4, 64, 64, nullptr, nullptr, 64, nullptr), FP4Q_ERR_NULL_PTR);
  CHECK(fp4q_hadamard32_scale(f16, FP4Q_BF16, 4, 64, 64, nullptr, fl, 32, nullptr), FP4Q_ERR_BAD_SHAPE);
  CHECK(fp4q_balance_scale(nullptr, FP4Q_F32, 8, 64, 64, f16, FP4Q_F32, 8, 64, 0.75, fl, fl, nullptr), FP4Q_ERR_NULL_PTR);
  // Sigma-Delta family: host segment tables
  fp4q_sd_segment seg[2];
  std::memset(seg, 0, sizeof(seg));
  seg[0] = {fl, u16, fl, fl, u16, 16, 64};
  seg[1] = {fl, u16, fl, fl, u16, 16, 48};                       // cols % 16 == 0 but not % 32? fine for NVFP4
  CHECK(fp4q_sigma_delta_requant(nullptr, 1, 1, 0, nullptr), FP4Q_ERR_NULL_PTR);
  CHECK(fp4q_sigma_delta_requant(seg, 0, 1, 0, nullptr), FP4Q_ERR_BAD_ARG);
  CHECK(fp4q_sigma_delta_requant(seg, 1, 0, 0, nullptr), FP4Q_ERR_BAD_ARG);
  seg[1].cols = 40;
  CHECK(fp4q_sigma_delta_requant(seg, 2, 1, 0, nullptr), FP4Q_ERR_BAD_SHAPE);
  seg[1].cols = 48;
  seg[1].w = nullptr;
  CHECK(fp4q_sigma_delta_requant(seg, 2, 1, 0, nullptr), FP4Q_ERR_NULL_PTR);
  seg[1].w = fl;
  CHECK(fp4q_sigma_delta_schedule(seg, 1, -1, 4, 0, nullptr), FP4Q_ERR_BAD_ARG);
  CHECK(fp4q_stochastic_round_requant(seg, 1, 0, 0, 42, 0, nullptr), FP4Q_ERR_BAD_ARG);
  CHECK(fp4q_two_point_requant(seg, 1, 0, 0, 0, nullptr), FP4Q_ERR_BAD_ARG);
  // harmonization
  fp4q_nv_member mem[2] = {{u16, fl, 4, 64}, {u16, fl + 1, 4, 64}};
  CHECK(fp4q_harmonize_nvfp4(nullptr, 1, fl, nullptr), FP4Q_ERR_NULL_PTR);
  CHECK(fp4q_harmonize_nvfp4(mem, 0, fl, nullptr), FP4Q_ERR_BAD_ARG);
  CHECK(fp4q_harmonize_nvfp4(mem, 2, fl, nullptr), FP4Q_ERR_BAD_ARG);           // the two scale ranges overlap
  // MACaQ
  CHECK(fp4q_hessian_accumulate(nullptr, 4, 8, 8, db, nullptr), FP4Q_ERR_NULL_PTR);
  CHECK(fp4q_hessian_accumulate(fl, 4, 8, 4, db, nullptr), FP4Q_ERR_BAD_SHAPE);
  CHECK(fp4q_macaq_workspace_bytes(10, 16400) == -1 ? 0 : 1, 0);
  CHECK(fp4q_macaq_refine(fl, 10, 48, 48, db, 1.0, 4, u16, u16, nullptr, f16, 1 << 20, nullptr), FP4Q_ERR_BAD_SHAPE);
  CHECK(fp4q_macaq_refine(fl, 10, 64, 64, db, -1.0, 4, u16, u16, nullptr, f16, 1 << 20, nullptr), FP4Q_ERR_BAD_ARG);
  CHECK(fp4q_macaq_refine(fl, 10, 64, 64, db, 1.0, 4, u16, u16, nullptr, f16, 8, nullptr), FP4Q_ERR_BAD_ARG);
  CHECK(fp4q_macaq_refine_noalloc(fl, 10, 16416, 16416, db, 1.0, 4, u16, u16, nullptr, nullptr), FP4Q_ERR_BAD_SHAPE);
  CHECK(fp4q_macaq_refine_noalloc(fl, 10, 64, 64, db, 1.0, -1, u16, u16, nullptr, nullptr), FP4Q_ERR_BAD_ARG);
  // GEMMs
  CHECK(fp4q_gemm_w4a4(9, u16, u16, fl, u16, u16, fl, 4, 4, 64, fl, 4, nullptr), FP4Q_ERR_BAD_DTYPE);
  CHECK(fp4q_gemm_w4a4(FP4Q_NVFP4, u16, u16, nullptr, u16, u16, fl, 4, 4, 64, fl, 4, nullptr), FP4Q_ERR_NULL_PTR);
  CHECK(fp4q_gemm_w4a4(FP4Q_MXFP4, u16, u16, nullptr, u16, u16, nullptr, 4, 4, 48, fl, 4, nullptr), FP4Q_ERR_BAD_SHAPE);
  CHECK(fp4q_gemm_w4a4(FP4Q_MXFP4, u16, u16, nullptr, u16, u16, nullptr, 4, 4, 64, fl, 2, nullptr), FP4Q_ERR_BAD_SHAPE);
  CHECK(fp4q_gemm_w4a16(f16, 64, u16, u16, fl, 4, 4, 48, fl, 4, nullptr), FP4Q_ERR_BAD_SHAPE);
  fp4q_w4a16_problem pr[2] = {{f16, 128, u16, u16, fl, 4, 4, 128, fl, 4}, {f16, 100, u16, u16, fl, 4, 4, 128, fl, 4}};
  CHECK(fp4q_gemm_w4a16_grouped(pr, 2, nullptr), FP4Q_ERR_BAD_SHAPE);
  CHECK(fp4q_gemm_w4a16_grouped(pr, 0, nullptr), FP4Q_ERR_BAD_ARG);
  CHECK(fp4q_linear_w4a4(f16, 64, fl, 0, u16, u16, fl, 17, 4, 64, fl, 4, nullptr), FP4Q_ERR_BAD_SHAPE);
  CHECK(fp4q_linear_w4a4(f16, 64, nullptr, 0, u16, u16, fl, 1, 4, 64, fl, 4, nullptr), FP4Q_ERR_NULL_PTR);
  // a long error message stays within its buffer
  for (int i = 0; i < 64; ++i) (void)fp4q_gemm_w4a16_grouped(pr, 2, nullptr);
  if (std::strlen(fp4q_last_error()) >= 512) ++fails;
  std::printf("%s %d\n", fails ? "failed" : "ok", n);
  return fails ? 1 : 0;
}
