// api.cpp -- the C ABI of libfp4q (include/fp4q.h): host-side argument
// validation, the gfx950 device check and dispatch to the kernel launchers.
// Nothing here allocates device memory or synchronizes a stream.

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/fp4q.h"
#include "internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FP4Q_OK;
  return fail(FP4Q_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The device check is cached per device ordinal; the cache is filled once
// per device under a mutex and is read-only afterwards.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(FP4Q_ERR_DEVICE, "no current HIP device");
  static std::mutex mu;
  static signed char ok[64] = {0};  // 0 unknown, 1 gfx950, -1 other
  if (dev >= 64) return fail(FP4Q_ERR_DEVICE, "device ordinal %d out of range", dev);
  {
    std::lock_guard<std::mutex> lk(mu);
    if (ok[dev] == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(FP4Q_ERR_DEVICE, "hipGetDeviceProperties failed");
      ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    }
    if (ok[dev] < 0) return fail(FP4Q_ERR_DEVICE, "device %d is not gfx950", dev);
  }
  return FP4Q_OK;
}

int check_dtype(int dt) {
  if (dt != FP4Q_F32 && dt != FP4Q_BF16) return fail(FP4Q_ERR_BAD_DTYPE, "unknown dtype %d", dt);
  return FP4Q_OK;
}

// Common checks of a [rows][ldx] input tensor whose cols are split in blocks.
int check_input(const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx, int64_t block,
                const char* name) {
  if (!x) return fail(FP4Q_ERR_NULL_PTR, "%s is NULL", name);
  if (int st = check_dtype(dt)) return st;
  if (rows <= 0 || cols <= 0) return fail(FP4Q_ERR_BAD_SHAPE, "%s: rows and cols must be > 0", name);
  if (cols % block) return fail(FP4Q_ERR_BAD_SHAPE, "%s: cols %lld not a multiple of %lld", name, (long long)cols, (long long)block);
  if (ldx < cols) return fail(FP4Q_ERR_BAD_SHAPE, "%s: ld %lld < cols %lld", name, (long long)ldx, (long long)cols);
  const int64_t es = dt == FP4Q_BF16 ? 2 : 4;
  if (!aligned16(x) || (ldx * es) % 16) return fail(FP4Q_ERR_BAD_ALIGN, "%s: pointer or row stride not 16-byte aligned", name);
  if (rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31)) return fail(FP4Q_ERR_BAD_SHAPE, "%s: size too large", name);
  return FP4Q_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Argument checks shared by both forms of the MACaQ refinement.
int check_macaq(const float* w, int64_t m, int64_t n, int64_t ldw, const double* h, double lambda, int k_iters,
                const uint8_t* codes, const uint8_t* scales) {
  if (!w || !h || !codes || !scales) return fail(FP4Q_ERR_NULL_PTR, "w, h, codes and scales are required");
  if (m < 1 || n < 32 || n % 32 || n > 16384 || ldw < n || ldw % 4)
    return fail(FP4Q_ERR_BAD_SHAPE, "bad shape (m >= 1, n %% 32 == 0, 32 <= n <= 16384, ldw >= n, ldw %% 4 == 0)");
  if (m > (int64_t(1) << 40) / ldw) return fail(FP4Q_ERR_BAD_SHAPE, "w too large");
  if (!aligned16(w) || !aligned16(codes)) return fail(FP4Q_ERR_BAD_ALIGN, "w and codes must be 16-byte aligned");
  if (!(lambda >= 0.0) || lambda > 1e300) return fail(FP4Q_ERR_BAD_ARG, "lambda must be finite and >= 0");
  if (k_iters < 0 || k_iters > (1 << 20)) return fail(FP4Q_ERR_BAD_ARG, "k_iters must be in [0, 2^20]");
  return FP4Q_OK;
}

}  // namespace

extern "C" {

int fp4q_abi_version(void) { return FP4Q_ABI_VERSION; }

const char* fp4q_status_str(int status) {
  switch (status) {
    case FP4Q_OK: return "FP4Q_OK";
    case FP4Q_ERR_NULL_PTR: return "FP4Q_ERR_NULL_PTR";
    case FP4Q_ERR_BAD_SHAPE: return "FP4Q_ERR_BAD_SHAPE";
    case FP4Q_ERR_BAD_ALIGN: return "FP4Q_ERR_BAD_ALIGN";
    case FP4Q_ERR_BAD_DTYPE: return "FP4Q_ERR_BAD_DTYPE";
    case FP4Q_ERR_BAD_ARG: return "FP4Q_ERR_BAD_ARG";
    case FP4Q_ERR_DEVICE: return "FP4Q_ERR_DEVICE";
    case FP4Q_ERR_LAUNCH: return "FP4Q_ERR_LAUNCH";
    default: return "FP4Q_ERR_UNKNOWN";
  }
}

const char* fp4q_last_error(void) { return g_last_error; }

namespace {
int quantize_nvfp4_impl(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                        uint8_t* codes, uint8_t* scales, float* tensor_scale,
                        int tensor_scale_is_input, int four_six, void* stream, const char* what) {
  g_last_error[0] = 0;
  if (int st = check_input(x, x_dtype, rows, cols, ldx, 16, "x")) return st;
  if (!codes || !scales || !tensor_scale) return fail(FP4Q_ERR_NULL_PTR, "codes, scales and tensor_scale are required");
  if (!aligned16(codes)) return fail(FP4Q_ERR_BAD_ALIGN, "codes not 16-byte aligned");
  if (!(reinterpret_cast<uintptr_t>(tensor_scale) % 4 == 0)) return fail(FP4Q_ERR_BAD_ALIGN, "tensor_scale not 4-byte aligned");
  if (tensor_scale_is_input != 0 && tensor_scale_is_input != 1) return fail(FP4Q_ERR_BAD_ARG, "tensor_scale_is_input must be 0 or 1");
  // with a computed tensor scale the scales buffer first holds 32-bit
  // partial maxima
  if (!tensor_scale_is_input && (reinterpret_cast<uintptr_t>(scales) & 3u))
    return fail(FP4Q_ERR_BAD_ALIGN, "scales must be 4-byte aligned when the tensor scale is computed");
  // every workgroup reads the tensor-scale cell while others write scales
  {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(scales), hi = lo + (uintptr_t)(rows * (cols / 16));
    const uintptr_t c = reinterpret_cast<uintptr_t>(tensor_scale);
    if (c + sizeof(float) > lo && c < hi) return fail(FP4Q_ERR_BAD_ARG, "tensor_scale lies inside the scales buffer");
  }
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_quant_nvfp4(x, x_dtype == FP4Q_BF16, rows, cols, ldx, codes, scales,
                                                tensor_scale, tensor_scale_is_input, four_six,
                                                as_stream(stream)),
                       what);
}
}  // namespace

int fp4q_quantize_nvfp4(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                        uint8_t* codes, uint8_t* scales, float* tensor_scale,
                        int tensor_scale_is_input, void* stream) {
  return quantize_nvfp4_impl(x, x_dtype, rows, cols, ldx, codes, scales, tensor_scale, tensor_scale_is_input,
                             0, stream, "quantize_nvfp4");
}

int fp4q_quantize_nvfp4_46(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t* codes, uint8_t* scales, float* tensor_scale,
                           int tensor_scale_is_input, void* stream) {
  return quantize_nvfp4_impl(x, x_dtype, rows, cols, ldx, codes, scales, tensor_scale, tensor_scale_is_input,
                             1, stream, "quantize_nvfp4_46");
}

int fp4q_quantize_mxfp4(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                        const float* chan_scale, int hadamard32, uint8_t* codes, uint8_t* scales,
                        void* stream) {
  g_last_error[0] = 0;
  if (int st = check_input(x, x_dtype, rows, cols, ldx, 32, "x")) return st;
  if (!codes || !scales) return fail(FP4Q_ERR_NULL_PTR, "codes and scales are required");
  if (!aligned16(codes)) return fail(FP4Q_ERR_BAD_ALIGN, "codes not 16-byte aligned");
  if (chan_scale && !aligned16(chan_scale)) return fail(FP4Q_ERR_BAD_ALIGN, "chan_scale not 16-byte aligned");
  if (hadamard32 != 0 && hadamard32 != 1) return fail(FP4Q_ERR_BAD_ARG, "hadamard32 must be 0 or 1");
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_quant_mxfp4(x, x_dtype == FP4Q_BF16, rows, cols, ldx, chan_scale,
                                                hadamard32, codes, scales, as_stream(stream)),
                       "quantize_mxfp4");
}

int fp4q_hadamard32_scale(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                          const float* chan_scale, float* y, int64_t ldy, void* stream) {
  g_last_error[0] = 0;
  if (int st = check_input(x, x_dtype, rows, cols, ldx, 32, "x")) return st;
  if (!y) return fail(FP4Q_ERR_NULL_PTR, "y is NULL");
  if (ldy < cols) return fail(FP4Q_ERR_BAD_SHAPE, "ldy < cols");
  if (!aligned16(y) || ldy % 4) return fail(FP4Q_ERR_BAD_ALIGN, "y or ldy not 16-byte aligned");
  if (chan_scale && !aligned16(chan_scale)) return fail(FP4Q_ERR_BAD_ALIGN, "chan_scale not 16-byte aligned");
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_hadamard32_scale(x, x_dtype == FP4Q_BF16, rows, cols, ldx, chan_scale,
                                                     y, ldy, as_stream(stream)),
                       "hadamard32_scale");
}

int fp4q_balance_scale(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ldw,
                       const void* x, int x_dtype, int64_t M, int64_t ldx, double alpha,
                       float* t_out, float* u_out, void* stream) {
  g_last_error[0] = 0;
  if (!w || !x || !t_out || !u_out) return fail(FP4Q_ERR_NULL_PTR, "w, x, t_out and u_out are required");
  if (int st = check_dtype(w_dtype)) return st;
  if (int st = check_dtype(x_dtype)) return st;
  if (N <= 0 || K <= 0 || M <= 0) return fail(FP4Q_ERR_BAD_SHAPE, "N, K and M must be > 0");
  if (ldw < K || ldx < K) return fail(FP4Q_ERR_BAD_SHAPE, "ldw and ldx must be >= K");
  if (!(alpha >= 0.0 && alpha <= 1.0)) return fail(FP4Q_ERR_BAD_ARG, "alpha must be in [0, 1]");
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_balance_scale(w, w_dtype == FP4Q_BF16, N, K, ldw, x, x_dtype == FP4Q_BF16,
                                                  M, ldx, alpha, t_out, u_out, as_stream(stream)),
                       "balance_scale");
}

int fp4q_sigma_delta_requant(const fp4q_sd_segment* segs, int nseg, int steps,
                             int64_t bank_stride_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!segs) return fail(FP4Q_ERR_NULL_PTR, "segs is NULL");
  if (nseg < 1 || nseg > 64) return fail(FP4Q_ERR_BAD_ARG, "nseg must be in [1, 64]");
  if (steps < 1) return fail(FP4Q_ERR_BAD_ARG, "steps must be >= 1");
  for (int i = 0; i < nseg; ++i) {
    const fp4q_sd_segment& g = segs[i];
    if (!g.w || !g.scales || !g.tensor_scale || !g.residue || !g.codes)
      return fail(FP4Q_ERR_NULL_PTR, "segment %d has a NULL pointer", i);
    if (g.rows <= 0 || g.cols <= 0 || g.cols % 16) return fail(FP4Q_ERR_BAD_SHAPE, "segment %d: bad shape", i);
    if (g.rows * g.cols > (int64_t(1) << 34)) return fail(FP4Q_ERR_BAD_SHAPE, "segment %d: too large", i);
    if (!aligned16(g.w) || !aligned16(g.residue) || !aligned16(g.codes))
      return fail(FP4Q_ERR_BAD_ALIGN, "segment %d: w, residue and codes must be 16-byte aligned", i);
    if (steps > 1 && (bank_stride_bytes < g.rows * g.cols / 2 || bank_stride_bytes % 16))
      return fail(FP4Q_ERR_BAD_ARG, "segment %d: bank_stride_bytes too small or not a multiple of 16", i);
  }
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_sigma_delta(segs, nseg, steps, steps > 1 ? bank_stride_bytes : 0, 0, 0,
                                                as_stream(stream)),
                       "sigma_delta_requant");
}

int fp4q_sigma_delta_schedule(const fp4q_sd_segment* segs, int nseg, int n_rtn, int n_tail,
                              int64_t bank_stride_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!segs) return fail(FP4Q_ERR_NULL_PTR, "segs is NULL");
  if (nseg < 1 || nseg > 64) return fail(FP4Q_ERR_BAD_ARG, "nseg must be in [1, 64]");
  if (n_rtn < 0 || n_tail < 1 || n_rtn > 4096 || n_tail > 4096)
    return fail(FP4Q_ERR_BAD_ARG, "n_rtn must be in [0, 4096] and n_tail in [1, 4096]");
  const int banks = n_rtn + n_tail;
  for (int i = 0; i < nseg; ++i) {
    const fp4q_sd_segment& g = segs[i];
    if (!g.w || !g.scales || !g.tensor_scale || !g.codes)
      return fail(FP4Q_ERR_NULL_PTR, "segment %d has a NULL pointer", i);
    if (g.rows <= 0 || g.cols <= 0 || g.cols % 16) return fail(FP4Q_ERR_BAD_SHAPE, "segment %d: bad shape", i);
    if (g.rows * g.cols > (int64_t(1) << 34)) return fail(FP4Q_ERR_BAD_SHAPE, "segment %d: too large", i);
    if (!aligned16(g.w) || !aligned16(g.codes))
      return fail(FP4Q_ERR_BAD_ALIGN, "segment %d: w and codes must be 16-byte aligned", i);
    if (banks > 1 && (bank_stride_bytes < g.rows * g.cols / 2 || bank_stride_bytes % 16))
      return fail(FP4Q_ERR_BAD_ARG, "segment %d: bank_stride_bytes too small or not a multiple of 16", i);
  }
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_sigma_delta(segs, nseg, n_tail, banks > 1 ? bank_stride_bytes : 0, 1, n_rtn,
                                                as_stream(stream)),
                       "sigma_delta_schedule");
}

namespace {
int check_bank_segments(const fp4q_sd_segment* segs, int nseg, int steps, int64_t bank_stride_bytes) {
  if (!segs) return fail(FP4Q_ERR_NULL_PTR, "segs is NULL");
  if (nseg < 1 || nseg > 64) return fail(FP4Q_ERR_BAD_ARG, "nseg must be in [1, 64]");
  if (steps < 1 || steps > 4096) return fail(FP4Q_ERR_BAD_ARG, "steps must be in [1, 4096]");
  for (int i = 0; i < nseg; ++i) {
    const fp4q_sd_segment& g = segs[i];
    if (!g.w || !g.scales || !g.tensor_scale || !g.codes)
      return fail(FP4Q_ERR_NULL_PTR, "segment %d has a NULL pointer", i);
    if (g.rows <= 0 || g.cols <= 0 || g.cols % 16) return fail(FP4Q_ERR_BAD_SHAPE, "segment %d: bad shape", i);
    if (g.rows * g.cols > (int64_t(1) << 34)) return fail(FP4Q_ERR_BAD_SHAPE, "segment %d: too large", i);
    if (!aligned16(g.w) || !aligned16(g.codes))
      return fail(FP4Q_ERR_BAD_ALIGN, "segment %d: w and codes must be 16-byte aligned", i);
    if (steps > 1 && (bank_stride_bytes < g.rows * g.cols / 2 || bank_stride_bytes % 16))
      return fail(FP4Q_ERR_BAD_ARG, "segment %d: bank_stride_bytes too small or not a multiple of 16", i);
  }
  return FP4Q_OK;
}
}  // namespace

int fp4q_two_point_requant(const fp4q_sd_segment* segs, int nseg, int steps, int64_t bank_stride_bytes,
                           uint32_t step0, void* stream) {
  g_last_error[0] = 0;
  if (int st = check_bank_segments(segs, nseg, steps, bank_stride_bytes)) return st;
  if ((uint64_t)step0 + (uint64_t)steps >= (uint64_t(1) << 24))
    return fail(FP4Q_ERR_BAD_ARG, "step0 + steps must be below 2^24");
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_stochastic_round(segs, nseg, steps, steps > 1 ? bank_stride_bytes : 0, 0,
                                                     step0, 1, as_stream(stream)),
                       "two_point_requant");
}

int fp4q_stochastic_round_requant(const fp4q_sd_segment* segs, int nseg, int steps, int64_t bank_stride_bytes,
                                  uint64_t seed, uint32_t step0, void* stream) {
  g_last_error[0] = 0;
  if (int st = check_bank_segments(segs, nseg, steps, bank_stride_bytes)) return st;
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_stochastic_round(segs, nseg, steps, steps > 1 ? bank_stride_bytes : 0, seed,
                                                     step0, 0, as_stream(stream)),
                       "stochastic_round_requant");
}

int fp4q_harmonize_nvfp4(const fp4q_nv_member* members, int n_members,
                         float* shared_tensor_scale, void* stream) {
  g_last_error[0] = 0;
  if (!members || !shared_tensor_scale) return fail(FP4Q_ERR_NULL_PTR, "members or shared_tensor_scale is NULL");
  if (n_members < 1 || n_members > 16) return fail(FP4Q_ERR_BAD_ARG, "n_members must be in [1, 16]");
  for (int i = 0; i < n_members; ++i) {
    const fp4q_nv_member& m = members[i];
    if (!m.scales || !m.tensor_scale) return fail(FP4Q_ERR_NULL_PTR, "member %d has a NULL pointer", i);
    if (m.rows <= 0 || m.cols <= 0 || m.cols % 16) return fail(FP4Q_ERR_BAD_SHAPE, "member %d: bad shape", i);
    if (m.rows * (m.cols / 16) > (int64_t(1) << 36)) return fail(FP4Q_ERR_BAD_SHAPE, "member %d: too large", i);
  }
  // every scale range must be disjoint from the other scale ranges and
  // from every fp32 cell the kernels read or write
  auto lo = [&](int i) { return reinterpret_cast<uintptr_t>(members[i].scales); };
  auto hi = [&](int i) { return lo(i) + (uintptr_t)(members[i].rows * (members[i].cols / 16)); };
  auto hits = [&](int i, const void* cell) {
    const uintptr_t c = reinterpret_cast<uintptr_t>(cell);
    return c + sizeof(float) > lo(i) && c < hi(i);
  };
  for (int i = 0; i < n_members; ++i) {
    if (hits(i, shared_tensor_scale)) return fail(FP4Q_ERR_BAD_ARG, "member %d: scales overlap the shared cell", i);
    for (int j = 0; j < n_members; ++j) {
      if (hits(i, members[j].tensor_scale))
        return fail(FP4Q_ERR_BAD_ARG, "member %d: scales overlap the tensor scale of member %d", i, j);
      if (j != i && lo(i) < hi(j) && lo(j) < hi(i))
        return fail(FP4Q_ERR_BAD_ARG, "members %d and %d: scale ranges overlap", i, j);
    }
  }
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_harmonize_nvfp4(members, n_members, shared_tensor_scale, as_stream(stream)),
                       "harmonize_nvfp4");
}

int fp4q_hessian_accumulate(const float* x, int64_t T, int64_t n, int64_t ldx, double* h, void* stream) {
  g_last_error[0] = 0;
  if (!x || !h) return fail(FP4Q_ERR_NULL_PTR, "x or h is NULL");
  if (T < 1 || n < 1 || n > 65536 || ldx < n) return fail(FP4Q_ERR_BAD_SHAPE, "bad shape (T >= 1, 1 <= n <= 65536, ldx >= n)");
  if (T > (int64_t(1) << 40) / ldx) return fail(FP4Q_ERR_BAD_SHAPE, "x too large");
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_hessian(x, T, n, ldx, h, as_stream(stream)), "hessian_accumulate");
}

int64_t fp4q_macaq_workspace_bytes(int64_t m, int64_t n) {
  if (m < 1 || n < 1 || n > 16384 || m > (int64_t(1) << 40) / n) return -1;
  return 8 * (32 + ((n + 31) / 32) * 32 + m * n);
}

int fp4q_macaq_refine(const float* w, int64_t m, int64_t n, int64_t ldw, const double* h, double lambda,
                      int k_iters, uint8_t* codes, uint8_t* scales, int32_t* flips, void* workspace,
                      int64_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!workspace) return fail(FP4Q_ERR_NULL_PTR, "workspace is required");
  if (int st = check_macaq(w, m, n, ldw, h, lambda, k_iters, codes, scales)) return st;
  if (reinterpret_cast<uintptr_t>(workspace) & 7u) return fail(FP4Q_ERR_BAD_ALIGN, "workspace must be 8-byte aligned");
  if (workspace_bytes < fp4q_macaq_workspace_bytes(m, n))
    return fail(FP4Q_ERR_BAD_ARG, "workspace too small (%lld bytes needed)", (long long)fp4q_macaq_workspace_bytes(m, n));
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_macaq_refine(w, m, n, ldw, h, lambda, k_iters, codes, scales, flips,
                                                 static_cast<double*>(workspace), as_stream(stream)),
                       "macaq_refine");
}

int fp4q_macaq_refine_noalloc(const float* w, int64_t m, int64_t n, int64_t ldw, const double* h, double lambda,
                              int k_iters, uint8_t* codes, uint8_t* scales, int32_t* flips, void* stream) {
  g_last_error[0] = 0;
  if (int st = check_macaq(w, m, n, ldw, h, lambda, k_iters, codes, scales)) return st;
  if (fp4q::macaq_scratch_rows(n) < 1)
    return fail(FP4Q_ERR_BAD_ARG, "n = %lld: one row does not fit the %lld-byte static workspace", (long long)n,
                (long long)(8 * fp4q::kMacaqScratchDoubles));
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_macaq_refine_static(w, m, n, ldw, h, lambda, k_iters, codes, scales, flips,
                                                        as_stream(stream)),
                       "macaq_refine_noalloc");
}

int fp4q_gemm_w4a4(int fmt, const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tscale,
                   const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tscale,
                   int64_t M, int64_t N, int64_t K, float* y, int64_t ldy, void* stream) {
  g_last_error[0] = 0;
  if (fmt != FP4Q_NVFP4 && fmt != FP4Q_MXFP4) return fail(FP4Q_ERR_BAD_DTYPE, "unknown format %d", fmt);
  if (!a_codes || !a_scales || !b_codes || !b_scales || !y) return fail(FP4Q_ERR_NULL_PTR, "operand pointer is NULL");
  if (fmt == FP4Q_NVFP4 && (!a_tscale || !b_tscale)) return fail(FP4Q_ERR_NULL_PTR, "NVFP4 needs both tensor scales");
  if (M <= 0 || N <= 0 || K <= 0) return fail(FP4Q_ERR_BAD_SHAPE, "M, N and K must be > 0");
  if (K % 32) return fail(FP4Q_ERR_BAD_SHAPE, "K must be a multiple of 32");
  if ((reinterpret_cast<uintptr_t>(a_scales) | reinterpret_cast<uintptr_t>(b_scales)) & 7u)
    return fail(FP4Q_ERR_BAD_ALIGN, "scales must be 8-byte aligned");
  if (ldy < N) return fail(FP4Q_ERR_BAD_SHAPE, "ldy < N");
  if (M > (int64_t(1) << 31) || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return fail(FP4Q_ERR_BAD_SHAPE, "size too large");
  if (!aligned16(a_codes) || !aligned16(b_codes)) return fail(FP4Q_ERR_BAD_ALIGN, "codes must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(y) & 3u)) return fail(FP4Q_ERR_BAD_ALIGN, "y must be 4-byte aligned");
  if (int st = check_device()) return st;
  hipStream_t s = as_stream(stream);
  if (fmt == FP4Q_MXFP4)
    return launch_status(fp4q::launch_gemm_mxfp4(a_codes, a_scales, b_codes, b_scales, M, N, K, y, ldy, s), "gemm_mxfp4");
  if (M <= 16 && fp4q::skinny_supported(K))
    return launch_status(fp4q::launch_gemm_nvfp4_skinny(nullptr, 0, a_codes, a_scales, a_tscale, 0, b_codes,
                                                        b_scales, b_tscale, M, N, K, y, ldy, s),
                         "gemm_nvfp4_skinny");
  return launch_status(fp4q::launch_gemm_nvfp4(a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M, N, K,
                                               y, ldy, s),
                       "gemm_nvfp4");
}

namespace {
int check_w4a16(const void* a_bf16, int64_t lda, const uint8_t* b_codes, const uint8_t* b_scales,
                const float* b_tscale, int64_t M, int64_t N, int64_t K, const float* y, int64_t ldy) {
  if (!a_bf16 || !b_codes || !b_scales || !b_tscale || !y) return fail(FP4Q_ERR_NULL_PTR, "operand pointer is NULL");
  if (M <= 0 || N <= 0 || K <= 0) return fail(FP4Q_ERR_BAD_SHAPE, "M, N and K must be > 0");
  if (K % 32) return fail(FP4Q_ERR_BAD_SHAPE, "K must be a multiple of 32");
  if (lda < K || ldy < N) return fail(FP4Q_ERR_BAD_SHAPE, "lda < K or ldy < N");
  if (reinterpret_cast<uintptr_t>(b_scales) & 7u) return fail(FP4Q_ERR_BAD_ALIGN, "b_scales must be 8-byte aligned");
  if (M > (int64_t(1) << 31) || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return fail(FP4Q_ERR_BAD_SHAPE, "size too large");
  if (!aligned16(a_bf16) || lda % 8 || !aligned16(b_codes)) return fail(FP4Q_ERR_BAD_ALIGN, "a, lda or b_codes not 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(y) & 3u)) return fail(FP4Q_ERR_BAD_ALIGN, "y must be 4-byte aligned");
  return FP4Q_OK;
}
}  // namespace

int fp4q_gemm_w4a16_grouped(const fp4q_w4a16_problem* probs, int n, void* stream) {
  g_last_error[0] = 0;
  if (!probs) return fail(FP4Q_ERR_NULL_PTR, "probs is NULL");
  if (n < 1 || n > 64) return fail(FP4Q_ERR_BAD_ARG, "n must be in [1, 64]");
  for (int i = 0; i < n; ++i) {
    const fp4q_w4a16_problem& q = probs[i];
    if (int st = check_w4a16(q.a_bf16, q.lda, q.b_codes, q.b_scales, q.b_tscale, q.M, q.N, q.K, q.y, q.ldy)) {
      char msg[sizeof(g_last_error)];
      std::snprintf(msg, sizeof(msg), "%s", g_last_error);
      return fail(st, "problem %d: %s", i, msg);
    }
  }
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_gemm_w4a16_grouped(probs, n, as_stream(stream)), "gemm_w4a16_grouped");
}

int fp4q_gemm_w4a16(const void* a_bf16, int64_t lda, const uint8_t* b_codes, const uint8_t* b_scales,
                    const float* b_tscale, int64_t M, int64_t N, int64_t K, float* y, int64_t ldy,
                    void* stream) {
  g_last_error[0] = 0;
  if (int st = check_w4a16(a_bf16, lda, b_codes, b_scales, b_tscale, M, N, K, y, ldy)) return st;
  if (int st = check_device()) return st;
  return launch_status(fp4q::launch_gemm_w4a16(a_bf16, lda, b_codes, b_scales, b_tscale, M, N, K, y, ldy,
                                               as_stream(stream)),
                       "gemm_w4a16");
}

int fp4q_linear_w4a4(const void* a_bf16, int64_t lda, float* a_tscale, int a_tscale_is_input,
                     const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tscale,
                     int64_t M, int64_t N, int64_t K, float* y, int64_t ldy, void* stream) {
  g_last_error[0] = 0;
  if (!a_bf16 || !a_tscale || !b_codes || !b_scales || !b_tscale || !y) return fail(FP4Q_ERR_NULL_PTR, "operand pointer is NULL");
  if (M < 1 || M > 16) return fail(FP4Q_ERR_BAD_SHAPE, "M must be in [1, 16]");
  if (N <= 0 || K <= 0) return fail(FP4Q_ERR_BAD_SHAPE, "N and K must be > 0");
  if (K % 32) return fail(FP4Q_ERR_BAD_SHAPE, "K must be a multiple of 32");
  if (!fp4q::skinny_supported(K)) return fail(FP4Q_ERR_BAD_SHAPE, "K too large for the fused decode kernel (max 7168)");
  if (lda < K || ldy < N) return fail(FP4Q_ERR_BAD_SHAPE, "lda < K or ldy < N");
  if (reinterpret_cast<uintptr_t>(b_scales) & 7u) return fail(FP4Q_ERR_BAD_ALIGN, "b_scales must be 8-byte aligned");
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return fail(FP4Q_ERR_BAD_SHAPE, "size too large");
  if (!aligned16(a_bf16) || lda % 8 || !aligned16(b_codes)) return fail(FP4Q_ERR_BAD_ALIGN, "a, lda or b_codes not 16-byte aligned");
  if (a_tscale_is_input != 0 && a_tscale_is_input != 1) return fail(FP4Q_ERR_BAD_ARG, "a_tscale_is_input must be 0 or 1");
  if ((reinterpret_cast<uintptr_t>(y) & 3u)) return fail(FP4Q_ERR_BAD_ALIGN, "y must be 4-byte aligned");
  if (int st = check_device()) return st;
  hipStream_t s = as_stream(stream);
  return launch_status(fp4q::launch_gemm_nvfp4_skinny(a_bf16, lda, nullptr, nullptr, a_tscale, !a_tscale_is_input,
                                                      b_codes, b_scales, b_tscale, M, N, K, y, ldy, s),
                       "linear_w4a4");
}

}  // extern "C"
