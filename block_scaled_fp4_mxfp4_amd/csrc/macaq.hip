// macaq.hip -- weight-side refinement of an MXFP4 weight on gfx950
// ("MACaQ: Fast, Model Agnostic Calibrated Quantization for Low-Precision
// Weights and Activations", "Core method" (iii)-(iv), "Method steps" 0, 3
// and 4): calibration Hessian H = sum_t x_t^T x_t, ridge
// H_f = H + lambda * mean(diag H) * I, Hessian-weighted E8M0 exponent
// screen over {e0, e0 + 1, e0 - 1} (equation 12) and Flip-Refinement
// (Algorithm 1: gain = 2 D g_ij - D^2 (H_f)_jj, g_i <- g_i - D (H_f)_j).
//
// Every quantity is float64 and every sum runs in one fixed sequential
// order, so each decision (an exponent, a flip) is reproducible bit for bit:
//  * H_jk: over tokens in order, starting from the caller's h;
//  * sum of diag H: over j in order (one thread);
//  * block error: over the 32 elements in order (one thread per block);
//  * g_ij = sum_k r_ik (H_f)_kj: over k in order, product rounded, then the
//    add (this file is built with -ffp-contract=off; no fma there).
// A product of two float32 is exact in float64, so the Hessian uses fma.  A
// flip step D is a power of two, so 2 D g, D^2 (H_f)_jj and D (H_f)_jk are
// exact and every gain or update is one rounding.
//
// Ties: the screen keeps e0 unless e0 + 1, then e0 - 1, is strictly
// better; a flip takes the largest gain, the smallest j on ties, the move
// down before the move up.  A zero value is code 0x8 when w has its sign bit
// set; an all-zero block keeps scale byte 0 and codes 0 and is not flipped.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "codec.h"
#include "internal.h"

namespace fp4q {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kWsHd = 32;        // workspace: [0] ridge delta, [32, 32 + n) diag(H_f), then g

__device__ __forceinline__ double pow2d(int32_t e) {          // 2^e, e in [-1022, 1023]
  return __longlong_as_double((long long)(e + 1023) << 52);
}

// Value of flip-grid index gi: 0..14 are -6, -4, -3, -2, -1.5, -1, -0.5, 0,
// 0.5, ..., 6 (the 15 distinct E2M1 values in increasing order).
__device__ __forceinline__ double grid_value(int gi) {
  const int m = gi >= 7 ? gi - 7 : 7 - gi;
  const double v = (double)e2m1_decode((uint32_t)m);
  return gi < 7 ? -v : v;
}

// ------------------------------------------------------------- Hessian ----
// 64 x 64 tile of h per workgroup, 4 x 4 entries per thread; 32 tokens at a
// time staged in LDS as float32 (converted to float64 exactly on use).

constexpr int kHt = 64, kHc = 32;

__global__ __launch_bounds__(kThreads) void k_hessian(const float* __restrict__ x, int64_t T, int64_t n,
                                                      int64_t ldx, double* __restrict__ h) {
  __shared__ float xa[kHc][kHt];
  __shared__ float xb[kHc][kHt];
  const int64_t j0 = (int64_t)blockIdx.y * kHt, k0 = (int64_t)blockIdx.x * kHt;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t j = j0 + ty * 4 + a, k = k0 + tx * 4 + b;
      acc[a][b] = (j < n && k < n) ? h[j * n + k] : 0.0;
    }
  for (int64_t t0 = 0; t0 < T; t0 += kHc) {
    const int cnt = (T - t0) < kHc ? (int)(T - t0) : kHc;
    for (int q = threadIdx.x; q < kHc * kHt; q += kThreads) {
      const int tt = q / kHt, c = q % kHt;
      const bool row = tt < cnt;
      xa[tt][c] = (row && j0 + c < n) ? x[(t0 + tt) * ldx + j0 + c] : 0.0f;
      xb[tt][c] = (row && k0 + c < n) ? x[(t0 + tt) * ldx + k0 + c] : 0.0f;
    }
    __syncthreads();
    for (int tt = 0; tt < cnt; ++tt) {                 // tokens in order
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = (double)xa[tt][ty * 4 + u];
        b[u] = (double)xb[tt][tx * 4 + u];
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = __builtin_fma(a[p], b[q], acc[p][q]);   // exact product
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t j = j0 + ty * 4 + a, k = k0 + tx * 4 + b;
      if (j < n && k < n) h[j * n + k] = acc[a][b];
    }
}

// --------------------------------------------------------------- ridge ----
// delta = lambda * (sum_j h_jj / n), the sum by one thread in order (the
// diagonal staged through LDS 2048 entries at a time, so its loads are
// parallel); then diag(H_f)_j = h_jj + delta for every j.

constexpr int kRc = 2048;

__global__ __launch_bounds__(kThreads) void k_ridge(const double* __restrict__ h, int64_t n, double lam,
                                                    double* __restrict__ ws) {
  __shared__ double dg[kRc];
  __shared__ double s_delta;
  double s = 0.0;
  for (int64_t c0 = 0; c0 < n; c0 += kRc) {
    const int cnt = (n - c0) < kRc ? (int)(n - c0) : kRc;
    for (int q = threadIdx.x; q < cnt; q += kThreads) dg[q] = h[(c0 + q) * n + c0 + q];
    __syncthreads();
    if (threadIdx.x == 0)
      for (int q = 0; q < cnt; ++q) s = s + dg[q];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double d = lam * (s / (double)n);
    s_delta = d;
    ws[0] = d;
  }
  __syncthreads();
  const double d = s_delta;
  for (int64_t j = threadIdx.x; j < n; j += kThreads) ws[kWsHd + j] = h[j * n + j] + d;
}

// -------------------------------------------------------------- screen ----
// One thread per (row, 32-block).

__device__ __forceinline__ double screen_error(const float v[32], const double* __restrict__ hd, int32_t e,
                                               uint32_t pk[4]) {
  const float inv = pow2_neg(e);                       // e in [-127, 126]: a normal float
  const double s = pow2d(e);
  double err = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) pk[q] = 0u;
#pragma unroll
  for (int j = 0; j < 32; ++j) {                       // elements in order
    const uint32_t c = e2m1_encode(v[j] * inv);
    pk[j >> 3] |= c << (4 * (j & 7));
    const double d = (double)v[j] - (double)e2m1_decode(c) * s;   // exact
    err = err + hd[j] * (d * d);
  }
  return err;
}

__global__ __launch_bounds__(kThreads) void k_screen(const float* __restrict__ w, int64_t m, int64_t n,
                                                     int64_t ldw, const double* __restrict__ ws,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t nb = n / 32;
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= m * nb) return;
  const int64_t i = id / nb, b = id - i * nb;
  const float4* p = reinterpret_cast<const float4*>(w + i * ldw + b * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float4 t = p[q];
    v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
  }
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) a = fmaxf(a, __builtin_fabsf(v[j]));
  uint4 out = {0u, 0u, 0u, 0u};
  uint32_t byte = 0u;
  if (a > 0.0f) {
    const double* hd = ws + kWsHd + b * 32;
    const int32_t e0 = mx_block_exponent(a);          // <= 125 for a finite float
    uint32_t best[4], pk[4];
    int32_t be = e0;
    double berr = screen_error(v, hd, e0, best);
    const double eu = screen_error(v, hd, e0 + 1, pk);
    if (eu < berr) {
      berr = eu; be = e0 + 1;
#pragma unroll
      for (int q = 0; q < 4; ++q) best[q] = pk[q];
    }
    if (e0 - 1 >= -127) {
      const double ed = screen_error(v, hd, e0 - 1, pk);
      if (ed < berr) {
        be = e0 - 1;
#pragma unroll
        for (int q = 0; q < 4; ++q) best[q] = pk[q];
      }
    }
    out = make_uint4(best[0], best[1], best[2], best[3]);
    byte = (uint32_t)(be + 127);
  }
  *reinterpret_cast<uint4*>(codes + i * (n / 2) + b * 16) = out;
  scales[i * nb + b] = (uint8_t)byte;
}

// ------------------------------------------------------------ gradient ----
// g = R H_f, R_ik = w_ik - value(code_ik) * 2^e: 64 x 64 output tile per
// workgroup, 4 x 4 per thread, k in chunks of 16 staged in LDS, each output
// summed over k in order.

constexpr int kGt = 64, kGk = 16;

__global__ __launch_bounds__(kThreads) void k_grad(const float* __restrict__ w, int64_t m, int64_t n,
                                                   int64_t ldw, const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scales, const double* __restrict__ h,
                                                   const double* __restrict__ ws, double* __restrict__ g) {
  __shared__ double rs[kGk][kGt];      // [k][i]
  __shared__ double hs[kGk][kGt];      // [k][j]
  const int64_t i0 = (int64_t)blockIdx.y * kGt, j0 = (int64_t)blockIdx.x * kGt;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const double delta = ws[0];
  const int64_t nb = n / 32;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int64_t k0 = 0; k0 < n; k0 += kGk) {            // n % 32 == 0: no partial chunk
    for (int q = threadIdx.x; q < kGk * kGt; q += kThreads) {
      const int ii = q / kGk, kk = q % kGk;
      const int64_t i = i0 + ii, k = k0 + kk;
      double r = 0.0;
      if (i < m) {
        const uint32_t c = (codes[i * (n / 2) + (k >> 1)] >> (4 * (k & 1))) & 0xFu;
        const double s = pow2d((int32_t)scales[i * nb + (k >> 5)] - 127);
        r = (double)w[i * ldw + k] - (double)e2m1_decode(c) * s;          // exact
      }
      rs[kk][ii] = r;
      const int kk2 = q / kGt, jj = q % kGt;
      const int64_t k2 = k0 + kk2, j = j0 + jj;
      double hv = 0.0;
      if (j < n) hv = (k2 == j) ? h[k2 * n + j] + delta : h[k2 * n + j];
      hs[kk2][jj] = hv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGk; ++kk) {                 // k in order
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = rs[kk][ty * 4 + u];
        b[u] = hs[kk][tx * 4 + u];
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const double prod = a[p] * b[q];
          acc[p][q] = acc[p][q] + prod;
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t i = i0 + ty * 4 + a, j = j0 + tx * 4 + b;
      if (i < m && j < n) g[i * n + j] = acc[a][b];
    }
}

// ---------------------------------------------------------------- flip ----
// One workgroup of NT threads per row; thread t owns elements
// j = t + NT u (u < U), with g, diag(H_f), the block exponent and the grid
// index of each in registers.  Each round: every thread scans its elements
// in increasing j, the workgroup reduces (gain, 2j + up, D) to the largest
// gain and smallest index (shuffles, then one LDS slot per wavefront,
// double-buffered so one barrier per round suffices), and every thread
// updates its g with row j of H_f (H_f symmetric as the calibration Hessian
// is).  A 32-block is 32 consecutive threads, so its all-zero flag is one
// ballot.

// log2 |grid[gi - 1] - grid[gi]| + 1 in bits 2 gi, 2 gi + 1 for gi = 1..14
// (steps 2, 1, 1, then eight of 0.5, then 1, 1, 2); the step up from gi is
// the step down from gi + 1
constexpr uint32_t kStepLog2 = 0x25000058u;

__device__ __forceinline__ bool better(double g, int f, double bg, int bf) {
  return g > bg || (g == bg && f < bf);
}

template <int NT, int U>
__global__ __launch_bounds__(NT) void k_flip(const float* __restrict__ w, int64_t n, int64_t ldw,
                                             const double* __restrict__ h, const double* __restrict__ ws,
                                             const double* __restrict__ gin, uint8_t* __restrict__ codes,
                                             const uint8_t* __restrict__ scales, int k_iters,
                                             int32_t* __restrict__ flips) {
  constexpr int kW = NT / 64;
  __shared__ double red_g[2][kW];
  __shared__ double red_d[2][kW];
  __shared__ int red_f[2][kW];
  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const double* hdg = ws + kWsHd;
  const float* wr = w + i * ldw;
  uint8_t* cr = codes + i * (n / 2);
  const int64_t nb = n / 32;

  // per element: g, diag(H_f) and a packed state word
  // (bits 0-3 grid index, 4-11 scale byte, 12 active, 13 sign bit of w)
  double g[U], hd[U];
  uint32_t st[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = tid + (int64_t)NT * u;
    const bool in = j < n;
    const int64_t jc = in ? j : 0;
    const uint32_t wb = __float_as_uint(wr[jc]);
    const uint32_t c = (cr[jc >> 1] >> (4 * (jc & 1))) & 0xFu;
    const uint32_t gix = (c & 8u) ? 7u - (c & 7u) : 7u + (c & 7u);
    hd[u] = hdg[jc];
    g[u] = (k_iters > 0 && in) ? gin[i * n + jc] : 0.0;
    const unsigned long long bal = __ballot(in && (wb & 0x7FFFFFFFu) != 0u);
    const uint32_t half = lane < 32 ? (uint32_t)bal : (uint32_t)(bal >> 32);
    const bool act = in && half != 0u;
    st[u] = gix | ((uint32_t)scales[i * nb + (jc >> 5)] << 4) | (act ? 1u << 12 : 0u) | ((wb >> 31) << 13);
  }

  int nflips = 0;
  for (int it = 0; it < k_iters; ++it) {
    double bg = -__builtin_inf(), bd = 0.0;
    int bf = 0x7FFFFFFF;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!(st[u] & (1u << 12))) continue;
      const int64_t j = tid + (int64_t)NT * u;
      // d = (grid[gi -+ 1] - grid[gi]) * 2^e is a signed power of two,
      // 2^(e + l), with l = log2 of the grid step (kStepLog2), so 2d and
      // d * d are built from the exponent; the gain is then the same
      // rounded expression (2d) g - (d d) hd as with d formed by subtraction
      const int gi = (int)(st[u] & 15u);
      const int e = (int)((st[u] >> 4) & 0xFFu) - 127;
      if (gi > 0) {
        const int a = e + (int)((kStepLog2 >> (2 * gi)) & 3u) - 1;          // d = -2^a
        const double gain = (-pow2d(a + 1)) * g[u] - pow2d(2 * a) * hd[u];
        if (gain > bg) { bg = gain; bf = (int)(2 * j); bd = -pow2d(a); }
      }
      if (gi < 14) {
        const int a = e + (int)((kStepLog2 >> (2 * (gi + 1))) & 3u) - 1;    // d = +2^a
        const double gain = pow2d(a + 1) * g[u] - pow2d(2 * a) * hd[u];
        if (gain > bg) { bg = gain; bf = (int)(2 * j + 1); bd = pow2d(a); }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double og = __shfl_xor(bg, off, 64), od = __shfl_xor(bd, off, 64);
      const int of = __shfl_xor(bf, off, 64);
      if (better(og, of, bg, bf)) { bg = og; bf = of; bd = od; }
    }
    const int buf = it & 1;
    if (lane == 0) { red_g[buf][wave] = bg; red_f[buf][wave] = bf; red_d[buf][wave] = bd; }
    __syncthreads();
    bg = red_g[buf][0]; bf = red_f[buf][0]; bd = red_d[buf][0];
#pragma unroll
    for (int q = 1; q < kW; ++q)
      if (better(red_g[buf][q], red_f[buf][q], bg, bf)) { bg = red_g[buf][q]; bf = red_f[buf][q]; bd = red_d[buf][q]; }
    if (!(bg > 0.0)) break;                            // uniform: no positive gain
    const int64_t j = bf >> 1;
    const double* hr = h + j * n;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = tid + (int64_t)NT * u;
      if (k < n) {
        const double hjk = (k == j) ? hd[u] : hr[k];
        g[u] = g[u] - bd * hjk;                        // bd * hjk exact
        if (k == j) st[u] = (bf & 1) ? st[u] + 1u : st[u] - 1u;   // grid index +-1 (stays in 0..14)
      }
    }
    ++nflips;
  }

  // codes: a zero value takes the sign of w; all-zero blocks stay 0
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = tid + (int64_t)NT * u;
    uint32_t c = 0u;
    if (st[u] & (1u << 12)) {
      const int gi = (int)(st[u] & 15u);
      const uint32_t mag = (uint32_t)(gi >= 7 ? gi - 7 : 7 - gi);
      c = mag | ((gi < 7 || (gi == 7 && (st[u] >> 13) & 1u)) ? 8u : 0u);
    }
    const uint32_t hi = (uint32_t)__shfl_xor((int)c, 1, 64);    // element j + 1 (NT even)
    if (!(tid & 1) && j < n) cr[j >> 1] = (uint8_t)(c | (hi << 4));
  }
  if (flips && tid == 0) flips[i] = nflips;
}

inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

}  // namespace

hipError_t launch_hessian(const float* x, int64_t T, int64_t n, int64_t ldx, double* h, hipStream_t s) {
  const unsigned t = cdiv(n, kHt);
  hipLaunchKernelGGL(k_hessian, dim3(t, t), dim3(kThreads), 0, s, x, T, n, ldx, h);
  return hipGetLastError();
}

namespace {

// Screen, gradient and flips for rows [0, m) of w / codes / scales / flips
// (already offset by the caller); ws holds the ridge delta and diag(H_f)
// from k_ridge and room for an m x n gradient after them.  Rows are
// independent, so any split of the rows gives the same bytes.
void launch_rows(const float* w, int64_t m, int64_t n, int64_t ldw, const double* h, int k_iters,
                 uint8_t* codes, uint8_t* scales, int32_t* flips, double* ws, hipStream_t s) {
  hipLaunchKernelGGL(k_screen, dim3(cdiv(m * (n / 32), kThreads)), dim3(kThreads), 0, s, w, m, n, ldw, ws,
                     codes, scales);
  double* g = ws + kWsHd + ((n + 31) / 32) * 32;
  if (k_iters > 0)
    hipLaunchKernelGGL(k_grad, dim3(cdiv(n, kGt), cdiv(m, kGt)), dim3(kThreads), 0, s, w, m, n, ldw, codes,
                       scales, h, ws, g);
  auto flip = [&](auto kern, int nt) {
    hipLaunchKernelGGL(kern, dim3((unsigned)m), dim3(nt), 0, s, w, n, ldw, h, ws, g, codes, scales, k_iters,
                       flips);
  };
  if (n <= 256) flip(k_flip<256, 1>, 256);
  else if (n <= 512) flip(k_flip<256, 2>, 256);
  else if (n <= 1024) flip(k_flip<256, 4>, 256);
  else if (n <= 2048) flip(k_flip<256, 8>, 256);
  else if (n <= 4096) flip(k_flip<256, 16>, 256);
  else if (n <= 8192) flip(k_flip<512, 16>, 512);
  else flip(k_flip<1024, 16>, 1024);                  // n <= 16384
}

// Workspace of the no-allocation form: one array per device, loaded with
// the code object and held until the process ends.  Host code never names
// it as an address (the host-side symbol is only a stand-in); it uses the
// device address that hipGetSymbolAddress returns, taken once per device.
static __device__ __align__(256) double scratch[kMacaqScratchDoubles];

hipError_t scratch_address(double** out) {
  static std::mutex mu;
  static double* addr[64] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<double*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_macaq_refine(const float* w, int64_t m, int64_t n, int64_t ldw, const double* h, double lam,
                               int k_iters, uint8_t* codes, uint8_t* scales, int32_t* flips, double* ws,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_ridge, dim3(1), dim3(kThreads), 0, s, h, n, lam, ws);
  launch_rows(w, m, n, ldw, h, k_iters, codes, scales, flips, ws, s);
  return hipGetLastError();
}

int64_t macaq_scratch_rows(int64_t n) {
  if (n < 1) return 0;
  return (kMacaqScratchDoubles - kWsHd - ((n + 31) / 32) * 32) / n;
}

hipError_t launch_macaq_refine_static(const float* w, int64_t m, int64_t n, int64_t ldw, const double* h,
                                      double lam, int k_iters, uint8_t* codes, uint8_t* scales, int32_t* flips,
                                      hipStream_t s) {
  const int64_t rows = macaq_scratch_rows(n);
  if (rows < 1) return hipErrorInvalidValue;
  double* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_ridge, dim3(1), dim3(kThreads), 0, s, h, n, lam, ws);
  for (int64_t r0 = 0; r0 < m; r0 += rows) {
    const int64_t mc = m - r0 < rows ? m - r0 : rows;
    launch_rows(w + r0 * ldw, mc, n, ldw, h, k_iters, codes + r0 * (n / 2), scales + r0 * (n / 32),
                flips ? flips + r0 : nullptr, ws, s);
  }
  return hipGetLastError();
}

}  // namespace fp4q
