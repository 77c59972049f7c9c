// A layer's outputs computed with its updated weight, as the next layer's
// calibration inputs ("GPTQ implementation with tensor subclasses", section
// Background: track the activations reaching a linear, update its weight,
// use the updated weight to generate that linear's outputs, go on to the
// next linear).
//
// Activations keep the layout the Hessian accumulation reads: features x
// tokens, bf16, tokens contiguous.  The product runs on the fp32 MFMA GEMM
// (bf16 inputs widen exactly), and each output is rounded to bf16 once.
#include <algorithm>
#include <cmath>
#include <string>

#include "common.h"

namespace gptq {
namespace {

constexpr int kThreads = 256;

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ inline uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__global__ __launch_bounds__(kThreads) void widen_bf16_kernel(
    const uint16_t *__restrict__ X, int64_t rows, int64_t n, int64_t ld,
    float *__restrict__ Y) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= rows * n) return;
  const int64_t r = i / n, t = i - r * n;
  Y[i] = bf16_to_f32(X[r * ld + t]);
}

__global__ __launch_bounds__(kThreads) void narrow_bf16_kernel(
    const float *__restrict__ Y, int64_t rows, int64_t n, uint16_t *__restrict__ out,
    int64_t ld_out) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= rows * n) return;
  const int64_t r = i / n, t = i - r * n;
  out[r * ld_out + t] = f32_to_bf16(Y[i]);
}

// A = bf16(silu(G) * U), silu(g) = g / (1 + e^-g), in float32.
__global__ __launch_bounds__(kThreads) void silu_mul_kernel(
    const uint16_t *__restrict__ G, const uint16_t *__restrict__ U, int64_t rows, int64_t n,
    int64_t ld, uint16_t *__restrict__ A, int64_t ld_a) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= rows * n) return;
  const int64_t r = i / n, t = i - r * n;
  const float g = bf16_to_f32(G[r * ld + t]), u = bf16_to_f32(U[r * ld + t]);
  const float s = g / (1.f + expf(-g));
  A[r * ld_a + t] = f32_to_bf16(s * u);
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" {

size_t gptq_linear_forward_ws_bytes(int64_t rows, int64_t cols, int64_t n_tok) {
  if (rows < 1 || cols < 1 || n_tok < 0) return 0;
  return align256(sizeof(float) * size_t(cols) * size_t(n_tok)) +
         align256(sizeof(float) * size_t(rows) * size_t(n_tok)) + 256;
}

gptq_status gptq_linear_forward(const float *W, int64_t rows, int64_t cols, const uint16_t *X,
                                int64_t n_tok, int64_t ld_x, uint16_t *Y, int64_t ld_y,
                                void *ws, size_t ws_bytes, void *stream) {
  if (rows < 1 || cols < 1 || rows > (int64_t(1) << 24) || cols > (int64_t(1) << 20))
    return fail(GPTQ_ERR_INVALID_ARG, "rows and cols must be in [1, 2^24] x [1, 2^20]");
  if (n_tok < 0 || n_tok > (int64_t(1) << 30))
    return fail(GPTQ_ERR_INVALID_ARG, "n_tok must be in [0, 2^30]");
  if (n_tok == 0) return GPTQ_OK;
  if (!W || !X || !Y) return fail(GPTQ_ERR_INVALID_ARG, "W, X and Y must not be NULL");
  if (ld_x < n_tok || ld_y < n_tok)
    return fail(GPTQ_ERR_INVALID_ARG, "ld_x and ld_y must be >= n_tok");
  if (rows > INT32_MAX || cols > INT32_MAX || n_tok > INT32_MAX)
    return fail(GPTQ_ERR_INVALID_ARG, "sizes exceed the GEMM's 32-bit extents");
  const size_t need = gptq_linear_forward_ws_bytes(rows, cols, n_tok);
  if (!ws) return fail(GPTQ_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(GPTQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(GPTQ_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) +
                                        " bytes, got " + std::to_string(ws_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *X32 = static_cast<float *>(ws);
  float *Y32 = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                         align256(sizeof(float) * size_t(cols) * size_t(n_tok)));
  const int64_t nx = cols * n_tok, ny = rows * n_tok;
  GPTQ_TRY(launch("fwd_widen", widen_bf16_kernel, dim3(cdiv(nx, kThreads)), dim3(kThreads), 0,
                  s, X, cols, n_tok, ld_x, X32));
  GPTQ_TRY(gemm_f32(W, cols, X32, n_tok, Y32, n_tok, int(rows), int(n_tok), int(cols), 1.f, 0.f,
                    0, 0, 0, 0, s, "fwd_gemm"));
  GPTQ_TRY(launch("fwd_narrow", narrow_bf16_kernel, dim3(cdiv(ny, kThreads)), dim3(kThreads), 0,
                  s, (const float *)Y32, rows, n_tok, Y, ld_y));
  return GPTQ_OK;
}

gptq_status gptq_silu_mul(const uint16_t *G, const uint16_t *U, int64_t rows, int64_t n_tok,
                          int64_t ld, uint16_t *A, int64_t ld_a, void *stream) {
  if (rows < 1 || n_tok < 0) return fail(GPTQ_ERR_INVALID_ARG, "rows >= 1 and n_tok >= 0");
  if (n_tok == 0) return GPTQ_OK;
  if (!G || !U || !A) return fail(GPTQ_ERR_INVALID_ARG, "G, U and A must not be NULL");
  if (ld < n_tok || ld_a < n_tok) return fail(GPTQ_ERR_INVALID_ARG, "ld and ld_a must be >= n_tok");
  const int64_t total = rows * n_tok;
  return launch("fwd_silu_mul", silu_mul_kernel, dim3(cdiv(total, kThreads)), dim3(kThreads), 0,
                static_cast<hipStream_t>(stream), G, U, rows, n_tok, ld, A, ld_a);
}

}  // extern "C"
