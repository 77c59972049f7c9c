// Internal helpers shared by the library's HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "gptq.h"

namespace gptq {

// ------------------------------------------------------------ error state
void set_error(const std::string &msg);
gptq_status fail(gptq_status st, const std::string &msg);

// ----------------------------------------------------- launch + profiling
// Every kernel launch goes through launch(): it checks the launch, and when
// profiling is on it brackets the launch with a pair of events on `stream`.
struct ProfileToken {
  hipEvent_t start = nullptr;
  int slot = -1;
};
ProfileToken profile_begin(const char *name, hipStream_t stream);
void profile_end(ProfileToken tok, hipStream_t stream);

template <typename Kernel, typename... Args>
inline gptq_status launch(const char *name, Kernel kernel, dim3 grid, dim3 block,
                          size_t shmem, hipStream_t stream, Args... args) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return GPTQ_OK;
  ProfileToken tok = profile_begin(name, stream);
  hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...);
  hipError_t e = hipGetLastError();
  profile_end(tok, stream);
  if (e != hipSuccess)
    return fail(GPTQ_ERR_DEVICE, std::string("launch of ") + name + " failed: " +
                                     hipGetErrorString(e));
  return GPTQ_OK;
}

// Per-device set-up shared by all entry points, safe to call from several
// host threads at once (a lock guards the caches): raise a kernel's dynamic
// LDS limit on the current device (once per kernel, device and size), and
// the current device's compute-unit count (256 if it cannot be read).
gptq_status allow_dynamic_lds(const void *kernel, size_t bytes);
int device_cu_count();

#define GPTQ_TRY(expr)                  \
  do {                                  \
    gptq_status _st = (expr);           \
    if (_st != GPTQ_OK) return _st;     \
  } while (0)

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------- fp32 GEMM engine
// C = alpha * A * op(B) + beta * C on fp32 MFMA, A row-major M x K.
// op(B) = B (row-major K x N) when transB == 0, B^T (B row-major N x K) when
// transB == 1.  Flags:
//   lower_out  only tiles/elements with row >= col + diag_off are computed and
//              stored (for symmetric updates of a lower triangle);
//   a_lower    A is lower triangular (A[i][k] == 0 for k > i): K range cut;
//   b_lower    op(B) is lower triangular (B[k][j] == 0 for k < j): K range cut.
struct GemmProblem {
  const float *A;
  const float *B;
  float *C;
  int64_t lda, ldb, ldc;
  int32_t M, N, K;
  int32_t tile_begin;  // first tile index of this problem in the grouped grid
  int32_t tiles_n;     // tiles along N
  float alpha, beta;
};
constexpr int kMaxGemmGroup = 40;
struct GemmGroup {
  GemmProblem p[kMaxGemmGroup];
  int32_t count;
  int32_t total_tiles;
  int32_t transB;
  int32_t lower_out;
  int32_t a_lower;
  int32_t b_lower;
};
gptq_status gemm_f32_grouped(const GemmGroup &g, hipStream_t stream, const char *name);
gptq_status gemm_f32(const float *A, int64_t lda, const float *B, int64_t ldb, float *C,
                     int64_t ldc, int M, int N, int K, float alpha, float beta, int transB,
                     int lower_out, int a_lower, int b_lower, hipStream_t stream,
                     const char *name);

// ----------------------------------------------------------- step drivers
gptq_status hessian_accumulate_impl(float *H, double *hdiag, int64_t d, const void *X,
                                    int x_dtype, int64_t n_tok, int64_t ld_x, void *ws,
                                    size_t ws_bytes, hipStream_t stream);
size_t hessian_ws_bytes(int64_t d);
gptq_status prepare_hinv_impl(const float *H, const double *hdiag, int64_t d,
                              const gptq_params &p, float *U, int32_t *perm, uint8_t *dead,
                              void *ws, size_t ws_bytes, hipStream_t stream);
size_t prepare_ws_bytes(int64_t d);
gptq_status quantize_layer_impl(float *W, int64_t rows, int64_t cols, const float *U,
                                const int32_t *perm, const uint8_t *dead, const double *hdiag,
                                const gptq_params &p,
                                uint8_t *q, int32_t *g_idx, float *scale, uint8_t *zero,
                                uint16_t *D, uint16_t *Dm, uint8_t *sc, uint8_t *mc, void *ws,
                                size_t ws_bytes, hipStream_t stream);
size_t quantize_ws_bytes(int64_t rows, int64_t cols, const gptq_params &p);
gptq_status pack_impl(const uint8_t *codes, int64_t rows, int64_t cols, int bits,
                      uint32_t *packed, hipStream_t stream);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace gptq
