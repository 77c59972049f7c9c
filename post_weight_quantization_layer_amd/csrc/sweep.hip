// Column-by-column quantization with Optimal Brain Surgeon compensation and
// lazy block updates ("GPTQ", section Jak dziala; section Komponenty: block
// updates), on the affine per-group grid or the two-level Q4_K grid ("Add
// gguf q4_k quantization", summary).
//
// For each block of B <= 128 columns (processing order):
//   sweep kernel    one wavefront per row; lane l holds the row's block
//                   columns l and l+64 in registers; the B x B block of U sits
//                   in LDS.  Step j broadcasts w_j (readlane), quantizes it,
//                   forms e_j = (w_j - q(w_j)) / U_jj and updates the lanes'
//                   later columns with -e_j U_jk.  Group grids are chosen at a
//                   group's first column with wavefront min/max reductions.
//                   Writes the block's w^ and codes, and e_j into Err.
//   trailing GEMM   W[:, i2:] -= Err * U[block, i2:] on fp32 MFMA.
//
// Grid decisions (scale, zero, code) are taken in fp32 with IEEE division
// and round-half-to-even (v_rndne_f32), fp16 super-scales with
// round-to-nearest-even.
#include <algorithm>

#include "common.h"

namespace gptq {
namespace {

constexpr int kMaxB = 128;
constexpr int kSweepThreads = 512;  // 8 wavefronts, one row each at a time
constexpr int kSweepMaxWG = 512;

struct SweepArgs {
  float *W;        // working weights, row-major, ld = cols (processing order)
  uint8_t *q;      // codes, ld = cols
  float *Err;      // rows x kMaxB
  const float *U;  // ld = cols
  int64_t rows, cols;
  int i1, B;
  int bits, group;
  float *scale;    // affine: rows x (cols/group)
  uint8_t *zero;
  uint16_t *D, *Dm;   // q4k: rows x (cols/256)
  uint8_t *sc, *mc;   // q4k: rows x (cols/32)
};

__device__ __forceinline__ float bcast(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

__device__ __forceinline__ float wave_min(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_max(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// float -> IEEE half bits, round to nearest even (subnormals exact).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  const uint32_t x = __float_as_uint(f);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t a = x & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);
  if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);  // rounds to inf
  if (a >= 0x38800000u) {                                  // normal half
    uint32_t r = a - 0x38000000u;
    r += 0xfffu + ((r >> 13) & 1u);
    return (uint16_t)(sign | (r >> 13));
  }
  const float m = __builtin_rintf(__uint_as_float(a) * 16777216.0f);  // units of 2^-24
  return (uint16_t)(sign | (uint32_t)m);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  const uint32_t sign = uint32_t(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
  if (e == 0) {
    const float v = float(m) * 5.9604644775390625e-08f;  // m * 2^-24, exact
    return __uint_as_float(__float_as_uint(v) | sign);
  }
  if (e == 31) return __uint_as_float(sign | 0x7f800000u | (m << 13));
  return __uint_as_float(sign | ((e + 112u) << 23) | (m << 13));
}

template <int kQ4K>
__global__ void __launch_bounds__(kSweepThreads) sweep_kernel(SweepArgs a) {
  extern __shared__ float Ub[];  // B x kMaxB, upper part of U's block
  const int tid = threadIdx.x;
  const int B = a.B;
  const int64_t ld = a.cols;
  for (int e = tid; e < B * B; e += kSweepThreads) {
    const int j = e / B, k = e % B;
    Ub[j * kMaxB + k] = k >= j ? a.U[int64_t(a.i1 + j) * ld + a.i1 + k] : 0.f;
  }
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int64_t nwaves = int64_t(gridDim.x) * (kSweepThreads / 64);
  const int G = kQ4K ? 256 : a.group;
  const float maxq = float((1 << a.bits) - 1);
  const bool v0 = lane < B, v1 = lane + 64 < B;
  const int64_t ngroups = a.cols / G;

  for (int64_t row = int64_t(blockIdx.x) * (kSweepThreads / 64) + wave; row < a.rows;
       row += nwaves) {
    float *wrow = a.W + row * ld + a.i1;
    float w0 = v0 ? wrow[lane] : 0.f;
    float w1 = v1 ? wrow[64 + lane] : 0.f;
    float q0 = 0.f, q1 = 0.f, e0 = 0.f, e1 = 0.f;

    // grid state of the current group
    float s = 1.f, z = 0.f;           // affine
    float Sv = 0.f, Mv = 0.f;         // q4k: lane b < 8 holds S_b, M_b

    if (a.i1 % G != 0) {  // group began in an earlier block: read its grid back
      const int64_t gi = a.i1 / G;
      if (!kQ4K) {
        s = a.scale[row * ngroups + gi];
        z = float(a.zero[row * ngroups + gi]);
      } else {
        const float Df = f16_to_f32(a.D[row * ngroups + gi]);
        const float Dmf = f16_to_f32(a.Dm[row * ngroups + gi]);
        if (lane < 8) {
          const int64_t sb = row * (a.cols / 32) + gi * 8 + lane;
          Sv = Df * float(a.sc[sb]);
          Mv = Dmf * float(a.mc[sb]);
        }
      }
    }

    for (int j = 0; j < B; ++j) {
      const int col = a.i1 + j;
      if (col % G == 0) {
        const int64_t gi = col / G;
        if (!kQ4K) {
          float mn = INFINITY, mx = -INFINITY;
          if (v0 && lane >= j && lane < j + G) {
            mn = w0;
            mx = w0;
          }
          if (v1 && lane + 64 >= j && lane + 64 < j + G) {
            mn = fminf(mn, w1);
            mx = fmaxf(mx, w1);
          }
          for (int c = B + lane; c < j + G; c += 64) {  // group reaches past the block
            const float v = wrow[c];
            mn = fminf(mn, v);
            mx = fmaxf(mx, v);
          }
          mn = wave_min(mn, 64);
          mx = wave_max(mx, 64);
          float xmin = fminf(mn, 0.f), xmax = fmaxf(mx, 0.f);
          if (xmin == xmax) {
            xmin = -1.f;
            xmax = 1.f;
          }
          s = (xmax - xmin) / maxq;
          z = fminf(fmaxf(__builtin_rintf(-xmin / s), 0.f), maxq);
          if (lane == 0) {
            a.scale[row * ngroups + gi] = s;
            a.zero[row * ngroups + gi] = (uint8_t)z;
          }
        } else {
          // super-block of 256 starting at this column (always a block start)
          float sb_s[4], sb_m[4];
          float smax = 0.f, mmax = 0.f;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int p = lane + 64 * t;
            float v;
            if (p < B) v = (t == 0) ? w0 : w1;
            else v = wrow[p];
            float mn = wave_min(v, 32), mx = wave_max(v, 32);
            mn = fminf(mn, 0.f);
            mx = fmaxf(mx, 0.f);
            sb_s[t] = (mx - mn) / 15.f;
            sb_m[t] = -mn;
            smax = fmaxf(smax, sb_s[t]);
            mmax = fmaxf(mmax, sb_m[t]);
          }
          smax = fmaxf(smax, __shfl_xor(smax, 32));
          mmax = fmaxf(mmax, __shfl_xor(mmax, 32));
          const uint16_t Dh = f32_to_f16_rne(smax / 63.f);
          const uint16_t Dmh = f32_to_f16_rne(mmax / 63.f);
          const float Df = f16_to_f32(Dh), Dmf = f16_to_f32(Dmh);
          float Sb[4], Mb[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float scq = (sb_s[t] > 0.f && Df > 0.f)
                                  ? fminf(fmaxf(__builtin_rintf(sb_s[t] / Df), 1.f), 63.f)
                                  : 0.f;
            const float mcq =
                (Dmf > 0.f) ? fminf(fmaxf(__builtin_rintf(sb_m[t] / Dmf), 0.f), 63.f) : 0.f;
            Sb[t] = Df * scq;
            Mb[t] = Dmf * mcq;
            if ((lane & 31) == 0) {
              const int b = 2 * t + (lane >> 5);
              const int64_t o = row * (a.cols / 32) + gi * 8 + b;
              a.sc[o] = (uint8_t)scq;
              a.mc[o] = (uint8_t)mcq;
            }
          }
          if (lane == 0) {
            a.D[row * ngroups + gi] = Dh;
            a.Dm[row * ngroups + gi] = Dmh;
          }
          // lane b < 8 <- S_b, M_b (b = 2t + half)
          float sv = 0.f, mv = 0.f;
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const float S_ = bcast(Sb[b >> 1], (b & 1) * 32);
            const float M_ = bcast(Mb[b >> 1], (b & 1) * 32);
            if (lane == b) {
              sv = S_;
              mv = M_;
            }
          }
          Sv = sv;
          Mv = mv;
        }
      }

      const float wj = bcast(j < 64 ? w0 : w1, j & 63);
      float qj, wq;
      if (!kQ4K) {
        qj = fminf(fmaxf(__builtin_rintf(wj / s) + z, 0.f), maxq);
        wq = s * (qj - z);
      } else {
        const int b = (col & 255) >> 5;
        const float S = bcast(Sv, b), M = bcast(Mv, b);
        qj = (S > 0.f) ? fminf(fmaxf(__builtin_rintf((wj + M) / S), 0.f), 15.f) : 0.f;
        wq = S * qj - M;
      }
      const float ej = (wj - wq) / Ub[j * kMaxB + j];
      const float u0 = Ub[j * kMaxB + lane];
      const float u1 = Ub[j * kMaxB + 64 + lane];
      if (v0 && lane > j) w0 = fmaf(-ej, u0, w0);
      if (v1 && lane + 64 > j) w1 = fmaf(-ej, u1, w1);
      if (lane == (j & 63)) {
        if (j < 64) {
          w0 = wq;
          q0 = qj;
          e0 = ej;
        } else {
          w1 = wq;
          q1 = qj;
          e1 = ej;
        }
      }
    }

    uint8_t *qrow = a.q + row * ld + a.i1;
    float *erow = a.Err + row * kMaxB;
    if (v0) {
      wrow[lane] = w0;
      qrow[lane] = (uint8_t)q0;
      erow[lane] = e0;
    }
    if (v1) {
      wrow[64 + lane] = w1;
      qrow[64 + lane] = (uint8_t)q1;
      erow[64 + lane] = e1;
    }
  }
}

// Wp[r][p] = dead[perm[p]] ? 0 : W[r][perm[p]]
__global__ void __launch_bounds__(256)
    gather_cols_kernel(const float *__restrict__ W, int64_t rows, int64_t cols, const int32_t *__restrict__ perm,
                       const uint8_t *__restrict__ dead, float *__restrict__ Wp) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    for (int64_t p = int64_t(blockIdx.x) * 256 + threadIdx.x; p < cols;
         p += int64_t(gridDim.x) * 256) {
      const int32_t c = perm[p];
      Wp[r * cols + p] = dead[c] ? 0.f : W[r * cols + c];
    }
}

// W[r][perm[p]] = Wp[r][p], q[r][perm[p]] = qp[r][p]
__global__ void __launch_bounds__(256)
    scatter_cols_kernel(const float *__restrict__ Wp, const uint8_t *__restrict__ qp, int64_t rows,
                        int64_t cols,
                        const int32_t *__restrict__ perm, float *__restrict__ W,
                        uint8_t *__restrict__ q) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    for (int64_t p = int64_t(blockIdx.x) * 256 + threadIdx.x; p < cols;
         p += int64_t(gridDim.x) * 256) {
      const int32_t c = perm[p];
      W[r * cols + c] = Wp[r * cols + p];
      q[r * cols + c] = qp[r * cols + p];
    }
}

__global__ void __launch_bounds__(256)
    zero_dead_kernel(float *__restrict__ W, int64_t rows, int64_t cols,
                     const uint8_t *__restrict__ dead) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    for (int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x; c < cols;
         c += int64_t(gridDim.x) * 256)
      if (dead[c]) W[r * cols + c] = 0.f;
}

__global__ void __launch_bounds__(256)
    g_idx_kernel(const int32_t *__restrict__ perm, int64_t cols, int gsz, int32_t *__restrict__ g_idx) {
  const int64_t p = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (p < cols) g_idx[perm[p]] = (int32_t)(p / gsz);
}

bool g_sweep_lds_set[2] = {false, false};

}  // namespace

size_t quantize_ws_bytes(int64_t rows, int64_t cols, const gptq_params &p) {
  size_t n = align256(size_t(rows) * kMaxB * sizeof(float));  // Err
  if (p.act_order) {
    n += align256(size_t(rows) * size_t(cols) * sizeof(float));  // Wp
    n += align256(size_t(rows) * size_t(cols));                  // qp
  }
  return n;
}

gptq_status quantize_layer_impl(float *W, int64_t rows, int64_t cols, const float *U,
                                const int32_t *perm, const uint8_t *dead, const gptq_params &p,
                                uint8_t *q, int32_t *g_idx, float *scale, uint8_t *zero,
                                uint16_t *D, uint16_t *Dm, uint8_t *sc, uint8_t *mc, void *ws,
                                size_t ws_bytes, hipStream_t stream) {
  (void)ws_bytes;
  uint8_t *base = static_cast<uint8_t *>(ws);
  float *Err = reinterpret_cast<float *>(base);
  base += align256(size_t(rows) * kMaxB * sizeof(float));
  float *Wp = W;
  uint8_t *qp = q;
  const unsigned gx = (unsigned)std::min<int64_t>(cdiv(cols, 256), 64);
  const unsigned gy = (unsigned)std::min<int64_t>(rows, 16384);
  if (p.act_order) {
    Wp = reinterpret_cast<float *>(base);
    base += align256(size_t(rows) * size_t(cols) * sizeof(float));
    qp = base;
    GPTQ_TRY(launch("quant_gather", gather_cols_kernel, dim3(gx, gy), dim3(256), 0, stream,
                    (const float *)W, rows, cols, perm, dead, Wp));
  } else {
    GPTQ_TRY(launch("quant_zero_dead", zero_dead_kernel, dim3(gx, gy), dim3(256), 0, stream,
                    W, rows, cols, dead));
  }

  const int q4k = p.grid == GPTQ_GRID_Q4K;
  const int B = p.block;
  const size_t lds = size_t(B) * kMaxB * sizeof(float);
  if (lds > 65536 && !g_sweep_lds_set[q4k]) {
    hipError_t e = hipFuncSetAttribute(
        q4k ? (const void *)sweep_kernel<1> : (const void *)sweep_kernel<0>,
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
      return fail(GPTQ_ERR_DEVICE, std::string("cannot raise LDS limit: ") + hipGetErrorString(e));
    g_sweep_lds_set[q4k] = true;
  }
  const unsigned nwg = (unsigned)std::min<int64_t>(cdiv(rows, kSweepThreads / 64), kSweepMaxWG);

  SweepArgs a{};
  a.W = Wp;
  a.q = qp;
  a.Err = Err;
  a.U = U;
  a.rows = rows;
  a.cols = cols;
  a.bits = p.bits;
  a.group = p.group;
  a.scale = scale;
  a.zero = zero;
  a.D = D;
  a.Dm = Dm;
  a.sc = sc;
  a.mc = mc;
  for (int64_t i1 = 0; i1 < cols; i1 += B) {
    const int Bc = (int)std::min<int64_t>(B, cols - i1);
    a.i1 = (int)i1;
    a.B = Bc;
    if (q4k)
      GPTQ_TRY(launch("sweep_q4k", sweep_kernel<1>, dim3(nwg), dim3(kSweepThreads), lds, stream, a));
    else
      GPTQ_TRY(launch("sweep_affine", sweep_kernel<0>, dim3(nwg), dim3(kSweepThreads), lds, stream,
                      a));
    const int64_t i2 = i1 + Bc;
    if (i2 < cols) {
      GPTQ_TRY(gemm_f32(Err, kMaxB, U + i1 * cols + i2, cols, Wp + i2, cols, (int)rows,
                        (int)(cols - i2), Bc, -1.f, 1.f, 0, 0, 0, 0, stream, "trailing_gemm"));
    }
  }

  if (p.act_order)
    GPTQ_TRY(launch("quant_scatter", scatter_cols_kernel, dim3(gx, gy), dim3(256), 0, stream,
                    (const float *)Wp, (const uint8_t *)qp, rows, cols, perm, W, q));
  const int gsz = q4k ? 32 : p.group;
  GPTQ_TRY(launch("quant_g_idx", g_idx_kernel, dim3((unsigned)cdiv(cols, 256)), dim3(256), 0, stream,
                  perm, cols, gsz, g_idx));
  return GPTQ_OK;
}

}  // namespace gptq
