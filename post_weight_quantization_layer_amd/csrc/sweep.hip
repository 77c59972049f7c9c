// Column-by-column quantization with Optimal Brain Surgeon compensation and
// lazy block updates ("GPTQ", section Jak dziala; section Komponenty: block
// updates), on the affine per-group grid or the two-level Q4_K grid ("Add
// gguf q4_k quantization", summary).
//
// For each block of B <= 128 columns (processing order):
//   sweep kernel    a wavefront holds 4 rows of the block in registers, 16
//                   lanes per row and 8 columns per lane; the B x B block of
//                   U and the reciprocals of its diagonal sit in LDS.  Step j
//                   broadcasts w_j within the row's lanes, quantizes it,
//                   forms e_j = (w_j - q(w_j)) / U_jj and updates the lanes'
//                   later columns with -e_j U_jk.  Group grids are chosen at a
//                   group's first column with 16-lane min/max reductions.
//                   Writes the block's w^ and codes, and e_j into Err.  One
//                   launch sweeps a whole super-block of blocks; before each
//                   block a workgroup applies the earlier blocks' errors to
//                   its own rows (near_update, fp32 MFMA).
//   trailing GEMMs  on fp32 MFMA: after a super-block its errors reach the
//                   rest of its far group, after a far group every later
//                   column (see the host loop below).
//
// Grid decisions (scale, zero, code) are taken in fp32 with IEEE division
// and round-half-to-even (v_rndne_f32), fp16 super-scales with
// round-to-nearest-even.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace gptq {
namespace {

constexpr int kMaxB = 128;
constexpr int kMaxSuper = 512;      // columns per lazy super-block (one sweep launch)
constexpr int kMaxGroupCols = 2048; // columns per far-update group of super-blocks
constexpr int kSweepThreads = 256;  // 4 wavefronts, 4 rows each at a time
constexpr int kSweepMaxWG = 512;

struct SweepArgs {
  float *W;        // working weights, row-major, ld = cols (processing order)
  uint8_t *q;      // codes, ld = cols
  float *Err;      // the super-block's first column of the error buffer, ld = ldE
  int ldE;
  const float *U;  // ld = cols
  // Hessian-factor route (null on the inverse-factor route): the weights
  // before any compensation, processing order, ld = cols.  U then holds the
  // inverse factor's diagonal blocks U_BB (B = 128), and above each of them
  // R_{<B,B} U_BB, R the Hessian's reversed Cholesky factor (Hp = R R^T).
  const float *Wo;
  int64_t rows, cols;
  int s1, B, nblk; // nblk blocks of B columns from column s1 (the last may be shorter)
  int gblk;        // blocks per group when a group spans several blocks of a launch, else 1
  int bits, group;
  int sub_bits;    // two-level grid: width of the sub-block scale/min codes
  int search;      // affine: importance-weighted grid choice
  const double *hp;  // search: importance of each column, processing order
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

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Half-width of the window around a half-integer inside which y = num * rden
// (rden = 1/den rounded) and the IEEE quotient num / den may round to
// different integers.  rden and the product each carry a relative error of
// at most 2^-24, and the IEEE quotient one more, so the two differ by at most
// |y| * 3 * 2^-24 < |y| * 1.8e-7; the window is 1e-5 + |y| * 2.5e-7.  With the
// zero point the quotient reaches |num/den| = 2^bits - 1 (255 at 8 bits,
// where the relative term is 6.4e-5).
__device__ __forceinline__ float tie_window(float y) { return fmaf(fabsf(y), 2.5e-7f, 1e-5f); }

// rint(num / den) exactly as if num / den were computed with a correctly
// rounded IEEE division: the quotient is formed as num * rden and only when
// that lands inside tie_window of a half-integer -- where the two roundings
// could disagree -- is the IEEE division done.  The exact path is a
// wavefront-uniform branch taken only when some lane is near a tie.
__device__ __forceinline__ float rint_div(float num, float den, float rden) {
  const float y = num * rden;
  float r = __builtin_rintf(y);
  const bool near = fabsf(y - floorf(y) - 0.5f) < tie_window(y);
  if (__builtin_expect(__any(near), 0)) r = near ? __builtin_rintf(num / den) : r;
  return r;
}

// Row groups: a wavefront sweeps 4 rows at once, 16 lanes per row, each
// lane owning 8 contiguous block columns (B <= 128).  The per-column chain
// (quantize w_j, error, update) is computed by the 16 lanes of a row group
// together, so every instruction of the chain serves 4 rows.
constexpr int kLPR = 16;  // lanes per row
constexpr int kCPL = 8;   // columns per lane

__device__ __forceinline__ float shfl(float v, int src) { return __shfl(v, src); }

// Value of sub-lane `sub` of this lane's row group, for all four groups at
// once: four readlanes (VALU, no LDS round trip) and a select.
__device__ __forceinline__ float group_bcast(float v, int sub, int grp) {
  const float g0 = bcast(v, sub), g1 = bcast(v, 16 + sub);
  const float g2 = bcast(v, 32 + sub), g3 = bcast(v, 48 + sub);
  return grp < 2 ? (grp == 0 ? g0 : g1) : (grp == 2 ? g2 : g3);
}

__device__ __forceinline__ float group_min(float v) {
#pragma unroll
  for (int off = 1; off < kLPR; off <<= 1) v = fminf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = 1; off < kLPR; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
// Butterfly sum over the row's 16 lanes: every lane adds the same pairs
// (addition commutes exactly), so all of them hold the same bits.
__device__ __forceinline__ double group_sum(double v) {
#pragma unroll
  for (int off = 1; off < kLPR; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// Value of lane `sub` of this lane's 16-lane row, by a DPP row broadcast
// (one VALU move; the source lane is an immediate).
template <int kSub>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + kSub, 0xf, 0xf, false));
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// kG8: the group size is a multiple of 8, so groups start only at the first
// column of an 8-column step (the check runs once per 8 columns).
// One block [i1, i1 + B) of the sweep for all of this workgroup's rows.
template <int kQ4K, bool kG8, bool kH>
__device__ __forceinline__ void sweep_block(const SweepArgs &a, const int i1, const int B,
                                            float *const Err) {
  // LDS: U's block (rows 0 .. Bp+1 of kMaxB floats, Bp = B rounded up to 8,
  // rows and columns past B zero: the fast pass reads two rows ahead), then
  // Bp + 2 reciprocals of the diagonal (zero past B, so padding steps change
  // nothing).
  extern __shared__ __align__(16) float Ub[];
  const int Bp = (B + 7) & ~7;
  float *Uinv = Ub + (Bp + 2) * kMaxB;
  // search: the block's column importances (doubles, 8-byte aligned)
  double *hs = reinterpret_cast<double *>(Uinv + ((Bp + 2 + 1) & ~1));
  const int tid = threadIdx.x;
  const int64_t ld = a.cols;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, sl = lane & 15;
  const int gbase = lane & 48;  // first lane of this row group
  const int c0 = sl * kCPL;     // first block column owned by this lane
  const int G = kQ4K ? 256 : a.group;
  const float maxq = float((1 << a.bits) - 1);
  const float kmax = float((1 << a.sub_bits) - 1);   // two-level grid: sub-code limit
  const int64_t ngroups = a.cols / G;
  const int64_t rows_per_pass = int64_t(gridDim.x) * (kSweepThreads / 64) * 4;
  // 16-byte W accesses need a 4-float aligned row stride and block start
  const bool vec = (ld & 3) == 0 && (i1 & 3) == 0;
  const bool evec = (a.ldE & 3) == 0 && (reinterpret_cast<uintptr_t>(Err) & 15) == 0;
  const bool full = vec && c0 + kCPL <= B;  // this lane's 8 columns, 16-byte accesses

  // The first row group's weights are requested before the U block, so the
  // two latencies overlap.
  // w: current weights of this lane's 8 block columns; o: the same columns
  // before any compensation (Hessian-factor route only)
  float w[kCPL], o[kCPL] = {};
  // Hessian-factor route (a.Wo set): the block arrives compensated by the
  // updates through F = R U_BB above the diagonal blocks, is swept on U_BB
  // like the inverse route, and hands on the error w^_j - o_j
  const bool hroute = kH && a.Wo != nullptr;
  auto load_w = [&](int64_t r0) {
    const int64_t rowc = min(r0 + grp, a.rows - 1);
    const float *wrow = a.W + rowc * ld + i1;
    if (full) {
      const f32x4_t t0 = *reinterpret_cast<const f32x4_t *>(wrow + c0);
      const f32x4_t t1 = *reinterpret_cast<const f32x4_t *>(wrow + c0 + 4);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        w[x] = t0[x];
        w[4 + x] = t1[x];
      }
      if (hroute) {
        const float *orow = a.Wo + rowc * ld + i1;
        const f32x4_t v0 = *reinterpret_cast<const f32x4_t *>(orow + c0);
        const f32x4_t v1 = *reinterpret_cast<const f32x4_t *>(orow + c0 + 4);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          o[x] = v0[x];
          o[4 + x] = v1[x];
        }
      }
    } else {
#pragma unroll
      for (int x = 0; x < kCPL; ++x) w[x] = (c0 + x < B) ? wrow[c0 + x] : 0.f;
    }
  };
  int64_t r0 = (int64_t(blockIdx.x) * (kSweepThreads / 64) + wave) * 4;
  if (r0 < a.rows) load_w(r0);

  // U block: rows i1 .. i1+B-1, columns i1 .. i1+B-1, all loads of a thread
  // in one batch before any use; the diagonal's reciprocals from loads of
  // their own.
  const float *Ublk = a.U + int64_t(i1) * ld + i1;
  const float udiag = Ublk[int64_t(min(tid, B - 1)) * (ld + 1)];
  if ((ld & 3) == 0 && (i1 & 3) == 0 && (B & 3) == 0) {
    constexpr int kPer = kMaxB * kMaxB / 4 / kSweepThreads;  // float4 chunks per thread
    const int nq = B * B / 4;
    f32x4_t v[kPer];
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const int e = min(tid + t * kSweepThreads, nq - 1);
      const int j = e / (B / 4), k = (e % (B / 4)) * 4;
      // chunks wholly left of the diagonal are zero in LDS: not fetched
      v[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (k + 3 >= j) v[t] = *reinterpret_cast<const f32x4_t *>(Ublk + int64_t(j) * ld + k);
    }
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const int e = tid + t * kSweepThreads;
      if (e < nq) {
        const int j = e / (B / 4), k = (e % (B / 4)) * 4;
        f32x4_t u;
#pragma unroll
        for (int x = 0; x < 4; ++x) u[x] = (k + x >= j) ? v[t][x] : 0.f;
        *reinterpret_cast<f32x4_t *>(Ub + j * kMaxB + k) = u;
      }
    }
  } else {
    for (int e = tid; e < B * B; e += kSweepThreads) {
      const int j = e / B, k = e % B;
      const float u = Ublk[int64_t(j) * ld + k];
      Ub[j * kMaxB + k] = k >= j ? u : 0.f;
    }
  }
  if (tid < B) Uinv[tid] = 1.f / udiag;
  // columns past B of rows < B, and the padding rows B .. Bp+1, are zero
  for (int e = tid; e < B * (kMaxB - B); e += kSweepThreads)
    Ub[(e / (kMaxB - B)) * kMaxB + B + e % (kMaxB - B)] = 0.f;
  for (int e = tid; e < (Bp + 2 - B) * kMaxB; e += kSweepThreads) Ub[B * kMaxB + e] = 0.f;
  for (int j = B + tid; j < Bp + 2; j += kSweepThreads) Uinv[j] = 0.f;
  if (a.search)
    for (int c = tid; c < B; c += kSweepThreads) hs[c] = a.hp[i1 + c];
  __syncthreads();

  for (; r0 < a.rows; r0 += rows_per_pass) {
    // The row group's weights have arrived.  Waiting here explicitly keeps
    // the compiler from waiting at every step instead, where the counter
    // would also cover the previous steps' result stores.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    const int64_t row = r0 + grp;
    const bool rv = row < a.rows;  // whole row group is valid or not
    const int64_t rowc = rv ? row : a.rows - 1;
    float *wrow = a.W + rowc * ld + i1;

    // grid state of the current group (per row group, identical in its lanes)
    float s = 1.f, rs = 1.f, z = 0.f;       // affine
    float Sv = 0.f, Mv = 0.f, rSv = 0.f;    // q4k: sub-lane b < 8 holds S_b, M_b, 1/S_b

    if (i1 % G != 0) {  // group began in an earlier block: read its grid back
      const int64_t gi = i1 / G;
      if (!kQ4K) {
        s = a.scale[rowc * ngroups + gi];
        rs = 1.f / s;
        z = float(a.zero[rowc * ngroups + gi]);
      } else {
        const float Df = f16_to_f32(a.D[rowc * ngroups + gi]);
        const float Dmf = f16_to_f32(a.Dm[rowc * ngroups + gi]);
        const int64_t sb = rowc * (a.cols / 32) + gi * 8 + (sl & 7);
        Sv = Df * float(a.sc[sb]);
        Mv = Dmf * float(a.mc[sb]);
        rSv = Sv > 0.f ? 1.f / Sv : 0.f;
      }
    }

    // next block column at which a group starts (scalar counter, no division)
    int jg = (G - i1 % G) % G;
    // choose the grid of the group starting at block column j (from the
    // current, compensated weights)
    auto choose_grid = [&](int j) {
      const int col = i1 + j;
      const int64_t gi = col / G;
          if (!kQ4K) {
            float mn = INFINITY, mx = -INFINITY;
#pragma unroll
            for (int y = 0; y < kCPL; ++y) {
              const int c = c0 + y;
              if (c < B && c >= j && c < j + G) {
                mn = fminf(mn, w[y]);
                mx = fmaxf(mx, w[y]);
              }
            }
            for (int c = B + sl; c < j + G; c += kLPR) {  // group reaches past the block
              const float v = wrow[c];
              mn = fminf(mn, v);
              mx = fmaxf(mx, v);
            }
            mn = group_min(mn);
            mx = group_max(mx);
            float xmin = fminf(mn, 0.f), xmax = fmaxf(mx, 0.f);
            if (xmin == xmax) {
              xmin = -1.f;
              xmax = 1.f;
            }
            s = (xmax - xmin) / maxq;
            rs = 1.f / s;
            z = fminf(fmaxf(__builtin_rintf(-xmin / s), 0.f), maxq);
            if (a.search) {
              // Importance-weighted choice among the scales (1 - k/32) s,
              // k = 0..15, at the same zero point: codes in float32 as the
              // sweep takes them, errors h (w - w^)^2 summed in float64; the
              // first least error wins.
              const float s0 = s;
              double best = INFINITY;
              for (int k = 0; k < 16; ++k) {
                const float sk = (1.f - float(k) * 0.03125f) * s0;
                const float rsk = 1.f / sk;
                double e = 0.0;
#pragma unroll
                for (int y = 0; y < kCPL; ++y) {
                  const int c = c0 + y;
                  if (c < B && c >= j && c < j + G) {
                    const float qv =
                        __builtin_amdgcn_fmed3f(rint_div(w[y], sk, rsk) + z, 0.f, maxq);
                    const float d = __fsub_rn(w[y], __fmul_rn(sk, qv - z));
                    e = fma(hs[c], double(d) * double(d), e);
                  }
                }
                for (int c = B + sl; c < j + G; c += kLPR) {  // group reaches past the block
                  const float v = wrow[c];
                  const float qv = __builtin_amdgcn_fmed3f(rint_div(v, sk, rsk) + z, 0.f, maxq);
                  const float d = __fsub_rn(v, __fmul_rn(sk, qv - z));
                  e = fma(a.hp[i1 + c], double(d) * double(d), e);
                }
                e = group_sum(e);
                if (e < best) {
                  best = e;
                  s = sk;
                }
              }
              rs = 1.f / s;
            }
            if (sl == 0 && rv) {
              a.scale[row * ngroups + gi] = s;
              a.zero[row * ngroups + gi] = (uint8_t)z;
            }
          } else {
            // super-block of 256 starting here (always a block start): the
            // lane's columns 128t + c0 + y for t = 0, 1; sub-block
            // b = 4t + sl/4 is a group of 4 lanes.
            float sb_s[2], sb_m[2];
            float smax = 0.f, mmax = 0.f;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              float mn = INFINITY, mx = -INFINITY;
#pragma unroll
              for (int y = 0; y < kCPL; ++y) {
                const int p = 128 * t + c0 + y;
                const float v = (p < B) ? w[y] : wrow[p];
                mn = fminf(mn, v);
                mx = fmaxf(mx, v);
              }
              mn = fminf(mn, __shfl_xor(mn, 1));
              mn = fminf(mn, __shfl_xor(mn, 2));
              mx = fmaxf(mx, __shfl_xor(mx, 1));
              mx = fmaxf(mx, __shfl_xor(mx, 2));
              mn = fminf(mn, 0.f);
              mx = fmaxf(mx, 0.f);
              sb_s[t] = (mx - mn) / maxq;
              sb_m[t] = -mn;
              if (a.search) {
                // importance-weighted choice of the sub-block's (scale, min)
                // among (1 - k/32) x the min-max pair, k = 0..15: codes in
                // float32, errors in float64 over the sub-block's 4 lanes
                // (butterfly: the same bits in all of them), first least wins
                const float s0 = sb_s[t], m0 = sb_m[t];
                double best = INFINITY;
                for (int k = 0; k < 16; ++k) {
                  const float f = 1.f - float(k) * 0.03125f;
                  const float sk = f * s0, mk = f * m0;
                  const float rsk = 1.f / sk;
                  double e = 0.0;
#pragma unroll
                  for (int y = 0; y < kCPL; ++y) {
                    const int p = 128 * t + c0 + y;
                    const float v = (p < B) ? w[y] : wrow[p];
                    const double hv = (p < B) ? hs[p] : a.hp[i1 + p];
                    const float qv =
                        sk > 0.f
                            ? __builtin_amdgcn_fmed3f(rint_div(__fadd_rn(v, mk), sk, rsk), 0.f, maxq)
                            : 0.f;
                    const float d = __fsub_rn(v, __fsub_rn(__fmul_rn(sk, qv), mk));
                    e = fma(hv, double(d) * double(d), e);
                  }
                  e += __shfl_xor(e, 1);
                  e += __shfl_xor(e, 2);
                  if (e < best) {
                    best = e;
                    sb_s[t] = sk;
                    sb_m[t] = mk;
                  }
                }
              }
              smax = fmaxf(smax, sb_s[t]);
              mmax = fmaxf(mmax, sb_m[t]);
            }
            smax = group_max(smax);
            mmax = group_max(mmax);
            const uint16_t Dh = f32_to_f16_rne(smax / kmax);
            const uint16_t Dmh = f32_to_f16_rne(mmax / kmax);
            const float Df = f16_to_f32(Dh), Dmf = f16_to_f32(Dmh);
            float Sb[2], Mb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const float scq = (sb_s[t] > 0.f && Df > 0.f)
                                    ? fminf(fmaxf(__builtin_rintf(sb_s[t] / Df), 1.f), kmax)
                                    : 0.f;
              const float mcq =
                  (Dmf > 0.f) ? fminf(fmaxf(__builtin_rintf(sb_m[t] / Dmf), 0.f), kmax) : 0.f;
              Sb[t] = Df * scq;
              Mb[t] = Dmf * mcq;
              if ((sl & 3) == 0 && rv) {
                const int b = 4 * t + (sl >> 2);
                const int64_t o = row * (a.cols / 32) + gi * 8 + b;
                a.sc[o] = (uint8_t)scq;
                a.mc[o] = (uint8_t)mcq;
              }
            }
            if (sl == 0 && rv) {
              a.D[row * ngroups + gi] = Dh;
              a.Dm[row * ngroups + gi] = Dmh;
            }
            // sub-lane b < 8 <- S_b, M_b: b = 4t + g is held by sub-lane 4g of half t
            const int src = gbase + 4 * (sl & 3);
            const float S0 = shfl(Sb[0], src), S1 = shfl(Sb[1], src);
            const float M0 = shfl(Mb[0], src), M1 = shfl(Mb[1], src);
            Sv = (sl & 4) ? S1 : S0;
            Mv = (sl & 4) ? M1 : M0;
            rSv = Sv > 0.f ? 1.f / Sv : 0.f;
          }
    };
    // Q4_K: the grid values of the sub-block holding this lane's 8 columns
    // (a 32-column sub-block spans 4 lanes), refreshed whenever a
    // super-block's grid is chosen or read back.
    float Sl = 0.f, Ml = 0.f, rSl = 0.f;
    auto own_subblock = [&]() {
      if (kQ4K) {
        const int src = gbase + (((i1 & 255) + c0) >> 5);
        Sl = shfl(Sv, src);
        Ml = shfl(Mv, src);
        rSl = shfl(rSv, src);
      }
    };
    own_subblock();

    // Results of the current 8-column step (identical in all lanes of a row
    // group: w^_j, code, e_j); its owner lane stores them after the step.
    float wt[kCPL] = {}, qt[kCPL] = {}, et[kCPL] = {};
    auto store_step = [&](int j8) {
      if (!(rv && sl == (j8 >> 3))) return;
      uint8_t *qrow = a.q + row * ld + i1;
      float *erow = Err + row * a.ldE;
      // Hessian-factor route: the later columns take the error against the
      // uncompensated weight, w^_j - o_j, through R_{<B,B} U_BB
      if (hroute) {
#pragma unroll
        for (int x = 0; x < kCPL; ++x) et[x] = wt[x] - o[x];
      }
      if (full && evec) {
        *reinterpret_cast<f32x4_t *>(wrow + c0) = f32x4_t{wt[0], wt[1], wt[2], wt[3]};
        *reinterpret_cast<f32x4_t *>(wrow + c0 + 4) = f32x4_t{wt[4], wt[5], wt[6], wt[7]};
        *reinterpret_cast<f32x4_t *>(erow + c0) = f32x4_t{et[0], et[1], et[2], et[3]};
        *reinterpret_cast<f32x4_t *>(erow + c0 + 4) = f32x4_t{et[4], et[5], et[6], et[7]};
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          lo |= uint32_t(qt[x]) << (8 * x);
          hi |= uint32_t(qt[4 + x]) << (8 * x);
        }
        *reinterpret_cast<uint32_t *>(qrow + c0) = lo;
        *reinterpret_cast<uint32_t *>(qrow + c0 + 4) = hi;
      } else {
#pragma unroll
        for (int x = 0; x < kCPL; ++x)
          if (c0 + x < B) {
            wrow[c0 + x] = wt[x];
            erow[c0 + x] = et[x];
            qrow[c0 + x] = (uint8_t)qt[x];
          }
      }
    };

    // Column step j (block column) with the exact rounding and a generic
    // broadcast: the path for group sizes that are not a multiple of 8, and
    // the one a step is redone on when its fast pass saw a possible tie.
    auto column_exact = [&](int j8, int x) {
      const int j = j8 + x;
      const int col = i1 + j;
      const f32x4_t u0 = *reinterpret_cast<const f32x4_t *>(Ub + j * kMaxB + c0);
      const f32x4_t u1 = *reinterpret_cast<const f32x4_t *>(Ub + j * kMaxB + c0 + 4);
      const float uinv = Uinv[j];
      if (!kG8 && j == jg && j < B) {
        jg += G;
        choose_grid(j);
        own_subblock();
      }
      float wx = 0.f;  // w[x] without dynamic register indexing
#pragma unroll
      for (int y = 0; y < kCPL; ++y) wx = (y == x) ? w[y] : wx;
      const float wj = group_bcast(wx, j >> 3, grp);
      float qj, wq;
      if (!kQ4K) {
        qj = __builtin_amdgcn_fmed3f(rint_div(wj, s, rs) + z, 0.f, maxq);
        wq = s * (qj - z);
      } else {
        const int bsub = (col & 255) >> 5;
        const float S = group_bcast(Sv, bsub, grp), M = group_bcast(Mv, bsub, grp);
        qj = (S > 0.f) ? __builtin_amdgcn_fmed3f(rint_div(wj + M, S, group_bcast(rSv, bsub, grp)),
                                                 0.f, maxq)
                       : 0.f;
        wq = S * qj - M;
      }
      const float ej = (wj - wq) * uinv;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        w[y] = fmaf(-ej, u0[y], w[y]);
        w[4 + y] = fmaf(-ej, u1[y], w[4 + y]);
      }
#pragma unroll
      for (int y = 0; y < kCPL; ++y) {
        wt[y] = (y == x) ? wq : wt[y];
        qt[y] = (y == x) ? qj : qt[y];
        et[y] = (y == x) ? ej : et[y];
      }
    };

    // U rows j and j+1 of the fast pass (read two columns ahead)
    f32x4_t pa0 = *reinterpret_cast<const f32x4_t *>(Ub + c0);
    f32x4_t pa1 = *reinterpret_cast<const f32x4_t *>(Ub + c0 + 4);
    float pai = Uinv[0];
    f32x4_t pb0 = *reinterpret_cast<const f32x4_t *>(Ub + kMaxB + c0);
    f32x4_t pb1 = *reinterpret_cast<const f32x4_t *>(Ub + kMaxB + c0 + 4);
    float pbi = Uinv[1];
    // Fast pass over one 8-column step whose owner (lane j8/8 of each row)
    // is the immediate kOwner, so that w_j is broadcast with one DPP move.
    // It rounds w_j * (1/s) directly and tracks, for every rounded value,
    // its distance from its integer plus the value-dependent part of
    // tie_window: past 0.5 - 1e-5 the exact quotient could round the other
    // way.
    auto fast_step = [&](auto owner, float *tdist) {
      constexpr int kOwner = decltype(owner)::value;
      constexpr int j8 = kOwner * kCPL;
      float S = 0.f, M = 0.f, rS = 0.f;
      if (kQ4K) {  // the step's 8 columns lie in one sub-block
        S = row_bcast<kOwner>(Sl);
        M = row_bcast<kOwner>(Ml);
        rS = row_bcast<kOwner>(rSl);
      }
      static_for<0, kCPL>([&](auto xs) {
        constexpr int x = decltype(xs)::value;
        constexpr int j = j8 + x;
        const f32x4_t u0 = pa0, u1 = pa1;
        const float uinv = pai;
        pa0 = pb0;
        pa1 = pb1;
        pai = pbi;
        pb0 = *reinterpret_cast<const f32x4_t *>(Ub + (j + 2) * kMaxB + c0);
        pb1 = *reinterpret_cast<const f32x4_t *>(Ub + (j + 2) * kMaxB + c0 + 4);
        pbi = Uinv[j + 2];
        // keep these reads here: sunk next to their use they would stall
        __builtin_amdgcn_sched_barrier(0);
        const float wj = row_bcast<kOwner>(w[x]);
        const float y = kQ4K ? (wj + M) * rS : wj * rs;
        const float r = __builtin_rintf(y);
        *tdist = fmaxf(*tdist, fmaf(fabsf(y), 2.5e-7f, fabsf(y - r)));
        float qj, wq, ej;
        if (!kQ4K) {
          // q - z = clamp(r, -z, maxq - z) (small integers: exact), and the
          // division by U_jj is folded into both terms of w - s (q - z), so
          // that a single fma follows the clamp on the column's dependent
          // chain (one rounding of w / U_jj and of s / U_jj instead of one
          // of w - s (q - z) and one of the quotient)
          const float rq = __builtin_amdgcn_fmed3f(r, -z, maxq - z);
          ej = fmaf(-(s * uinv), rq, wj * uinv);
          qj = rq + z;
          wq = s * rq;
        } else {
          qj = (S > 0.f) ? __builtin_amdgcn_fmed3f(r, 0.f, maxq) : 0.f;
          wq = S * qj - M;
          ej = (wj - wq) * uinv;
        }
        // No masks: U's block row j is zero left of the diagonal (and past
        // B); a lane's finished columns are never read again.
#pragma unroll
        for (int yy = 0; yy < 4; ++yy) {
          w[yy] = fmaf(-ej, u0[yy], w[yy]);
          w[4 + yy] = fmaf(-ej, u1[yy], w[4 + yy]);
        }
        wt[x] = wq;
        qt[x] = qj;
        et[x] = ej;
      });
    };

    for (int j8 = 0; j8 < Bp; j8 += kCPL) {
      if (!kG8) {  // a group may start at any column: exact path throughout
#pragma unroll 1
        for (int x = 0; x < kCPL; ++x) column_exact(j8, x);
        store_step(j8);
        continue;
      }
      if (j8 == jg && j8 < B) {
        jg += G;
        choose_grid(j8);
        own_subblock();
      }
      float w0[kCPL];
#pragma unroll
      for (int yy = 0; yy < kCPL; ++yy) w0[yy] = w[yy];
      float tdist = 0.f;
      switch (j8 >> 3) {
#define GPTQ_SWEEP_STEP(k) \
  case k: fast_step(std::integral_constant<int, k>{}, &tdist); break;
        GPTQ_SWEEP_STEP(0) GPTQ_SWEEP_STEP(1) GPTQ_SWEEP_STEP(2) GPTQ_SWEEP_STEP(3)
        GPTQ_SWEEP_STEP(4) GPTQ_SWEEP_STEP(5) GPTQ_SWEEP_STEP(6) GPTQ_SWEEP_STEP(7)
        GPTQ_SWEEP_STEP(8) GPTQ_SWEEP_STEP(9) GPTQ_SWEEP_STEP(10) GPTQ_SWEEP_STEP(11)
        GPTQ_SWEEP_STEP(12) GPTQ_SWEEP_STEP(13) GPTQ_SWEEP_STEP(14) GPTQ_SWEEP_STEP(15)
#undef GPTQ_SWEEP_STEP
        default: break;
      }
      // a possible tie anywhere in the wave: redo the step from its saved
      // state with the exact quotient (grids only change before a step)
      if (__builtin_expect(__any(tdist > 0.5f - 1e-5f), 0)) {
#pragma unroll
        for (int yy = 0; yy < kCPL; ++yy) w[yy] = w0[yy];
#pragma unroll 1
        for (int x = 0; x < kCPL; ++x) column_exact(j8, x);
      }
      store_step(j8);
    }
    if (r0 + rows_per_pass < a.rows) load_w(r0 + rows_per_pass);
  }
}

// The updates a block receives from the earlier blocks of its super-block
// ("GPTQ", section Komponenty: block updates), applied before its columns
// are next read: W[rows, i1:i1+B] -= Err[rows, k_lo:k_hi] U[s1+k_lo:s1+k_hi,
// i1:i1+B] (k counted from the super-block's first column), for this
// workgroup's 16-row slices of every pass.  The errors are the ones this
// workgroup wrote while sweeping those blocks, so no other workgroup is
// involved.  fp32 MFMA 16x16x4: wave w owns block columns [32 w, 32 w + 32)
// as two 16 x 16 tiles; lane l = 16 g + n feeds A[n][k] = -Err[row n][k]
// and B[k][n] = U[k][col n] with k = k0 + 4 g + e for MFMA e of a 16-k step
// (every MFMA sums four k, one per lane group), and holds D[4 g + i][n].
__device__ __forceinline__ void near_update(const SweepArgs &a, const int i1, const int B,
                                            const int k_lo, const int k_hi) {
  constexpr int kC = 32;            // k per chunk: 2 16-k steps
  constexpr int kQ = kC / 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t ld = a.cols;
  const int64_t rows_per_pass = int64_t(gridDim.x) * (kSweepThreads / 64) * 4;
  const int K = k_hi - k_lo;
  // this wave's two 16-column tiles (none past B)
  const int ntile = min(2, max(0, (B - 32 * wave + 15) / 16));
  if (ntile == 0) return;   // wave-uniform; the barrier that follows is the caller's
  int cc[2];
  bool cok[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int col = 32 * wave + 16 * t + n;
    cok[t] = t < ntile && col < B;
    cc[t] = cok[t] ? col : 0;
  }
  const float *Ublk = a.U + int64_t(a.s1 + k_lo + 4 * g) * ld + i1;
  for (int64_t rb = int64_t(blockIdx.x) * 16; rb < a.rows; rb += rows_per_pass) {
    const int64_t ra = min(rb + n, a.rows - 1);          // this lane's A row
    const float *er = a.Err + ra * a.ldE + k_lo + 4 * g;
    f32x4_t acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = min(rb + 4 * g + i, a.rows - 1);
        acc[t][i] = a.W[r * ld + i1 + cc[t]];
      }
    // a chunk of kC k: Err[ra][k + 4g .. +3] for its 16-k steps q, and
    // U[k + 4g + x][col] for q, x; fetched one chunk ahead of its MFMAs
    f32x4_t e[2][kQ];
    float u[2][2][4 * kQ];
    auto fetch = [&](int buf, int kc) {
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const int k = min(kc + 16 * q, K - 16);   // past K: a valid, unused step
        e[buf][q] = *reinterpret_cast<const f32x4_t *>(er + k);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int x = 0; x < 4; ++x) u[buf][t][4 * q + x] = Ublk[int64_t(k + x) * ld + cc[t]];
      }
    };
    fetch(0, 0);
    for (int kc = 0; kc < K; kc += 2 * kC) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int k0 = kc + half * kC;
        if (k0 >= K) break;
        if (k0 + kC < K) fetch(half ^ 1, k0 + kC);
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          if (k0 + 16 * q >= K) break;
#pragma unroll
          for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int t = 0; t < 2; ++t)
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                  -e[half][q][x], cok[t] ? u[half][t][4 * q + x] : 0.f, acc[t], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = rb + 4 * g + i;
        if (r < a.rows && cok[t]) a.W[r * ld + i1 + cc[t]] = acc[t][i];
      }
  }
}

// A launch sweeps the nblk blocks of one super-block [s1, s1 + nblk B).
// Before a block is swept it takes the updates of the earlier blocks of the
// super-block (near_update).  A group is chosen at its first column from
// all of its columns, so where a group spans gblk > 1 blocks, its later
// blocks are brought up to date at the group's start and take only the
// updates of the group's own earlier blocks at their turn.  A workgroup
// keeps the same rows throughout and reads only the errors it wrote, so
// the blocks need no synchronization beyond the workgroup's own barriers.
template <int kQ4K, bool kG8, bool kH>
__global__ void __launch_bounds__(kSweepThreads) sweep_kernel(SweepArgs a) {
  for (int blk = 0; blk < a.nblk; ++blk) {
    const int i1 = a.s1 + blk * a.B;
    const int B = min(a.B, int(a.cols - i1));
    if (blk > 0) {
      __syncthreads();   // the previous block's LDS reads and its W/Err stores are done
      const int first = blk - blk % a.gblk;   // first block of this block's group
      if (blk == first) {
        for (int b2 = blk; b2 < min(blk + a.gblk, a.nblk); ++b2) {
          const int j1 = a.s1 + b2 * a.B;
          near_update(a, j1, min(a.B, int(a.cols - j1)), 0, blk * a.B);
        }
      } else {
        near_update(a, i1, B, first * a.B, blk * a.B);
      }
      __syncthreads();   // the updated weights are visible to every wave
    }
    sweep_block<kQ4K, kG8, kH>(a, i1, B, a.Err + blk * a.B);
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

// Row-staged forms of the two kernels above: one workgroup per row, the
// source row read contiguously into LDS, permuted there, and the output row
// written contiguously (the plain forms gather or scatter single elements
// straight from and to memory).
__global__ void __launch_bounds__(256)
    gather_cols_lds_kernel(const float *__restrict__ W, int64_t rows, int64_t cols,
                           const int32_t *__restrict__ perm, const uint8_t *__restrict__ dead,
                           float *__restrict__ Wp) {
  extern __shared__ float srow[];
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    __syncthreads();
#pragma unroll 8
    for (int64_t c = threadIdx.x; c < cols; c += 256) srow[c] = dead[c] ? 0.f : W[r * cols + c];
    __syncthreads();
#pragma unroll 8
    for (int64_t p = threadIdx.x; p < cols; p += 256)
      Wp[r * cols + p] = srow[min(max(perm[p], 0), (int32_t)(cols - 1))];
  }
}

__global__ void __launch_bounds__(256)
    scatter_cols_lds_kernel(const float *__restrict__ Wp, const uint8_t *__restrict__ qp,
                            int64_t rows, int64_t cols, const int32_t *__restrict__ perm,
                            float *__restrict__ W, uint8_t *__restrict__ q) {
  extern __shared__ float srow[];
  uint8_t *qrow = reinterpret_cast<uint8_t *>(srow + cols);
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    __syncthreads();
#pragma unroll 8
    for (int64_t p = threadIdx.x; p < cols; p += 256) {
      const int32_t c = min(max(perm[p], 0), (int32_t)(cols - 1));
      srow[c] = Wp[r * cols + p];
      qrow[c] = qp[r * cols + p];
    }
    __syncthreads();
#pragma unroll 8
    for (int64_t c = threadIdx.x; c < cols; c += 256) {
      W[r * cols + c] = srow[c];
      q[r * cols + c] = qrow[c];
    }
  }
}

// Form of the row-staged gather that also stages the column map in LDS,
// once per workgroup, and walks rows grid-stride (about one workgroup per
// CU): the map is read from memory once per workgroup instead of once per
// row.  idx[p] is the source column of output position p, or -1 for a dead
// column.  (The same staging made the scatter slower: with one workgroup
// per CU its scattered LDS writes no longer overlap another row's loads.)
__global__ void __launch_bounds__(256)
    gather_cols_map_kernel(const float *__restrict__ W, int64_t rows, int64_t cols,
                           const int32_t *__restrict__ perm, const uint8_t *__restrict__ dead,
                           float *__restrict__ Wp) {
  extern __shared__ float sm[];
  float *srow = sm;
  int32_t *idx = reinterpret_cast<int32_t *>(sm + cols);
  for (int64_t p = threadIdx.x; p < cols; p += 256) {
    const int32_t c = min(max(perm[p], 0), (int32_t)(cols - 1));
    idx[p] = dead[c] ? -1 : c;
  }
  const bool vec = (cols & 3) == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    __syncthreads();  // the map is staged; the previous row's reads are done
    const float *src = W + r * cols;
    if (vec) {
#pragma unroll 4
      for (int64_t c4 = threadIdx.x; c4 < cols / 4; c4 += 256)
        reinterpret_cast<f32x4_t *>(srow)[c4] = reinterpret_cast<const f32x4_t *>(src)[c4];
    } else {
#pragma unroll 4
      for (int64_t c = threadIdx.x; c < cols; c += 256) srow[c] = src[c];
    }
    __syncthreads();
    float *dst = Wp + r * cols;
#pragma unroll 4
    for (int64_t p = threadIdx.x; p < cols; p += 256) {
      const int32_t c = idx[p];
      dst[p] = c < 0 ? 0.f : srow[c];
    }
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

// Importance of each column in processing order: its activation energy.
__global__ void __launch_bounds__(256)
    importance_kernel(const double *__restrict__ hdiag, const int32_t *__restrict__ perm,
                      int64_t cols, double *__restrict__ hp) {
  const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (j < cols) hp[j] = hdiag[perm[j]];
}

}  // namespace

size_t quantize_ws_bytes(int64_t rows, int64_t cols, const gptq_params &p) {
  size_t n = align256(size_t(rows) * kMaxGroupCols * sizeof(float));  // Err
  if (p.act_order) {
    n += align256(size_t(rows) * size_t(cols) * sizeof(float));  // Wp
    n += align256(size_t(rows) * size_t(cols));                  // qp
  }
  if (p.search) n += align256(size_t(cols) * sizeof(double));    // importances, processing order
  if (p.route == GPTQ_ROUTE_HESSIAN)
    n += align256(size_t(rows) * size_t(cols) * sizeof(float));  // uncompensated weights
  return n;
}

gptq_status quantize_layer_impl(float *W, int64_t rows, int64_t cols, const float *U,
                                const int32_t *perm, const uint8_t *dead, const double *hdiag,
                                const gptq_params &p,
                                uint8_t *q, int32_t *g_idx, float *scale, uint8_t *zero,
                                uint16_t *D, uint16_t *Dm, uint8_t *sc, uint8_t *mc, void *ws,
                                size_t ws_bytes, hipStream_t stream) {
  (void)ws_bytes;
  uint8_t *base = static_cast<uint8_t *>(ws);
  float *Err = reinterpret_cast<float *>(base);
  base += align256(size_t(rows) * kMaxGroupCols * sizeof(float));
  float *Wp = W;
  uint8_t *qp = q;
  const unsigned gx = (unsigned)std::min<int64_t>(cdiv(cols, 256), 64);
  const unsigned gy = (unsigned)std::min<int64_t>(rows, 16384);
  // LDS of the row-staged gather/scatter (a float and a code per column);
  // wider rows take the plain kernels
  const size_t row_lds = size_t(cols) * 5;
  const unsigned growsn = (unsigned)std::min<int64_t>(rows, 65535);
  // the map-staging gather: row and map in LDS (8 bytes per column)
  constexpr size_t kMapLds = 160 * 1024;
  const size_t map_lds = size_t(cols) * 8;
  bool map_ok = false;
  unsigned map_grid = 1;
  if (p.act_order && map_lds <= kMapLds) {
    // without the larger LDS limit the row-staged gather below serves
    map_ok = allow_dynamic_lds((const void *)gather_cols_map_kernel, kMapLds) == GPTQ_OK;
    if (!map_ok) set_error("");
    const int map_cus = device_cu_count();
    map_grid = (unsigned)std::min<int64_t>(rows, std::max(map_cus, 1));
  }
  if (p.act_order) {
    Wp = reinterpret_cast<float *>(base);
    base += align256(size_t(rows) * size_t(cols) * sizeof(float));
    qp = base;
    base += align256(size_t(rows) * size_t(cols));
    if (map_ok)
      GPTQ_TRY(launch("quant_gather", gather_cols_map_kernel, dim3(map_grid), dim3(256), map_lds,
                      stream, (const float *)W, rows, cols, perm, dead, Wp));
    else if (row_lds <= 65536)
      GPTQ_TRY(launch("quant_gather", gather_cols_lds_kernel, dim3(growsn), dim3(256),
                      size_t(cols) * 4, stream, (const float *)W, rows, cols, perm, dead, Wp));
    else
      GPTQ_TRY(launch("quant_gather", gather_cols_kernel, dim3(gx, gy), dim3(256), 0, stream,
                      (const float *)W, rows, cols, perm, dead, Wp));
  } else {
    GPTQ_TRY(launch("quant_zero_dead", zero_dead_kernel, dim3(gx, gy), dim3(256), 0, stream,
                    W, rows, cols, dead));
  }

  // Hessian-factor route: the weights before any compensation, kept beside
  // the working copy (processing order, dead columns zeroed)
  const float *Wo = nullptr;
  if (p.route == GPTQ_ROUTE_HESSIAN) {
    float *o = reinterpret_cast<float *>(base);
    base += align256(size_t(rows) * size_t(cols) * sizeof(float));
    const hipError_t e = hipMemcpyAsync(o, Wp, size_t(rows) * size_t(cols) * sizeof(float),
                                        hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess)
      return fail(GPTQ_ERR_DEVICE, std::string("quantize_layer: ") + hipGetErrorString(e));
    Wo = o;
  }

  const double *hp = nullptr;
  if (p.search) {
    double *h = reinterpret_cast<double *>(base);
    base += align256(size_t(cols) * sizeof(double));
    GPTQ_TRY(launch("quant_importance", importance_kernel, dim3(cdiv(cols, 256)), dim3(256), 0,
                    stream, hdiag, perm, cols, h));
    hp = h;
  }

  const int q4k = p.grid == GPTQ_GRID_Q4K;
  const int B = p.block;
  const size_t Bp = (B + 7) & ~7;
  const size_t lds = ((Bp + 2) * kMaxB + Bp + 2 + 1) * sizeof(float) +
                     (p.search ? size_t(B) * sizeof(double) : 0);
  const int g8 = (q4k ? 256 : p.group) % 8 == 0;
  const int hr = p.route == GPTQ_ROUTE_HESSIAN;   // affine only (checked by the caller)
  const int variant = hr ? 4 + g8 : q4k * 2 + g8;
  // (Q4_K groups are 256 columns, always a multiple of 8: variant 3)
  const void *kfn[6] = {(const void *)sweep_kernel<0, false, false>,
                        (const void *)sweep_kernel<0, true, false>,
                        (const void *)sweep_kernel<1, true, false>,
                        (const void *)sweep_kernel<1, true, false>,
                        (const void *)sweep_kernel<0, false, true>,
                        (const void *)sweep_kernel<0, true, true>};
  // A launch with no more workgroups than compute units gets one per CU (its
  // LDS request is raised past half the CU's LDS), so that each wavefront
  // has a SIMD to itself: the sweep is a chain of dependent steps per row,
  // and a second wavefront on the SIMD would only halve its issue rate.
  constexpr size_t kSoloLds = 96 * 1024;
  const int n_cu = device_cu_count();
  GPTQ_TRY(allow_dynamic_lds(kfn[variant], std::max(lds, kSoloLds)));
  const unsigned nwg = (unsigned)std::min<int64_t>(cdiv(rows, kSweepThreads / 64 * 4), kSweepMaxWG);
  const size_t lds_launch = (n_cu > 0 && nwg <= (unsigned)n_cu) ? std::max(lds, kSoloLds) : lds;

  SweepArgs a{};
  a.W = Wp;
  a.q = qp;
  a.U = U;
  a.Wo = Wo;
  a.rows = rows;
  a.cols = cols;
  a.bits = p.bits;
  a.group = p.group;
  a.sub_bits = p.bits == 2 ? 4 : p.bits == 6 ? 8 : 6;
  a.search = p.search;
  a.hp = hp;
  a.scale = scale;
  a.zero = zero;
  a.D = D;
  a.Dm = Dm;
  a.sc = sc;
  a.mc = mc;
  // Lazy updates on three levels.  Blocks are grouped into super-blocks of
  // m blocks, and super-blocks into far groups of up to kMaxGroupCols
  // columns.  Inside a super-block a block's updates reach the super-block's
  // later blocks (K = B); after a super-block its errors reach the rest of
  // its far group (K = m B); after a far group, its errors reach every later
  // column in one product (K = the group's width), the largest and most
  // efficient GEMM.  The result is that of the unblocked definition ("GPTQ",
  // section Komponenty: block updates) as long as every column a group's
  // grid is chosen from is up to date when it is chosen: the super-block
  // and far-group widths divide the group size or are multiples of it.
  //
  // With B a multiple of 16 a super-block is one launch: each workgroup
  // applies the updates inside the super-block to its own rows itself
  // (near_update, fp32 MFMA), from the errors it wrote, just before a block
  // is swept.  Otherwise every block is a launch of its own, followed by a
  // GEMM that updates the rest of its super-block.
  const int G = q4k ? 256 : p.group;
  auto compatible = [&](int w) { return (G % w) == 0 || (w % G) == 0; };
  int m = 1;
  if ((B & 3) == 0)
    for (int c = kMaxSuper / B; c > 1; --c)
      if (compatible(c * B)) {
        m = c;
        break;
      }
  const int SB = m * B;
  int FG = SB;   // far-group width: a multiple of SB
  for (int c = kMaxGroupCols / SB; c > 1; --c)
    if (compatible(c * SB)) {
      FG = c * SB;
      break;
    }
  const bool fused = m > 1 && (B % 16) == 0;
  a.ldE = FG > SB ? FG : (m == 1 ? kMaxB : SB);
  a.gblk = (fused && G > B && G < SB) ? G / B : 1;
  const char *nm = q4k ? "sweep_q4k" : "sweep_affine";
  const dim3 grid(nwg), blk(kSweepThreads);
  auto sweep_launch = [&]() -> gptq_status {
    switch (variant) {
      case 0: return launch(nm, sweep_kernel<0, false, false>, grid, blk, lds_launch, stream, a);
      case 1: return launch(nm, sweep_kernel<0, true, false>, grid, blk, lds_launch, stream, a);
      case 4: return launch(nm, sweep_kernel<0, false, true>, grid, blk, lds_launch, stream, a);
      case 5: return launch(nm, sweep_kernel<0, true, true>, grid, blk, lds_launch, stream, a);
      default: return launch(nm, sweep_kernel<1, true, false>, grid, blk, lds_launch, stream, a);
    }
  };
  for (int64_t g1 = 0; g1 < cols; g1 += FG) {
    const int64_t g2 = std::min<int64_t>(g1 + FG, cols);
    for (int64_t s1 = g1; s1 < g2; s1 += SB) {
      const int64_t s2 = std::min<int64_t>(s1 + SB, g2);
      float *Es = Err + (s1 - g1);   // this super-block's errors
      if (fused) {
        a.s1 = (int)s1;
        a.B = B;
        a.nblk = (int)cdiv(s2 - s1, B);
        a.Err = Es;
        GPTQ_TRY(sweep_launch());
      } else {
        for (int64_t i1 = s1; i1 < s2; i1 += B) {
          const int Bc = (int)std::min<int64_t>(B, s2 - i1);
          a.s1 = (int)i1;
          a.B = Bc;
          a.nblk = 1;
          a.Err = Es + (i1 - s1);
          GPTQ_TRY(sweep_launch());
          const int64_t i2 = i1 + Bc;
          if (i2 < s2)
            GPTQ_TRY(gemm_f32(Es + (i1 - s1), a.ldE, U + i1 * cols + i2, cols, Wp + i2, cols,
                              (int)rows, (int)(s2 - i2), Bc, -1.f, 1.f, 0, 0, 0, 0, stream,
                              "trailing_near"));
        }
      }
      if (s2 < g2)   // the rest of the far group
        GPTQ_TRY(gemm_f32(Es, a.ldE, U + s1 * cols + s2, cols, Wp + s2, cols, (int)rows,
                          (int)(g2 - s2), (int)(s2 - s1), -1.f, 1.f, 0, 0, 0, 0, stream,
                          "trailing_group"));
    }
    if (g2 < cols)   // every later column
      GPTQ_TRY(gemm_f32(Err, a.ldE, U + g1 * cols + g2, cols, Wp + g2, cols, (int)rows,
                        (int)(cols - g2), (int)(g2 - g1), -1.f, 1.f, 0, 0, 0, 0, stream,
                        "trailing_gemm"));
  }

  if (p.act_order)
  {
    if (row_lds <= 65536)
      GPTQ_TRY(launch("quant_scatter", scatter_cols_lds_kernel, dim3(growsn), dim3(256), row_lds,
                      stream, (const float *)Wp, (const uint8_t *)qp, rows, cols, perm, W, q));
    else
      GPTQ_TRY(launch("quant_scatter", scatter_cols_kernel, dim3(gx, gy), dim3(256), 0, stream,
                      (const float *)Wp, (const uint8_t *)qp, rows, cols, perm, W, q));
  }
  const int gsz = q4k ? 32 : p.group;
  GPTQ_TRY(launch("quant_g_idx", g_idx_kernel, dim3((unsigned)cdiv(cols, 256)), dim3(256), 0, stream,
                  perm, cols, gsz, g_idx));
  return GPTQ_OK;
}

}  // namespace gptq
