// Damping, activation order and the Cholesky factor of the inverse Hessian
// ("GPTQ", sections Komponenty and Hiperparametry).
//
// U (upper, U^T U = Hp^-1) is reached without forming Hp^-1:
//   A  = J Hp J            (J the exchange matrix: reversed processing order)
//   A  = L L^T             (blocked right-looking Cholesky, lower, in place;
//                           128-column diagonal blocks, trailing updates
//                           deferred per 512-column panel)
//   U  = J L^-1 J          (recursive triangular inverse, then a rotation)
// since Hp = (J L J)(J L J)^T with J L J upper, and the upper Cholesky factor
// of Hp^-1 is unique.  This costs d^3/3 + d^3/3 flops instead of the d^3 +
// d^3/3 of an explicit inverse followed by a second factorization.
//
// Workspace layout: A (d x d float) | T (scratch of the inverse products) |
// flag (int) and delta (double) | rank (int32 x d).  The symmetric copy of H
// that the permuting gather reads is staged in the output U.
#include <algorithm>
#include <vector>

#include "common.h"

namespace gptq {
namespace {

constexpr int kNB = 128;          // diagonal block of the factorization
constexpr int64_t kPanel = 1024;  // columns per deferred trailing update
constexpr int64_t kSub = 256;      // columns per sub-panel inside a panel

struct Node {
  int b0, bm, b1, height;
};

int build_tree(int b0, int b1, std::vector<Node> &out) {
  if (b1 - b0 <= 1) return 0;
  const int bm = (b0 + b1) / 2;
  const int h = 1 + std::max(build_tree(b0, bm, out), build_tree(bm, b1, out));
  out.push_back({b0, bm, b1, h});
  return h;
}

int64_t ldT(int64_t m1) { return (m1 + 3) & ~int64_t(3); }

// Largest sum over one tree height of the T = L21 * X11 scratch (floats).
int64_t tree_scratch(int64_t d, std::vector<Node> *nodes_out, int *hmax_out) {
  const int nb = (int)cdiv(d, kNB);
  std::vector<Node> nodes;
  const int hmax = build_tree(0, nb, nodes);
  int64_t best = 0;
  for (int h = 1; h <= hmax; ++h) {
    int64_t s = 0;
    for (const Node &n : nodes)
      if (n.height == h) {
        const int64_t r0 = int64_t(n.b0) * kNB, rm = int64_t(n.bm) * kNB;
        const int64_t r1 = std::min<int64_t>(int64_t(n.b1) * kNB, d);
        s += (r1 - rm) * ldT(rm - r0);
      }
    best = std::max(best, s);
  }
  if (nodes_out) *nodes_out = nodes;
  if (hmax_out) *hmax_out = hmax;
  return best;
}

// ---------------------------------------------------------------- kernels
// dead flags, damping delta = percdamp * mean(diag with dead -> 1), flag := 0,
// rank := 0.
__global__ void __launch_bounds__(1024)
    diag_prep_kernel(const double *__restrict__ hdiag, int64_t d, double percdamp,
                     uint8_t *__restrict__ dead, double *__restrict__ delta, int *__restrict__ flag,
                     int32_t *__restrict__ rank) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += 1024) {
    const double v = hdiag[i];
    const bool z = v == 0.0;
    dead[i] = z ? 1 : 0;
    rank[i] = 0;
    s += z ? 1.0 : v;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *delta = percdamp * (red[0] / (double)d);
    *flag = 0;
  }
}

// Processing position of column i: the number of columns ahead of it by
// decreasing hdiag, ties to the lower index (a stable sort).  The j range is
// split over gridDim.y slices whose counts are added atomically.  NaN keys
// (only from non-finite inputs) are ordered as -inf so that the ranks always
// form a permutation.
constexpr int kRankSplit = 16;
__global__ void __launch_bounds__(256)
    rank_count_kernel(const double *__restrict__ hdiag, int64_t d, int32_t *__restrict__ rank) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per = (d + gridDim.y - 1) / gridDim.y;
  const int64_t j0 = int64_t(blockIdx.y) * per, j1 = min(d, j0 + per);
  __shared__ double keys[256];
  auto key = [](double v) { return v == v ? v : -INFINITY; };
  const double ki = i < d ? key(hdiag[i]) : 0.0;
  int cnt = 0;
  for (int64_t c0 = j0; c0 < j1; c0 += 256) {
    __syncthreads();
    const int64_t j = c0 + threadIdx.x;
    keys[threadIdx.x] = j < j1 ? key(hdiag[j]) : 0.0;
    __syncthreads();
    const int lim = (j1 - c0) < 256 ? (int)(j1 - c0) : 256;
#pragma unroll 8
    for (int t = 0; t < lim; ++t) {
      const double kj = keys[t];
      cnt += (kj > ki) || (kj == ki && c0 + t < i);
    }
  }
  if (i < d && cnt) atomicAdd(rank + i, cnt);
}

// perm[rank[i]] = i (identity without act-order).
__global__ void __launch_bounds__(256)
    rank_scatter_kernel(const int32_t *__restrict__ rank, int64_t d, int act_order,
                        int32_t *__restrict__ perm) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= d) return;
  if (!act_order) {
    perm[i] = (int32_t)i;
    return;
  }
  const int32_t r = rank[i];
  if (r >= 0 && r < d) perm[r] = (int32_t)i;
}

// S = H with its lower triangle filled from the upper one, by 64 x 64 tiles:
// upper tile (ti, tj) is read once and written to (ti, tj) and, transposed,
// to (tj, ti).  Reads and writes are row-contiguous.
__global__ void __launch_bounds__(256)
    symmetrize_kernel(const float *__restrict__ H, int64_t d, float *__restrict__ S) {
  const int ti = blockIdx.y, tj = blockIdx.x;
  if (ti > tj) return;
  __shared__ float t[64][65];
  const int c = threadIdx.x & 63, r0 = threadIdx.x >> 6;
  const int64_t I0 = int64_t(ti) * 64, J0 = int64_t(tj) * 64;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = r0 + 4 * k;
    const int64_t gr = I0 + r, gc = J0 + c;
    t[r][c] = (gr < d && gc < d) ? H[gr * d + gc] : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = r0 + 4 * k;
    const int64_t gr = I0 + r, gc = J0 + c;
    if (gr < d && gc < d) S[gr * d + gc] = (ti == tj && c < r) ? t[c][r] : t[r][c];
  }
  if (ti != tj) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = r0 + 4 * k;
      const int64_t gr = J0 + r, gc = I0 + c;
      if (gr < d && gc < d) S[gr * d + gc] = t[c][r];
    }
  }
}

// The same symmetrization launched over the upper tiles only (tile t of the
// upper triangle, row-major), with float4 reads and writes (d a multiple of
// 4, 16-byte aligned rows); tiles at the matrix edge take per-element masks.
__global__ void __launch_bounds__(256)
    symmetrize_vec_kernel(const float *__restrict__ H, int64_t d, int nt, float *__restrict__ S) {
  // upper tile t -> (ti, tj), ti <= tj: row ti holds nt - ti tiles
  int t = blockIdx.x, ti = 0;
  while (t >= nt - ti) {
    t -= nt - ti;
    ++ti;
  }
  const int tj = ti + t;
  __shared__ float tl[64][65];
  const int64_t I0 = int64_t(ti) * 64, J0 = int64_t(tj) * 64;
  const bool full = I0 + 64 <= d && J0 + 64 <= d;
  const int c4 = (threadIdx.x & 15) * 4, r0 = threadIdx.x >> 4;  // 16 float4 per tile row
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = r0 + 16 * k;
    const int64_t gr = I0 + r, gc = J0 + c4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (full) {
      const float4 x = *reinterpret_cast<const float4 *>(H + gr * d + gc);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (gr < d && gc + e < d) ? H[gr * d + gc + e] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tl[r][c4 + e] = v[e];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = r0 + 16 * k;
    float v[4], w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = c4 + e;
      v[e] = (ti == tj && c < r) ? tl[c][r] : tl[r][c];  // tile (ti, tj)
      w[e] = tl[c][r];                                     // tile (tj, ti), transposed
    }
    const int64_t gr = I0 + r, gc = J0 + c4;
    const int64_t hr = J0 + r, hc = I0 + c4;
    if (full) {
      *reinterpret_cast<float4 *>(S + gr * d + gc) = make_float4(v[0], v[1], v[2], v[3]);
      if (ti != tj) *reinterpret_cast<float4 *>(S + hr * d + hc) = make_float4(w[0], w[1], w[2], w[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (gr < d && gc + e < d) S[gr * d + gc + e] = v[e];
        if (ti != tj && hr < d && hc + e < d) S[hr * d + hc + e] = w[e];
      }
    }
  }
}

// Row a of A, on and below the diagonal: A[a][b] = Hp[d-1-a][d-1-b] with
// Hp[x][y] = S[perm[x]][perm[y]] (S the symmetric H), dead diagonal entries
// taken as 1 and delta added on the diagonal.  One workgroup per row: the
// source row of S is read contiguously (into LDS when kLds), then gathered by
// the permutation; the output row is written contiguously.  A's strict upper
// triangle is not written (nothing reads it).
template <bool kLds>
__global__ void __launch_bounds__(256)
    gather_rows_kernel(const float *__restrict__ S, int64_t d, const int32_t *__restrict__ perm,
                       const uint8_t *__restrict__ dead, const double *__restrict__ delta,
                       float *__restrict__ A) {
  extern __shared__ float srow[];
  const double dl = *delta;
  for (int64_t a = blockIdx.x; a < d; a += gridDim.x) {
    const int64_t x = min(max(perm[d - 1 - a], 0), (int32_t)(d - 1));
    const float *src = S + x * d;
    if (kLds) {
      __syncthreads();
#pragma unroll 8
      for (int64_t c = threadIdx.x; c < d; c += 256) srow[c] = src[c];
      __syncthreads();
    }
#pragma unroll 8
    for (int64_t b = threadIdx.x; b <= a; b += 256) {
      float v;
      if (b == a) {
        v = (float)((dead[x] ? 1.0 : (double)(kLds ? srow[x] : src[x])) + dl);
      } else {
        const int64_t y = min(max(perm[d - 1 - b], 0), (int32_t)(d - 1));
        v = kLds ? srow[y] : src[y];
      }
      A[a * d + b] = v;
    }
  }
}

// ------------------------------------------------------ diagonal block
// Factor the diagonal block A[k0:k0+m, k0:k0+m] = L11 L11^T and invert L11,
// in LDS, with 32 x 32 leaves:
//   for each leaf s (columns o = 32 s .. o + 31):
//     one wavefront factors and inverts the leaf in registers (lanes 0..31
//     hold the factor's rows, lanes 32..63 the inverse's columns; column
//     values of the factor are broadcast with readlane);
//     the panel below the leaf is solved against the leaf inverse and the
//     trailing part of the block is updated, as 32 x 32 fp32-MFMA tiles.
//     The wavefront that factors the next leaf first updates that leaf's own
//     diagonal tile, then factors it while the other wavefronts finish the
//     rest of the trailing update;
//   then L11^-1 is assembled from the leaf inverses: X_ba = -X_bb L_ba X_aa,
//   first for 32-pairs, then for the two 64-halves.
// The block is padded with an identity to 128 when m < 128.  X (lower) and
// zeros (upper) are written back over the block.  A pivot that is not > 0
// and finite sets *flag.
//
// Panel solve in the same launch: workgroups 1.. each take 64 rows of the
// panel below the block (rows k0 + 128 + 64 (b - 1) ..) and overwrite them
// with L21 = A21 L11^-T.  Every workgroup factors and inverts the block
// itself (the same instructions on the same data, so the same bits); only
// workgroup 0 writes the block and the flag.  The rows' loads are issued
// first and wait in registers while the block is factored.
constexpr int kDP = 130;            // LDS pitch (floats): conflict-light MFMA reads
constexpr int kDiagThreads = 256;   // 4 wavefronts
constexpr size_t kDiagLds = size_t(2) * 128 * kDP * sizeof(float);  // dynamic part

__device__ __forceinline__ float rl(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// acc += A(32 x K) * B(K x 32) over k in [k0, k1), A(m,k) = a(m,k), B(k,n) = b(k,n).
template <int k0, int k1, typename FA, typename FB>
__device__ __forceinline__ void mma32(f32x16_t &acc, int lane, FA a, FB b) {
#pragma unroll
  for (int kk = k0; kk < k1; kk += 2) {
    const int k = kk + (lane >> 5);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a(lane & 31, k), b(k, lane & 31), acc, 0, 0, 0);
  }
}

// 32x32 MFMA result layout: element v of lane l is (row, col) =
// (8*(v/4) + 4*(l/32) + v%4, l%32).
template <typename F>
__device__ __forceinline__ void for_acc(const f32x16_t &acc, int lane, F f) {
#pragma unroll
  for (int v = 0; v < 16; ++v) f(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), lane & 31, acc[v]);
}

// One wavefront: factor leaf s of the block in L (lower, in place) and write
// its inverse into X.  Lanes 0..31 hold the rows of the leaf; lanes 32..63
// hold the columns of the identity, which become the columns of L^-1.  Step j
// broadcasts column j of the factor with readlane, and one instruction
// stream serves both halves: r_k -= r_j l_kj is the right-looking factor
// update in the lower half and the right-looking inverse update (forward
// substitution by columns) in the upper half, after r_j *= 1/l_jj.
// Nothing selects on the lane index inside the steps: per-lane masks would
// be hoisted out of the leaf loop by the compiler and spill.
__device__ __forceinline__ void leaf_factor_inverse(float *L, float *X, int o, int lane,
                                                    unsigned &bad) {
  const int i = lane & 31;
  const bool inv_half = lane >= 32;
  const unsigned onehot = 1u << i;
  float r[32];
  // the block's upper part in LDS is zero, so the leaf row loads unmasked
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const float lv = L[(o + i) * kDP + o + k];
    r[k] = inv_half ? (float)((onehot >> k) & 1u) : lv;
  }
  // Entries of the lower half above the diagonal (k > i) take part
  // unmasked: they stay finite and are never read.
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float piv = rl(r[j], j);
    // 0 < piv < inf (NaN fails too), tested on the wave-uniform bit pattern
    // so the test stays in scalar registers
    const bool ok = (__float_as_uint(piv) - 1u) < 0x7f7fffffu;
    bad |= ok ? 0u : 1u;
    // lower half: l_ij (lane j itself gets piv / l_jj = l_jj);
    // upper half: column j of the inverse is final
    r[j] *= __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(ok ? piv : 1.f));
    float lk[32];
#pragma unroll
    for (int k = j + 1; k < 32; ++k) lk[k] = rl(r[j], k);
#pragma unroll
    for (int k = j + 1; k < 32; ++k) r[k] = fmaf(-r[j], lk[k], r[k]);
    // finish step j here: deferring its updates to where each column is
    // next used would keep many broadcast values alive at once in scalar
    // registers, which then spill
#pragma unroll
    for (int k = j + 1; k < 32; ++k) asm volatile("" : "+v"(r[k]));
  }
  if (!inv_half) {
#pragma unroll
    for (int k = 0; k < 32; ++k) L[(o + i) * kDP + o + k] = r[k];
  } else {
#pragma unroll
    for (int k = 0; k < 32; ++k) X[(o + k) * kDP + o + i] = r[k];
  }
}

__global__ void __launch_bounds__(kDiagThreads)
    potrf_inv_block_kernel(float *__restrict__ A, int64_t d, int64_t k0, int m,
                           int *__restrict__ flag) {
  extern __shared__ float sm[];
  float *L = sm;                // 128 x kDP: the block, factored in place (lower)
  float *X = L + 128 * kDP;     // 128 x kDP: the inverse (lower; each part written before read)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *Ab = A + k0 * d + k0;
  // float4 rows when the block is full and rows are 16-byte aligned
  const bool vec = m == 128 && (d & 3) == 0;
  // panel rows of this workgroup (blockIdx.x >= 1 only; the launch
  // guarantees m == 128 and 16-byte aligned rows then): 8 float4 per thread,
  // piece e = tid + 256 t is row e / 32, columns 4 (e % 32) ..; rows past d
  // load row d - 1 and are not stored
  const int64_t pr0 = k0 + 128 + 64 * int64_t(blockIdx.x - 1);
  f32x4_t pv[8];
  if (blockIdx.x > 0) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int e = tid + kDiagThreads * t;
      const int64_t row = min(pr0 + (e >> 5), d - 1);
      pv[t] = *reinterpret_cast<const f32x4_t *>(A + row * d + k0 + (e & 31) * 4);
    }
  }
  if (vec) {
    f32x4_t v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int e = tid + kDiagThreads * t;
      v[t] = *reinterpret_cast<const f32x4_t *>(Ab + (e >> 5) * int(d) + (e & 31) * 4);
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int e = tid + kDiagThreads * t;
      const int i = e >> 5, j = (e & 31) * 4;
      float2 lo, hi;
      lo.x = j <= i ? v[t][0] : 0.f;
      lo.y = j + 1 <= i ? v[t][1] : 0.f;
      hi.x = j + 2 <= i ? v[t][2] : 0.f;
      hi.y = j + 3 <= i ? v[t][3] : 0.f;
      *reinterpret_cast<float2 *>(L + i * kDP + j) = lo;
      *reinterpret_cast<float2 *>(L + i * kDP + j + 2) = hi;
    }
  } else {
    // all 64 elements per thread in flight at once; unconditional loads from
    // clamped (valid) offsets, selected afterwards
    float v[64];
#pragma unroll
    for (int t = 0; t < 64; ++t) {
      const int e = tid + kDiagThreads * t;
      const int i = e >> 7, j = e & 127;
      v[t] = Ab[int(min(i, m - 1)) * int(d) + min(j, m - 1)];
    }
#pragma unroll
    for (int t = 0; t < 64; ++t) {
      const int e = tid + kDiagThreads * t;
      const int i = e >> 7, j = e & 127;
      L[i * kDP + j] = (i < m && j <= i) ? v[t] : (i == j && i >= m ? 1.f : 0.f);
    }
  }
  __syncthreads();

  unsigned bad = 0;
  for (int s = 0; s < 4; ++s) {
    const int o = 32 * s;
    // leaf s (its diagonal tile was finished by wave 0 itself)
    if (wave == 0) leaf_factor_inverse(L, X, o, lane, bad);
    __syncthreads();
    if (s == 3) break;
    const int nb = 3 - s;  // 32-row blocks below the leaf
    // panel: P_b = L[rows of b, leaf cols] * Xleaf^T
    if (wave < nb) {
      const int r0 = o + 32 + 32 * wave;
      f32x16_t acc = {};
      mma32<0, 32>(acc, lane, [&](int mm, int k) { return L[(r0 + mm) * kDP + o + k]; },
            [&](int k, int n) { return X[(o + n) * kDP + o + k]; });
      for_acc(acc, lane, [&](int r, int c, float v) { L[(r0 + r) * kDP + o + c] = v; });
    }
    __syncthreads();
    // trailing part of the block: L[bi][bj] -= P_bi P_bj^T, bj <= bi.  Wave 0
    // takes tile (0,0), the next leaf's diagonal tile, and goes on to factor
    // that leaf; waves 1..3 share the other tiles.  The barrier after the
    // next leaf orders all of them before the next panel solve.
    const int nblk = nb * (nb + 1) / 2;
    for (int t = (wave == 0 ? 0 : wave); t < nblk; t += (wave == 0 ? nblk : 3)) {
      int bi = 0;
      while ((bi + 1) * (bi + 2) / 2 <= t) ++bi;
      const int bj = t - bi * (bi + 1) / 2;
      const int ri = o + 32 + 32 * bi, rj = o + 32 + 32 * bj;
      f32x16_t acc = {};
      mma32<0, 32>(acc, lane, [&](int mm, int k) { return L[(ri + mm) * kDP + o + k]; },
            [&](int k, int n) { return L[(rj + n) * kDP + o + k]; });
      for_acc(acc, lane, [&](int r, int c, float v) {
        if (bi != bj || r >= c) L[(ri + r) * kDP + rj + c] -= v;
      });
    }
  }

  // ---- assemble L^-1 from the leaf inverses; scratch T lives in L's unused
  //      upper triangle.
  // level 1: pairs (0,1) and (2,3): X_ba = -X_bb (L_ba X_aa)
  if (wave < 2) {
    const int a0 = 64 * wave, b0 = a0 + 32;
    float *T = L + a0 * kDP + b0;  // rows a0.., cols b0.. (above the diagonal)
    f32x16_t acc = {};
    mma32<0, 32>(acc, lane, [&](int mm, int k) { return L[(b0 + mm) * kDP + a0 + k]; },
          [&](int k, int n) { return X[(a0 + k) * kDP + a0 + n]; });
    for_acc(acc, lane, [&](int r, int c, float v) { T[r * kDP + c] = v; });
    f32x16_t acc2 = {};
    mma32<0, 32>(acc2, lane, [&](int mm, int k) { return X[(b0 + mm) * kDP + b0 + k]; },
          [&](int k, int n) { return T[k * kDP + n]; });
    for_acc(acc2, lane, [&](int r, int c, float v) { X[(b0 + r) * kDP + a0 + c] = -v; });
  }
  __syncthreads();
  // level 2: halves [0,64) and [64,128): T = L[64:,:64] X[:64,:64]; X[64:,:64] = -X[64:,64:] T
  {
    float *T = L + 0 * kDP + 64;  // rows 0..63, cols 64..127 (above the diagonal)
    const int bi = wave >> 1, bj = wave & 1;
    f32x16_t acc = {};
    // X[:64,:64] is lower in 32-blocks: block (kb, bj) is zero for kb < bj
    auto la = [&](int mm, int k) { return L[(64 + 32 * bi + mm) * kDP + k]; };
    auto xb = [&](int k, int n) { return X[k * kDP + 32 * bj + n]; };
    mma32<32, 64>(acc, lane, la, xb);
    if (bj == 0) mma32<0, 32>(acc, lane, la, xb);
    __syncthreads();
    for_acc(acc, lane, [&](int r, int c, float v) { T[(32 * bi + r) * kDP + 32 * bj + c] = v; });
    __syncthreads();
    f32x16_t acc2 = {};
    // X[64:,64:] is lower in 32-blocks: block (bi, kb) is zero for kb > bi
    auto xa = [&](int mm, int k) { return X[(64 + 32 * bi + mm) * kDP + 64 + k]; };
    auto tb = [&](int k, int n) { return T[k * kDP + 32 * bj + n]; };
    mma32<0, 32>(acc2, lane, xa, tb);
    if (bi == 1) mma32<32, 64>(acc2, lane, xa, tb);
    for_acc(acc2, lane, [&](int r, int c, float v) { X[(64 + 32 * bi + r) * kDP + 32 * bj + c] = -v; });
  }
  __syncthreads();
  if (blockIdx.x > 0) {
    // L21 rows = A21 rows x X^T, with the rows staged in L's place:
    // out[i][j] = sum_k A21[i][k] X[j][k], k <= j (X lower).  Wave w takes
    // row tile w / 2 and column tiles {0, 3} or {1, 2} (five 32-k blocks
    // each).
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int e = tid + kDiagThreads * t;
      float *dst = L + (e >> 5) * kDP + (e & 31) * 4;
      *reinterpret_cast<float2 *>(dst) = float2{pv[t][0], pv[t][1]};
      *reinterpret_cast<float2 *>(dst + 2) = float2{pv[t][2], pv[t][3]};
    }
    __syncthreads();
    const int rt = wave >> 1;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int ct = (wave & 1) ? 1 + c : 3 * c;
      f32x16_t acc = {};
      for (int kb = 0; kb <= ct; ++kb)
        mma32<0, 32>(acc, lane, [&](int mm, int k) { return L[(32 * rt + mm) * kDP + 32 * kb + k]; },
                     [&](int k, int n) { return X[(32 * ct + n) * kDP + 32 * kb + k]; });
      for_acc(acc, lane, [&](int r, int cc, float v) {
        const int64_t row = pr0 + 32 * rt + r;
        if (row < d) A[row * d + k0 + 32 * ct + cc] = v;
      });
    }
    return;
  }
  if (tid == 0 && bad) *flag = 1;
  float *Aw = A + k0 * d + k0;
  if (vec) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int e = tid + kDiagThreads * t;
      const int i = e >> 5, j = (e & 31) * 4;
      const float2 lo = *reinterpret_cast<const float2 *>(X + i * kDP + j);
      const float2 hi = *reinterpret_cast<const float2 *>(X + i * kDP + j + 2);
      f32x4_t w;
      w[0] = j <= i ? lo.x : 0.f;
      w[1] = j + 1 <= i ? lo.y : 0.f;
      w[2] = j + 2 <= i ? hi.x : 0.f;
      w[3] = j + 3 <= i ? hi.y : 0.f;
      *reinterpret_cast<f32x4_t *>(Aw + i * int(d) + j) = w;
    }
  } else {
#pragma unroll 16
    for (int t = 0; t < 64; ++t) {
      const int e = tid + kDiagThreads * t;
      const int i = e >> 7, j = e & 127;
      if (i < m && j < m) Aw[int64_t(i) * d + j] = j <= i ? X[i * kDP + j] : 0.f;
    }
  }
}

// Hessian-factor route, first step.  After the blocked Cholesky A holds L
// below its 128 x 128 diagonal blocks and L_kk^-1 in them.  With R = J L J
// (Hp = R R^T) and U = R^-1, processing order, a = d-1-i, b = d-1-j, j >= i:
//   F[i][j] = U_ij = Linv[a][b]   a, b in one diagonal block,
//   F[i][j] = R_ij = L[a][b]      otherwise;
// 0 below the diagonal.  (The second step multiplies each block column of R
// above the diagonal block by that block, U_BB.)  Thread t owns the four
// columns 4t .. 4t+3, one reversed 16-byte segment of a row of A; d % 4 == 0
// and 16-byte aligned A and F.
__global__ void __launch_bounds__(256)
    rotate_factor_kernel(const float *__restrict__ A, int64_t d, float *__restrict__ F) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= d / 4) return;
  const int64_t j = 4 * t;
  for (int64_t i = blockIdx.y; i < d; i += gridDim.y) {
    f32x4_t out = {0.f, 0.f, 0.f, 0.f};
    if (j + 3 >= i) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t *>(A + (d - 1 - i) * d + (d - 4 - j));
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = j + e >= i ? v[3 - e] : 0.f;
    }
    *reinterpret_cast<f32x4_t *>(F + i * d + j) = out;
  }
}

// U[i][j] = Linv[d-1-i][d-1-j] for j >= i, 0 below the diagonal.
__global__ void __launch_bounds__(256)
    rotate_upper_kernel(const float *__restrict__ Linv, int64_t d, float *__restrict__ U) {
  for (int64_t i = blockIdx.y; i < d; i += gridDim.y)
    for (int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x; j < d; j += int64_t(gridDim.x) * 256)
      U[i * d + j] = j >= i ? Linv[(d - 1 - i) * d + (d - 1 - j)] : 0.f;
}

constexpr size_t kMaxRowLds = 160 * 1024;

// The same rotation four columns at a time (d a multiple of 4, 16-byte
// aligned rows): the source of U[i][j..j+3] is the float4 of row d-1-i at
// column d-4-j, reversed.  Chunks wholly below the diagonal are not read.
__global__ void __launch_bounds__(256)
    rotate_upper_vec_kernel(const float *__restrict__ Linv, int64_t d, float *__restrict__ U) {
  const int64_t d4 = d / 4;
  for (int64_t i = blockIdx.y; i < d; i += gridDim.y)
    for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < d4; t += int64_t(gridDim.x) * 256) {
      const int64_t j = 4 * t;
      f32x4_t out = {0.f, 0.f, 0.f, 0.f};
      if (j + 3 >= i) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t *>(Linv + (d - 1 - i) * d + (d - 4 - j));
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = j + e >= i ? v[3 - e] : 0.f;
      }
      *reinterpret_cast<f32x4_t *>(U + i * d + j) = out;
    }
}

}  // namespace

size_t prepare_ws_bytes(int64_t d) {
  const size_t a = align256(size_t(d) * size_t(d) * sizeof(float));
  const size_t t = align256(size_t(tree_scratch(d, nullptr, nullptr)) * sizeof(float));
  return a + t + 256 + align256(size_t(d) * sizeof(int32_t));
}

gptq_status prepare_hinv_impl(const float *H, const double *hdiag, int64_t d,
                              const gptq_params &p, float *U, int32_t *perm, uint8_t *dead,
                              void *ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws_bytes;
  std::vector<Node> nodes;
  int hmax = 0;
  const int64_t tsz = tree_scratch(d, &nodes, &hmax);
  uint8_t *base = static_cast<uint8_t *>(ws);
  float *A = reinterpret_cast<float *>(base);
  float *T = reinterpret_cast<float *>(base + align256(size_t(d) * size_t(d) * 4));
  uint8_t *tail = base + align256(size_t(d) * size_t(d) * 4) + align256(size_t(tsz) * 4);
  int *flag = reinterpret_cast<int *>(tail);
  double *delta = reinterpret_cast<double *>(tail + 8);
  int32_t *rank = reinterpret_cast<int32_t *>(tail + 256);

  GPTQ_TRY(launch("prep_diag", diag_prep_kernel, dim3(1), dim3(1024), 0, stream, hdiag, d,
                  (double)p.percdamp, dead, delta, flag, rank));
  if (p.act_order)
    GPTQ_TRY(launch("prep_rank_perm", rank_count_kernel,
                    dim3((unsigned)cdiv(d, 256), (unsigned)std::min<int64_t>(kRankSplit, d)),
                    dim3(256), 0, stream, hdiag, d, rank));
  GPTQ_TRY(launch("prep_rank_perm", rank_scatter_kernel, dim3((unsigned)cdiv(d, 256)), dim3(256), 0,
                  stream, (const int32_t *)rank, d, (int)p.act_order, perm));
  // the symmetric H is staged in U's memory (U is written last)
  const unsigned g64 = (unsigned)cdiv(d, 64);
  if ((d & 3) == 0 && (reinterpret_cast<uintptr_t>(H) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(U) & 15) == 0)
    GPTQ_TRY(launch("prep_symmetrize", symmetrize_vec_kernel, dim3(g64 * (g64 + 1) / 2), dim3(256),
                    0, stream, H, d, (int)g64, U));
  else
    GPTQ_TRY(launch("prep_symmetrize", symmetrize_kernel, dim3(g64, g64), dim3(256), 0, stream, H,
                    d, U));
  const unsigned growsn = (unsigned)std::min<int64_t>(d, 65535);
  const size_t srow_bytes = size_t(d) * sizeof(float);
  if (srow_bytes <= kMaxRowLds) {
    if (srow_bytes > 65536)
      GPTQ_TRY(allow_dynamic_lds((const void *)gather_rows_kernel<true>, kMaxRowLds));
    GPTQ_TRY(launch("prep_gather", gather_rows_kernel<true>, dim3(growsn), dim3(256), srow_bytes,
                    stream, (const float *)U, d, (const int32_t *)perm, (const uint8_t *)dead,
                    (const double *)delta, A));
  } else {
    GPTQ_TRY(launch("prep_gather", gather_rows_kernel<false>, dim3(growsn), dim3(256), 0, stream,
                    (const float *)U, d, (const int32_t *)perm, (const uint8_t *)dead,
                    (const double *)delta, A));
  }

  // ---- blocked Cholesky A = L L^T; diagonal blocks end up holding L_ii^-1
  const size_t lds = kDiagLds;
  GPTQ_TRY(allow_dynamic_lds((const void *)potrf_inv_block_kernel, lds));
  const int cus = device_cu_count();
  // Three levels: inside a sub-panel of kSub columns the trailing update
  // follows each diagonal block (K = 128); past a sub-panel, the rest of its
  // panel is updated once (K = kSub); past a panel of kPanel columns, the
  // rest of the matrix once (K = kPanel).
  for (int64_t c0 = 0; c0 < d; c0 += kPanel) {
    const int64_t c1 = std::min<int64_t>(c0 + kPanel, d);
    for (int64_t s0 = c0; s0 < c1; s0 += kSub) {
      const int64_t s1 = std::min<int64_t>(s0 + kSub, c1);
      bool last = false;
      for (int64_t k0 = s0; k0 < s1; k0 += kNB) {
        const int m = (int)std::min<int64_t>(kNB, d - k0);
        const int64_t r = d - k0 - m;
        // The panel below the block is solved in the same launch when its
        // 64-row slices, plus the block's own workgroup, fit in one round of
        // the chip (every workgroup factors the block; a second round would
        // repeat that on the critical path).
        const int64_t slices = r > 0 ? cdiv(r, 64) : 0;
        const bool fused = slices > 0 && (d & 3) == 0 && 1 + slices <= cus;
        GPTQ_TRY(launch("chol_diag_block", potrf_inv_block_kernel,
                        dim3(unsigned(fused ? 1 + slices : 1)), dim3(kDiagThreads), lds, stream, A,
                        d, k0, m, flag));
        if (r <= 0) {
          last = true;
          break;
        }
        float *A21 = A + (k0 + m) * d + k0;
        // L21 = A21 * L11^-T   (in place: each workgroup owns whole rows)
        if (!fused)
          GPTQ_TRY(gemm_f32(A21, d, A + k0 * d + k0, d, A21, d, (int)r, m, m, 1.f, 0.f, 1, 0, 0, 0,
                            stream, "chol_trsm"));
        // the rest of the sub-panel: A[k0+m:, k0+m:s1] -= L21 L21[0:s1-k0-m]^T
        // (the part of it above the diagonal is written too, and never read)
        const int64_t nn = s1 - (k0 + m);
        if (nn > 0)
          GPTQ_TRY(gemm_f32(A21, d, A21, d, A + (k0 + m) * d + (k0 + m), d, (int)r, (int)nn, m,
                            -1.f, 1.f, 1, 0, 0, 0, stream, "chol_near"));
      }
      if (last) break;
      // the rest of the panel past the sub-panel: A[s1:, s1:c1] -= Ls Ls[0:c1-s1]^T
      const int64_t nm = c1 - s1, rm = d - s1;
      if (nm > 0 && rm > 0) {
        const float *Ls = A + s1 * d + s0;
        GPTQ_TRY(gemm_f32(Ls, d, Ls, d, A + s1 * d + s1, d, (int)rm, (int)nm, (int)(s1 - s0),
                          -1.f, 1.f, 1, 0, 0, 0, stream, "chol_mid"));
      }
    }
    // the columns past the panel: A22 -= Lp Lp^T (lower triangle), K = c1 - c0
    const int64_t r2 = d - c1;
    if (r2 > 0) {
      const float *Lp = A + c1 * d + c0;
      GPTQ_TRY(gemm_f32(Lp, d, Lp, d, A + c1 * d + c1, d, (int)r2, (int)r2, (int)(c1 - c0), -1.f,
                        1.f, 1, 1, 0, 0, stream, "chol_syrk"));
    }
  }

  if (p.route == GPTQ_ROUTE_HESSIAN) {
    // no inverse past the diagonal blocks: U's blocks there, R above them,
    // then each block column of R times its diagonal block (in place; the
    // problems touch disjoint columns): F[0:b0, B] = R[0:b0, B] U_BB
    GPTQ_TRY(launch("prep_rotate", rotate_factor_kernel,
                    dim3((unsigned)(d / 4 + 255) / 256, (unsigned)std::min<int64_t>(d, 1024)),
                    dim3(256), 0, stream, (const float *)A, d, U));
    GemmGroup g{};
    g.transB = 0;
    for (int64_t b0 = kNB; b0 < d; b0 += kNB) {
      GemmProblem &q = g.p[g.count++];
      q.A = U + b0;                  // R[0:b0, B]
      q.lda = d;
      q.B = U + b0 * d + b0;         // U_BB
      q.ldb = d;
      q.C = U + b0;                  // over R
      q.ldc = d;
      q.M = (int)b0;
      q.N = kNB;
      q.K = kNB;
      q.alpha = 1.f;
      q.beta = 0.f;
      if (g.count == kMaxGemmGroup || b0 + kNB >= d) {
        GPTQ_TRY(gemm_f32_grouped(g, stream, "prep_factor_blocks"));
        g = GemmGroup{};
        g.transB = 0;
      }
    }
    hmax = 0;
  }

  // ---- recursive triangular inverse, bottom-up by tree height:
  //   T = L21 X11 ; X21 = -X22 T   (X11, X22 already inverted)
  for (int h = 1; h <= hmax; ++h) {
    std::vector<Node> lv;
    for (const Node &n : nodes)
      if (n.height == h) lv.push_back(n);
    for (size_t s = 0; s < lv.size(); s += kMaxGemmGroup) {
      const size_t e = std::min(lv.size(), s + kMaxGemmGroup);
      GemmGroup g1{}, g2{};
      g1.transB = 0;
      g1.b_lower = 1;
      g2.transB = 0;
      g2.a_lower = 1;
      int64_t off = 0;
      for (size_t k = s; k < e; ++k) {
        const Node &n = lv[k];
        const int64_t r0 = int64_t(n.b0) * kNB, rm = int64_t(n.bm) * kNB;
        const int64_t r1 = std::min<int64_t>(int64_t(n.b1) * kNB, d);
        const int m1 = (int)(rm - r0), m2 = (int)(r1 - rm);
        float *Tn = T + off;
        off += int64_t(m2) * ldT(m1);
        GemmProblem &a = g1.p[g1.count++];
        a.A = A + rm * d + r0;  // L21
        a.lda = d;
        a.B = A + r0 * d + r0;  // X11
        a.ldb = d;
        a.C = Tn;
        a.ldc = ldT(m1);
        a.M = m2;
        a.N = m1;
        a.K = m1;
        a.alpha = 1.f;
        a.beta = 0.f;
        GemmProblem &b = g2.p[g2.count++];
        b.A = A + rm * d + rm;  // X22
        b.lda = d;
        b.B = Tn;
        b.ldb = ldT(m1);
        b.C = A + rm * d + r0;  // X21 over L21
        b.ldc = d;
        b.M = m2;
        b.N = m1;
        b.K = m2;
        b.alpha = -1.f;
        b.beta = 0.f;
      }
      GPTQ_TRY(gemm_f32_grouped(g1, stream, "trtri_gemm"));
      GPTQ_TRY(gemm_f32_grouped(g2, stream, "trtri_gemm"));
    }
  }

  if (p.route == GPTQ_ROUTE_HESSIAN) {
    // written above
  } else if ((d & 3) == 0 && (reinterpret_cast<uintptr_t>(U) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(A) & 15) == 0)
    GPTQ_TRY(launch("prep_rotate", rotate_upper_vec_kernel,
                    dim3((unsigned)std::min<int64_t>(cdiv(d / 4, 256), 64),
                         (unsigned)std::min<int64_t>(d, 16384)),
                    dim3(256), 0, stream, (const float *)A, d, U));
  else
    GPTQ_TRY(launch("prep_rotate", rotate_upper_kernel,
                    dim3((unsigned)std::min<int64_t>(cdiv(d, 256), 64), (unsigned)std::min<int64_t>(d, 16384)),
                    dim3(256), 0,
                    stream, (const float *)A, d, U));

  int host_flag = 0;
  hipError_t e = hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess)
    return fail(GPTQ_ERR_DEVICE, std::string("prepare_hinv: ") + hipGetErrorString(e));
  if (host_flag) return fail(GPTQ_ERR_NOT_SPD, "damped Hessian is not positive definite");
  return GPTQ_OK;
}

}  // namespace gptq
