// fp32 GEMM engine on fp32 MFMA (v_mfma_f32_32x32x2f32).
//
//   C = alpha * A * op(B) + beta * C,  A row-major M x K,
//   op(B) = B (row-major K x N) or B^T (B row-major N x K).
//
// Used for the dense parts of the inverse-Hessian factorization (triangular
// solve against the diagonal block, trailing symmetric update, the products
// of the recursive triangular inverse) and for the lazy trailing update of
// the column sweep ("GPTQ", section Komponenty: block updates).
//
// Tiles are 128 x 128 with four 64 x 64 wave tiles, or 64 x 64 with four
// 32 x 32 wave tiles for launches too small to fill the chip with the large
// tile.  Operands are staged in LDS k-major ([k][m]) so that an MFMA operand
// read is 32 consecutive floats.  A grouped launch runs up to kMaxGemmGroup
// independent problems of one shape class, each workgroup finding its
// problem by tile index.
#include "common.h"

namespace gptq {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBK = 32;         // k per stage
constexpr int kThreads = 256;

// Staging geometry of one operand tile with kE rows (M or N edge).
template <int kE>
struct Edge {
  static constexpr int kPitch = kE + 4;                   // LDS row pitch of a k-major stage
  static constexpr int kChunks = kE * kBK / 4 / kThreads;  // float4 chunks per thread
  static constexpr int kW = kE / 2;                        // wave tile edge (2 x 2 waves)
  static constexpr int kF = kW / 32;                       // 32 x 32 MFMA tiles per wave edge
};

// Stage one operand tile (kT rows x kBK k, row-major in memory with leading
// dimension ld) into registers, kChunks float4 per thread.  Elements outside
// [0, rows) x [k0, kend) are zero.
template <int kT, bool kVec>
__device__ __forceinline__ void load_rows(const float *__restrict__ P, int64_t ld, int rows,
                                          int r0, int k0, int kend, int tid,
                                          f32x4_t (&v)[Edge<kT>::kChunks]) {
#pragma unroll
  for (int i = 0; i < Edge<kT>::kChunks; ++i) {
    const int c = tid + kThreads * i;
    const int r = c / (kBK / 4), kc = (c % (kBK / 4)) * 4;
    const int gr = r0 + r, gk = k0 + kc;
    f32x4_t x = {0.f, 0.f, 0.f, 0.f};
    if (gr < rows) {
      const float *p = P + int64_t(gr) * ld + gk;
      if (kVec && gk + 4 <= kend) {
        x = *reinterpret_cast<const f32x4_t *>(p);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (gk + e < kend) ? p[e] : 0.f;
      }
    }
    v[i] = x;
  }
}

// Interior form of load_rows: every row and k is in range, 16-byte aligned.
template <int kT>
__device__ __forceinline__ void load_rows_fast(const float *__restrict__ P, int64_t ld, int r0,
                                               int k0, int tid, f32x4_t (&v)[Edge<kT>::kChunks]) {
#pragma unroll
  for (int i = 0; i < Edge<kT>::kChunks; ++i) {
    const int c = tid + kThreads * i;
    const int r = c / (kBK / 4), kc = (c % (kBK / 4)) * 4;
    v[i] = *reinterpret_cast<const f32x4_t *>(P + int64_t(r0 + r) * ld + k0 + kc);
  }
}

// Transposing store of a row-major staged tile into k-major LDS.
template <int kT>
__device__ __forceinline__ void store_rows_kmajor(float *lds, int tid,
                                                  const f32x4_t (&v)[Edge<kT>::kChunks]) {
#pragma unroll
  for (int i = 0; i < Edge<kT>::kChunks; ++i) {
    const int c = tid + kThreads * i;
    const int r = c / (kBK / 4), kc = (c % (kBK / 4)) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) lds[(kc + e) * Edge<kT>::kPitch + r] = v[i][e];
  }
}

// B in row-major K x N: a tile (kBK k-rows x kT cols) is already k-major.
template <int kT, bool kVec>
__device__ __forceinline__ void load_kmajor(const float *__restrict__ P, int64_t ld, int cols,
                                            int c0, int k0, int kend, int tid,
                                            f32x4_t (&v)[Edge<kT>::kChunks]) {
  constexpr int kPerRow = kT / 4;  // float4 chunks per k-row
#pragma unroll
  for (int i = 0; i < Edge<kT>::kChunks; ++i) {
    const int c = tid + kThreads * i;
    const int k = c / kPerRow, nc = (c % kPerRow) * 4;
    const int gk = k0 + k, gc = c0 + nc;
    f32x4_t x = {0.f, 0.f, 0.f, 0.f};
    if (gk < kend) {
      const float *p = P + int64_t(gk) * ld + gc;
      if (kVec && gc + 4 <= cols) {
        x = *reinterpret_cast<const f32x4_t *>(p);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (gc + e < cols) ? p[e] : 0.f;
      }
    }
    v[i] = x;
  }
}

// Interior form of load_kmajor.
template <int kT>
__device__ __forceinline__ void load_kmajor_fast(const float *__restrict__ P, int64_t ld, int c0,
                                                 int k0, int tid, f32x4_t (&v)[Edge<kT>::kChunks]) {
  constexpr int kPerRow = kT / 4;
#pragma unroll
  for (int i = 0; i < Edge<kT>::kChunks; ++i) {
    const int c = tid + kThreads * i;
    const int k = c / kPerRow, nc = (c % kPerRow) * 4;
    v[i] = *reinterpret_cast<const f32x4_t *>(P + int64_t(k0 + k) * ld + c0 + nc);
  }
}

template <int kT>
__device__ __forceinline__ void store_kmajor(float *lds, int tid,
                                             const f32x4_t (&v)[Edge<kT>::kChunks]) {
  constexpr int kPerRow = kT / 4;
#pragma unroll
  for (int i = 0; i < Edge<kT>::kChunks; ++i) {
    const int c = tid + kThreads * i;
    const int k = c / kPerRow, nc = (c % kPerRow) * 4;
    *reinterpret_cast<f32x4_t *>(lds + k * Edge<kT>::kPitch + nc) = v[i];
  }
}

template <int kTM, int kTN, int kTransB, bool kVec>
__global__ void __launch_bounds__(kThreads) gemm_f32_kernel(GemmGroup g) {
  constexpr int kPA = Edge<kTM>::kPitch, kPB = Edge<kTN>::kPitch;
  constexpr int kWM = Edge<kTM>::kW, kFM = Edge<kTM>::kF;
  constexpr int kWN = Edge<kTN>::kW, kFN = Edge<kTN>::kF;
  // ---- find problem and tile
  int tile = blockIdx.x;
  int pi = 0;
  while (pi + 1 < g.count && tile >= g.p[pi + 1].tile_begin) ++pi;
  const GemmProblem &P = g.p[pi];
  tile -= P.tile_begin;
  int tm, tn;
  if (g.lower_out) {
    // lower tiles only (tn <= tm), row-major over the triangle
    tm = int((sqrtf(8.f * tile + 1.f) - 1.f) * 0.5f);
    while ((tm + 1) * (tm + 2) / 2 <= tile) ++tm;
    while (tm * (tm + 1) / 2 > tile) --tm;
    tn = tile - tm * (tm + 1) / 2;
  } else if (g.b_lower) {
    // the K range shrinks as tn grows: columns left to right, heavy tiles first
    const int tiles_m = (P.M + kTM - 1) / kTM;
    tn = tile / tiles_m;
    tm = tile % tiles_m;
  } else if (g.a_lower) {
    // the K range grows with tm: bottom row of tiles first
    const int tiles_m = (P.M + kTM - 1) / kTM;
    tm = tiles_m - 1 - tile / P.tiles_n;
    tn = tile % P.tiles_n;
  } else {
    tm = tile / P.tiles_n;
    tn = tile % P.tiles_n;
  }
  const int m0 = tm * kTM, n0 = tn * kTN;

  int kbeg = 0, kend = P.K;
  if (g.b_lower) kbeg = min(n0, P.K) & ~(kBK - 1);
  if (g.a_lower) kend = min(P.K, m0 + kTM);

  __shared__ __align__(16) float As[2][kBK * kPA];
  __shared__ __align__(16) float Bs[2][kBK * kPB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16_t acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // C tile prefetch (beta != 0): unconditional loads from clamped, valid
  // addresses, issued before the K loop so their latency overlaps it.
  const float alpha = P.alpha, beta = P.beta;
  float cv[kFM][kFN][16];
  if (beta != 0.f) {
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) {
        const int gc = min(n0 + wn * kWN + j * 32 + (lane & 31), P.N - 1);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int gr = min(m0 + wm * kWM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), P.M - 1);
          cv[i][j][v] = P.C[int64_t(gr) * P.ldc + gc];
        }
      }
  }

  const int nsteps = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;
  f32x4_t ra[Edge<kTM>::kChunks], rb[Edge<kTN>::kChunks];
  // Interior tiles (the common case) take unconditional float4 loads; edge
  // tiles and ragged k ranges take the masked loads.
  const bool rows_in = m0 + kTM <= P.M && n0 + kTN <= P.N;
  auto load = [&](int s) {
    const int k0 = kbeg + s * kBK;
    if (kVec && rows_in && k0 + kBK <= kend) {
      load_rows_fast<kTM>(P.A, P.lda, m0, k0, tid, ra);
      if (kTransB)
        load_rows_fast<kTN>(P.B, P.ldb, n0, k0, tid, rb);
      else
        load_kmajor_fast<kTN>(P.B, P.ldb, n0, k0, tid, rb);
      return;
    }
    load_rows<kTM, kVec>(P.A, P.lda, P.M, m0, k0, kend, tid, ra);
    if (kTransB)
      load_rows<kTN, kVec>(P.B, P.ldb, P.N, n0, k0, kend, tid, rb);
    else
      load_kmajor<kTN, kVec>(P.B, P.ldb, P.N, n0, k0, kend, tid, rb);
  };
  auto store = [&](int buf) {
    store_rows_kmajor<kTM>(As[buf], tid, ra);
    if (kTransB)
      store_rows_kmajor<kTN>(Bs[buf], tid, rb);
    else
      store_kmajor<kTN>(Bs[buf], tid, rb);
  };

  if (nsteps > 0) {
    load(0);
    store(0);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
      const int buf = s & 1;
      if (s + 1 < nsteps) load(s + 1);
      const float *A = As[buf];
      const float *B = Bs[buf];
      // operands of step kk+1 are read while step kk's MFMAs run
      float a[2][kFM], b[2][kFN];
      auto rd = [&](int slot, int kk) {
        const int k = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < kFM; ++i) a[slot][i] = A[k * kPA + wm * kWM + i * 32 + (lane & 31)];
#pragma unroll
        for (int j = 0; j < kFN; ++j) b[slot][j] = B[k * kPB + wn * kWN + j * 32 + (lane & 31)];
      };
      rd(0, 0);
#pragma unroll
      for (int kk = 0; kk < kBK / 2; ++kk) {
        if (kk + 1 < kBK / 2) rd((kk + 1) & 1, kk + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kFM; ++i)
#pragma unroll
          for (int j = 0; j < kFN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[kk & 1][i], b[kk & 1][j], acc[i][j],
                                                            0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (s + 1 < nsteps) store(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue (stores only).  32x32 result layout: lane l, element v ->
  //      row 8*(v/4) + 4*(l/32) + v%4, col l%32.
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int gc = n0 + wn * kWN + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int gr = m0 + wm * kWM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const float r = alpha * acc[i][j][v];
        const float out = (beta == 0.f) ? r : fmaf(beta, cv[i][j][v], r);
        if (gr < P.M && gc < P.N && (!g.lower_out || gr >= gc))
          P.C[int64_t(gr) * P.ldc + gc] = out;
      }
    }
}

bool vec_ok(const void *p, int64_t ld) {
  return (reinterpret_cast<uintptr_t>(p) % 16) == 0 && (ld % 4) == 0;
}

template <int kTM, int kTN>
gptq_status launch_grouped(const GemmGroup &g0, hipStream_t stream, const char *name) {
  GemmGroup g = g0;
  int total = 0;
  bool vec = true;
  int n = 0;
  for (int i = 0; i < g0.count; ++i) {
    const GemmProblem &p = g0.p[i];
    if (p.M <= 0 || p.N <= 0) continue;  // empty problem: nothing to write
    GemmProblem q = p;
    const int tm = (int)cdiv(p.M, kTM), tn = (int)cdiv(p.N, kTN);
    q.tiles_n = tn;
    q.tile_begin = total;
    total += g.lower_out ? tm * (tm + 1) / 2 : tm * tn;
    vec = vec && vec_ok(p.A, p.lda) && vec_ok(p.B, p.ldb);
    g.p[n++] = q;
  }
  g.count = n;
  g.total_tiles = total;
  if (n == 0) return GPTQ_OK;
  dim3 grid(total), block(kThreads);
  if (g.transB) {
    if (vec) return launch(name, gemm_f32_kernel<kTM, kTN, 1, true>, grid, block, 0, stream, g);
    return launch(name, gemm_f32_kernel<kTM, kTN, 1, false>, grid, block, 0, stream, g);
  }
  if (vec) return launch(name, gemm_f32_kernel<kTM, kTN, 0, true>, grid, block, 0, stream, g);
  return launch(name, gemm_f32_kernel<kTM, kTN, 0, false>, grid, block, 0, stream, g);
}

}  // namespace

// Large tiles unless they would leave most of the chip idle: with fewer
// than kSmallLaunch 128 x 128 tiles, 64-row tiles give more workgroups.
// A product written in place over its A operand (C == A, one column tile
// of N <= 128) keeps whole 128-column rows per workgroup: 64 x 128 tiles.
constexpr int kSmallLaunch = 256;

gptq_status gemm_f32_grouped(const GemmGroup &g0, hipStream_t stream, const char *name) {
  int64_t tiles128 = 0;
  bool inplace = false;
  for (int i = 0; i < g0.count; ++i) {
    const GemmProblem &p = g0.p[i];
    if (p.M <= 0 || p.N <= 0) continue;
    const int64_t tm = cdiv(p.M, 128), tn = cdiv(p.N, 128);
    tiles128 += g0.lower_out ? tm * (tm + 1) / 2 : tm * tn;
    inplace = inplace || p.C == p.A;
  }
  if (inplace) {
    for (int i = 0; i < g0.count; ++i)
      if (g0.p[i].N > 128 || g0.lower_out)
        return fail(GPTQ_ERR_INVALID_ARG, std::string(name) + ": in-place product wider than 128");
    return tiles128 < kSmallLaunch ? launch_grouped<64, 128>(g0, stream, name)
                                   : launch_grouped<128, 128>(g0, stream, name);
  }
  if (tiles128 < kSmallLaunch) return launch_grouped<64, 64>(g0, stream, name);
  return launch_grouped<128, 128>(g0, stream, name);
}

gptq_status gemm_f32(const float *A, int64_t lda, const float *B, int64_t ldb, float *C,
                     int64_t ldc, int M, int N, int K, float alpha, float beta, int transB,
                     int lower_out, int a_lower, int b_lower, hipStream_t stream,
                     const char *name) {
  GemmGroup g{};
  g.count = 1;
  g.transB = transB;
  g.lower_out = lower_out;
  g.a_lower = a_lower;
  g.b_lower = b_lower;
  GemmProblem &p = g.p[0];
  p.A = A;
  p.B = B;
  p.C = C;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.M = M;
  p.N = N;
  p.K = K;
  p.alpha = alpha;
  p.beta = beta;
  return gemm_f32_grouped(g, stream, name);
}

}  // namespace gptq
