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
// tile.  A grouped launch runs up to kMaxGemmGroup independent problems of
// one shape class, each workgroup finding its problem by tile index.
//
// Operand staging.  A tile of A (and of B in the B^T form) is copied into LDS
// as it lies in memory, row by row with k contiguous, in 16-byte pieces; no
// transpose.  The k order inside each 16-k chunk is permuted so that one
// 16-byte LDS read gives a lane the operands of four MFMAs: MFMA t (0..7) of
// a chunk takes k = 8 h + t in lane half h (lanes 0-31: h = 0, lanes 32-63:
// h = 1), so lane (h, row) reads k = 8h .. 8h+7 of its row as two 16-byte
// pieces.  The sum over k is the same sum in another order.  In the B form
// (k-major rows, n contiguous) B is also copied as it lies, and each MFMA
// operand is one 4-byte read of row k = 8h + t.
#include "common.h"

namespace gptq {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBK = 32;         // k per stage (two 16-k chunks)
constexpr int kPK = kBK + 4;    // LDS pitch (floats) of a [row][k] tile: 16-byte aligned rows;
                                // the 16-byte reads of 8 consecutive rows hit 8 distinct
                                // 4-bank groups
constexpr int kThreads = 256;

// Geometry of one operand tile with kE rows (M or N edge).
template <int kE>
struct Edge {
  static constexpr int kPN = kE + 4;                       // pitch of a [k][n] tile (B form)
  static constexpr int kChunks = kE * kBK / 4 / kThreads;  // 16-byte pieces per thread
  static constexpr int kW = kE / 2;                        // wave tile edge (2 x 2 waves)
  static constexpr int kF = kW / 32;                       // 32 x 32 MFMA tiles per wave edge
};

// Stage one [row][k] operand tile (kT rows x kBK k, row-major in memory with
// leading dimension ld) into registers.  Piece c of the tile is row c / 8,
// k = 4 (c % 8): eight lanes read one row's 128 contiguous bytes.  Elements
// outside [0, rows) x [k0, kend) are zero.
template <int kT, bool kVec>
__device__ __forceinline__ void load_rows(const float *__restrict__ P, int64_t ld, int rows,
                                          int r0, int k0, int kend, int tid,
                                          f32x4_t (&v)[Edge<kT>::kChunks]) {
#pragma unroll
  for (int i = 0; i < Edge<kT>::kChunks; ++i) {
    const int c = tid + kThreads * i;
    const int r = c >> 3, kc = (c & 7) * 4;
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
    v[i] = *reinterpret_cast<const f32x4_t *>(P + int64_t(r0 + (c >> 3)) * ld + k0 + (c & 7) * 4);
  }
}

template <int kT>
__device__ __forceinline__ void store_rows(float *lds, int tid, int i, const f32x4_t &v) {
  const int c = tid + kThreads * i;
  *reinterpret_cast<f32x4_t *>(lds + (c >> 3) * kPK + (c & 7) * 4) = v;
}

// B in row-major K x N: a tile (kBK k-rows x kT cols) is already k-major.
template <int kT, bool kVec>
__device__ __forceinline__ void load_kmajor(const float *__restrict__ P, int64_t ld, int cols,
                                            int c0, int k0, int kend, int tid,
                                            f32x4_t (&v)[Edge<kT>::kChunks]) {
  constexpr int kPerRow = kT / 4;  // 16-byte pieces per k-row
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
__device__ __forceinline__ void store_kmajor(float *lds, int tid, int i, const f32x4_t &v) {
  constexpr int kPerRow = kT / 4;
  const int c = tid + kThreads * i;
  *reinterpret_cast<f32x4_t *>(lds + (c / kPerRow) * Edge<kT>::kPN + (c % kPerRow) * 4) = v;
}

template <int kTM, int kTN, int kTransB, bool kVec>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
    gemm_f32_kernel(GemmGroup g) {
  constexpr int kWM = Edge<kTM>::kW, kFM = Edge<kTM>::kF;
  constexpr int kWN = Edge<kTN>::kW, kFN = Edge<kTN>::kF;
  constexpr int kCA = Edge<kTM>::kChunks, kCB = Edge<kTN>::kChunks;
  constexpr int kBStage = kTransB ? kTN * kPK : kBK * Edge<kTN>::kPN;
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

  __shared__ __align__(16) float As[2][kTM * kPK];
  __shared__ __align__(16) float Bs[2][kBStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;

  f32x16_t acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const float alpha = P.alpha, beta = P.beta;

  const int nsteps = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;
  // Two register sets of staged pieces, used by stage parity: the set of
  // stage s+2 is loaded while stage s is multiplied, so each load has a
  // stage and a half to land before its LDS store.
  struct Staged {
    f32x4_t a[kCA], b[kCB];
  };
  // Interior tiles (the common case) take unconditional 16-byte loads; edge
  // tiles and ragged k ranges take the masked loads.
  const bool rows_in = m0 + kTM <= P.M && n0 + kTN <= P.N;
  auto load = [&](Staged &r, int s) {
    const int k0 = kbeg + s * kBK;
    if (kVec && rows_in && k0 + kBK <= kend) {
      load_rows_fast<kTM>(P.A, P.lda, m0, k0, tid, r.a);
      if (kTransB)
        load_rows_fast<kTN>(P.B, P.ldb, n0, k0, tid, r.b);
      else
        load_kmajor_fast<kTN>(P.B, P.ldb, n0, k0, tid, r.b);
      return;
    }
    load_rows<kTM, kVec>(P.A, P.lda, P.M, m0, k0, kend, tid, r.a);
    if (kTransB)
      load_rows<kTN, kVec>(P.B, P.ldb, P.N, n0, k0, kend, tid, r.b);
    else
      load_kmajor<kTN, kVec>(P.B, P.ldb, P.N, n0, k0, kend, tid, r.b);
  };
  // staged piece q (A pieces first, then B) into LDS buffer buf
  auto store_one = [&](const Staged &r, int buf, int q) {
    if (q < kCA) {
      store_rows<kTM>(As[buf], tid, q, r.a[q]);
    } else if (kTransB) {
      store_rows<kTN>(Bs[buf], tid, q - kCA, r.b[q - kCA]);
    } else {
      store_kmajor<kTN>(Bs[buf], tid, q - kCA, r.b[q - kCA]);
    }
  };

  // Operands of one 16-k chunk: fa[i][u] holds k = 8h + 4u .. 8h + 4u + 3 of
  // A row (wave row tile, fragment i); likewise fb for B^T rows, or fbk[j][t]
  // the B value of MFMA t in the B form.
  struct Frag {
    f32x4_t a[kFM][2];
    f32x4_t b[kTransB ? kFN : 1][2];
    float bk[kTransB ? 1 : kFN][8];
  };
  auto read_chunk = [&](Frag &f, int buf, int ch) {
    const float *A = As[buf];
    const float *B = Bs[buf];
    const int kk = ch * 16 + 8 * h;
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        f.a[i][u] = *reinterpret_cast<const f32x4_t *>(A + (wm * kWM + i * 32 + l32) * kPK + kk + 4 * u);
    if (kTransB) {
#pragma unroll
      for (int j = 0; j < kFN; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          f.b[j][u] =
              *reinterpret_cast<const f32x4_t *>(B + (wn * kWN + j * 32 + l32) * kPK + kk + 4 * u);
    } else {
#pragma unroll
      for (int j = 0; j < kFN; ++j)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          f.bk[j][t] = B[(kk + t) * Edge<kTN>::kPN + wn * kWN + j * 32 + l32];
    }
  };
  // The MFMAs of one chunk; after MFMA q, hook(q) issues the memory
  // operations planned for that slot.
  auto mfma_chunk = [&](const Frag &f, auto &&hook) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j) {
          const float a = f.a[i][t >> 2][t & 3];
          const float b = kTransB ? f.b[j][t >> 2][t & 3] : f.bk[j][t];
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[i][j], 0, 0, 0);
          hook((t * kFM + i) * kFN + j);
          __builtin_amdgcn_sched_barrier(0);
        }
  };

  // Pipeline: the operands of chunk 1 are read from LDS while chunk 0's
  // MFMAs run; the staged pieces of stage s+1 (loaded during stage s-1) are
  // written to the other LDS buffer (last read before the previous barrier)
  // spread over chunk 1's MFMAs, and the pieces of stage s+2 are loaded.
  constexpr int kMfmas = 8 * kFM * kFN;          // per chunk
  constexpr int kPieces = kCA + kCB;             // staged 16-byte pieces per thread
  constexpr int kEvery = kMfmas / kPieces > 0 ? kMfmas / kPieces : 1;
  if (nsteps > 0) {
    Staged r0, r1;
    Frag x, y;
    load(r0, 0);
#pragma unroll
    for (int q = 0; q < kPieces; ++q) store_one(r0, 0, q);
    if (nsteps > 1) load(r1, 1);
    __syncthreads();
    read_chunk(x, 0, 0);
    // stage s: LDS buffer s & 1; `nxt` holds stage s+1, `cur` receives s+2
    auto stage = [&](int s, Staged &cur, Staged &nxt) {
      const int buf = s & 1;
      const bool more = s + 1 < nsteps;
      if (s + 2 < nsteps) load(cur, s + 2);
      read_chunk(y, buf, 1);
      mfma_chunk(x, [](int) {});
      mfma_chunk(y, [&](int q) {
        if (more && q % kEvery == 0 && q / kEvery < kPieces) store_one(nxt, buf ^ 1, q / kEvery);
      });
      __syncthreads();
      if (more) read_chunk(x, buf ^ 1, 0);
    };
    for (int s = 0; s < nsteps; s += 2) {
      stage(s, r0, r1);
      if (s + 1 < nsteps) stage(s + 1, r1, r0);
    }
  }

  // ---- epilogue.  32x32 result layout: lane l, element v ->
  //      row 8*(v/4) + 4*(l/32) + v%4, col l%32.  With beta != 0 the C tile is
  //      read first, all loads from clamped (valid) addresses before any store.
  float cv[kFM][kFN][16];
  if (beta != 0.f) {
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) {
        const int gc = min(n0 + wn * kWN + j * 32 + l32, P.N - 1);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int gr = min(m0 + wm * kWM + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3), P.M - 1);
          cv[i][j][v] = P.C[int64_t(gr) * P.ldc + gc];
        }
      }
  }
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int gc = n0 + wn * kWN + j * 32 + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int gr = m0 + wm * kWM + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
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
