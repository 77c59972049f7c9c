// fp32 GEMM engine.
//
//   C = alpha * A * op(B) + beta * C,  A row-major M x K,
//   op(B) = B (row-major K x N) or B^T (B row-major N x K).
//
// Used for the dense parts of the inverse-Hessian factorization (triangular
// solve against the diagonal block, trailing symmetric update, the products
// of the recursive triangular inverse) and for the lazy trailing update of
// the column sweep ("GPTQ", section Komponenty: block updates).
//
// Two kernels.  Launches of at least kSmallLaunch 128 x 128 tiles run on
// bf16 MFMAs with each fp32 operand split into three bf16 terms (six MFMAs
// per fp32 product, fp32 accumulation; see the section of gemm_x3_kernel).
// Smaller launches, products written in place over A and K < 16 run on fp32
// MFMAs (v_mfma_f32_32x32x2f32), described next.
//
// fp32 MFMA kernel.  Tiles are 128 x 128 with four 64 x 64 wave tiles, or
// 64 x 64 with four 32 x 32 wave tiles for launches too small to fill the
// chip with the large tile.  A grouped launch runs up to kMaxGemmGroup
// independent problems of one shape class, each workgroup finding its
// problem by tile index.
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

#include <type_traits>

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

// The tile of workgroup blockIdx.x: its problem, the tile origin and the
// k range [kbeg, kend) that can hold nonzero products (kbeg a multiple of
// kStep).
template <int kTM, int kTN, int kStep>
__device__ __forceinline__ const GemmProblem &find_tile(const GemmGroup &g, int &m0, int &n0,
                                                        int &kbeg, int &kend) {
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
  m0 = tm * kTM;
  n0 = tn * kTN;
  kbeg = 0;
  kend = P.K;
  if (g.b_lower) kbeg = min(n0, P.K) & ~(kStep - 1);
  if (g.a_lower) kend = min(P.K, m0 + kTM);
  return P;
}

// Epilogue of a wave's kFM x kFN 32 x 32 accumulator tiles at (r0, c0).
// 32x32 result layout: lane l, element v -> row 8*(v/4) + 4*(l/32) + v%4,
// col l%32.  With beta != 0 the C tile is read first, all loads from
// clamped (valid) addresses before any store.
template <int kFM, int kFN>
__device__ __forceinline__ void store_tile(const GemmGroup &g, const GemmProblem &P,
                                           const f32x16_t (&acc)[kFM][kFN], int r0, int c0,
                                           int lane) {
  const int h = lane >> 5, l32 = lane & 31;
  const float alpha = P.alpha, beta = P.beta;
  float cv[kFM][kFN][16];
  if (beta != 0.f) {
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) {
        const int gc = min(c0 + j * 32 + l32, P.N - 1);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int gr = min(r0 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3), P.M - 1);
          cv[i][j][v] = P.C[int64_t(gr) * P.ldc + gc];
        }
      }
  }
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int gc = c0 + j * 32 + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int gr = r0 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        const float r = alpha * acc[i][j][v];
        const float out = (beta == 0.f) ? r : fmaf(beta, cv[i][j][v], r);
        if (gr < P.M && gc < P.N && (!g.lower_out || gr >= gc))
          P.C[int64_t(gr) * P.ldc + gc] = out;
      }
    }
}

template <int kTM, int kTN, int kTransB, bool kVec>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
    gemm_f32_kernel(GemmGroup g) {
  constexpr int kWM = Edge<kTM>::kW, kFM = Edge<kTM>::kF;
  constexpr int kWN = Edge<kTN>::kW, kFN = Edge<kTN>::kF;
  constexpr int kCA = Edge<kTM>::kChunks, kCB = Edge<kTN>::kChunks;
  constexpr int kBStage = kTransB ? kTN * kPK : kBK * Edge<kTN>::kPN;
  int m0, n0, kbeg, kend;
  const GemmProblem &P = find_tile<kTM, kTN, kBK>(g, m0, n0, kbeg, kend);

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

  store_tile<kFM, kFN>(g, P, acc, m0 + wm * kWM, n0 + wn * kWN, lane);
}

// ---------------------------------------------------------------------------
// fp32 products on bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// gfx950's bf16 matrix rate is 16 times its fp32 one.  Each fp32 operand is
// split into three bf16 terms, a = a0 + a1 + a2 with a0 = bf16(a),
// a1 = bf16(a - a0), a2 = bf16(a - a0 - a1) (round to nearest even; the
// remainders are exact in fp32, |a1| <= 2^-8 |a|, |a2| <= 2^-16 |a|), and a
// product a b is taken as the six terms a0b0 + a0b1 + a1b0 + a0b2 + a1b1 +
// a2b0, every bf16 x bf16 product exact in the fp32 accumulator.  What is
// left out (a1b2 + a2b1 + a2b2, and the part of a below a2's precision) is
// at most about 4 * 2^-24 |a b|: the same order as the rounding of an fp32
// product, so the GEMM keeps fp32 accuracy at six bf16 MFMAs per fp32 one.
//
// Tiles are 128 x 128 with four 64 x 64 wave tiles (2 x 2 MFMA tiles of
// 32 x 32); k advances in stages of 16, one MFMA chunk.  Operands are split
// once, when a stage is copied into LDS: a row of A (or a column of op(B))
// holds its 16 k as six 16-byte pieces, plane p's k half h at piece 2p + h,
// in a 112-byte row (the pitch spreads the MFMA reads of 16 consecutive
// rows over distinct banks).  In the B form (B row-major K x N) the copy
// transposes: each lane gathers 8 k of one column with 4-byte loads that
// are contiguous across lanes.  LDS is double buffered, 56 KB per
// workgroup, two workgroups per CU; stage s+2 is loaded while stage s is
// multiplied, and stage s+1 is split and written to LDS between its MFMAs.
namespace x3 {
constexpr int kT = 128;                // tile edge
constexpr int kStep = 16;              // k per stage
constexpr int kPitch = 112;            // bytes per LDS row: 6 pieces + 16 bytes of padding
constexpr int kOperand = kT * kPitch;  // 14 KB
constexpr int kStage = 2 * kOperand;   // A, then op(B)
constexpr int kLds = 2 * kStage;       // 56 KB, double buffered
}  // namespace x3

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// byte offset of plane p, k half h of LDS row `row`
__device__ __forceinline__ int x3_piece(int row, int p, int h) {
  return row * x3::kPitch + (2 * p + h) * 16;
}

// Split 8 consecutive-k values (v[0], v[1]) of one row into the three
// planes, k half h, of LDS row `row` of operand op.
__device__ __forceinline__ void x3_split_store(uint8_t *op, int row, int h, const f32x4_t (&v)[2]) {
  u32x4_t p0, p1, p2;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x4_t &q = v[e >> 1];
    const f32x2_t a = {q[2 * (e & 1)], q[2 * (e & 1) + 1]};
    const bf16x2_t b0 = __builtin_convertvector(a, bf16x2_t);
    const f32x2_t r1 = a - __builtin_convertvector(b0, f32x2_t);
    const bf16x2_t b1 = __builtin_convertvector(r1, bf16x2_t);
    const f32x2_t r2 = r1 - __builtin_convertvector(b1, f32x2_t);
    const bf16x2_t b2 = __builtin_convertvector(r2, bf16x2_t);
    p0[e] = __builtin_bit_cast(uint32_t, b0);
    p1[e] = __builtin_bit_cast(uint32_t, b1);
    p2[e] = __builtin_bit_cast(uint32_t, b2);
  }
  *reinterpret_cast<u32x4_t *>(op + x3_piece(row, 0, h)) = p0;
  *reinterpret_cast<u32x4_t *>(op + x3_piece(row, 1, h)) = p1;
  *reinterpret_cast<u32x4_t *>(op + x3_piece(row, 2, h)) = p2;
}

template <int kTransB, bool kVec>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
    gemm_x3_kernel(GemmGroup g) {
  using namespace x3;
  int m0, n0, kbeg, kend;
  const GemmProblem &P = find_tile<kT, kT, kStep>(g, m0, n0, kbeg, kend);
  extern __shared__ __align__(16) uint8_t xs[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;
  // this thread's copy group in each operand: 8 k (half gh) of one row of
  // A or op(B) (grow), or in the B form of one column (gcol)
  const int grow = tid >> 1, gh = tid & 1;
  const int gcol = tid & (kT - 1), gkh = tid >> 7;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Stages: the full 16-k steps of [kbeg, kend), and a ragged one for the
  // last kend - kbeg mod 16 values, which is multiplied first (stage 0) so
  // that only the stages before the main loop take masked loads.  Rows of A
  // and columns of op(B) past the matrix are read clamped to its last one:
  // they only feed outputs that are never stored.
  const int nfull = kend > kbeg ? (kend - kbeg) / kStep : 0;
  const int ragged = kend > kbeg && (kend - kbeg) % kStep != 0 ? 1 : 0;
  const int nsteps = nfull + ragged;
  // s < 0: a stand-in stage at k = 0 (every problem has K >= 16), loaded
  // where the pipeline runs past the last stage so that no load is
  // conditional inside the main loop; its values are never multiplied.
  auto stage_k = [&](int s) {
    return s < 0 ? 0 : kbeg + kStep * (s < ragged ? nfull : s - ragged);
  };

  // staged fp32 values of one stage: a = the A group, b = the op(B) group
  struct Staged {
    f32x4_t a[2], b[2];
  };
  // kMask: k past kend reads as zero (the ragged stage only)
  auto load = [&](Staged &r, int s, auto mask_tag) {
    constexpr bool kMask = decltype(mask_tag)::value;
    const int k0 = stage_k(s);
    {
      const int gr = min(m0 + grow, P.M - 1), gk = k0 + 8 * gh;
      const float *p = P.A + int64_t(gr) * P.lda + gk;
      if (kVec && !kMask) {
        r.a[0] = *reinterpret_cast<const f32x4_t *>(p);
        r.a[1] = *reinterpret_cast<const f32x4_t *>(p + 4);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) r.a[e >> 2][e & 3] = (!kMask || gk + e < kend) ? p[e] : 0.f;
      }
    }
    if (kTransB) {
      const int gn = min(n0 + grow, P.N - 1), gk = k0 + 8 * gh;
      const float *p = P.B + int64_t(gn) * P.ldb + gk;
      if (kVec && !kMask) {
        r.b[0] = *reinterpret_cast<const f32x4_t *>(p);
        r.b[1] = *reinterpret_cast<const f32x4_t *>(p + 4);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) r.b[e >> 2][e & 3] = (!kMask || gk + e < kend) ? p[e] : 0.f;
      }
    } else {
      const int gn = min(n0 + gcol, P.N - 1), gk = k0 + 8 * gkh;
      const float *p = P.B + int64_t(gk) * P.ldb + gn;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        r.b[e >> 2][e & 3] = (!kMask || gk + e < kend) ? p[int64_t(e) * P.ldb] : 0.f;
    }
  };
  using Masked = std::integral_constant<bool, true>;
  using Full = std::integral_constant<bool, false>;
  // split and store group q (0: A, 1: op(B)) of a staged set into buffer buf
  auto store_one = [&](const Staged &r, int buf, int q) {
    uint8_t *base = xs + buf * kStage;
    if (q == 0)
      x3_split_store(base, grow, gh, r.a);
    else if (kTransB)
      x3_split_store(base + kOperand, grow, gh, r.b);
    else
      x3_split_store(base + kOperand, gcol, gkh, r.b);
  };

  // One plane of one operand: v[i] = rows (A) or columns (op(B)) of MFMA
  // tile i of this wave, k = 8 h .. 8 h + 7 of the stage.
  struct Plane {
    bf16x8_t v[2];
  };
  auto rd = [&](Plane &f, int buf, int opnd, int p) {
    const uint8_t *base = xs + buf * kStage + opnd * kOperand;
    const int w = opnd ? wn : wm;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      f.v[i] = *reinterpret_cast<const bf16x8_t *>(base + x3_piece(w * 64 + i * 32 + l32, p, h));
  };
  // the four MFMAs of one product term; hook(q) after MFMA q of the stage
  auto term = [&](const Plane &fa, const Plane &fb, int t, auto &&hook) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa.v[i], fb.v[j], acc[i][j], 0, 0, 0);
        hook(t * 4 + i * 2 + j);
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  // Pipeline.  Stage s (buffer s & 1): the loads of stage s+2 are issued;
  // the four planes a1, b1, a0, b2 of stage s are read; the six terms run,
  // smallest first (a2b0, a1b1, a0b2, a1b0, a0b1, a0b0), with the staged
  // groups of stage s+1 split and written to the other buffer after MFMAs
  // 0 (A) and 12 (op(B)).  After the fourth term a workgroup barrier makes
  // stage s+1 complete and ends every read of buffer s & 1 (the last is
  // waited for by the third term), which stage s+1 overwrites; then a2 and
  // b0 of stage s+1 are read while the last two terms run.  Inside the main
  // loop every load, store and LDS read is unconditional (past the last
  // stage they move stand-in data that is never multiplied), so the wait
  // counters see one fixed pattern and the loads of stage s+2 stay in
  // flight across stage s.
  if (nsteps > 0) {
    Staged r0, r1;
    Plane a2, b0;
    if (ragged)
      load(r0, 0, Masked{});
    else
      load(r0, 0, Full{});
    store_one(r0, 0, 0);
    store_one(r0, 0, 1);
    load(r1, nsteps > 1 ? 1 : -1, Full{});
    __syncthreads();
    rd(a2, 0, 0, 2);
    rd(b0, 0, 1, 0);
    auto stage = [&](int s, Staged &cur, Staged &nxt) {
      const int buf = s & 1;
      // keep the accumulators in AGPRs across the loop (without this the
      // loop-carried copies land in VGPRs and are moved back every pass)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) asm volatile("" : "+a"(acc[i][j]));
      load(cur, s + 2 < nsteps ? s + 2 : -1, Full{});
      auto hook = [&](int q) {
        if (q == 0) store_one(nxt, buf ^ 1, 0);
        if (q == 12) store_one(nxt, buf ^ 1, 1);
      };
      Plane a1, b1, a0, b2, b0n;
      rd(a1, buf, 0, 1);
      rd(b1, buf, 1, 1);
      rd(a0, buf, 0, 0);
      rd(b2, buf, 1, 2);
      term(a2, b0, 0, hook);
      term(a1, b1, 1, hook);
      term(a0, b2, 2, hook);
      term(a1, b0, 3, hook);
      __syncthreads();
      rd(a2, buf ^ 1, 0, 2);
      rd(b0n, buf ^ 1, 1, 0);
      term(a0, b1, 4, hook);
      term(a0, b0, 5, hook);
      b0 = b0n;
    };
    int s = 0;
    for (; s + 1 < nsteps; s += 2) {
      stage(s, r0, r1);
      stage(s + 1, r1, r0);
    }
    if (s < nsteps) stage(s, r0, r1);
  }
  store_tile<2, 2>(g, P, acc, m0 + wm * 64, n0 + wn * 64, lane);
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

template <int kTransB, bool kVec>
gptq_status launch_x3_one(const GemmGroup &g, hipStream_t stream, const char *name) {
  const void *k = reinterpret_cast<const void *>(gemm_x3_kernel<kTransB, kVec>);
  GPTQ_TRY(allow_dynamic_lds(k, x3::kLds));
  return launch(name, gemm_x3_kernel<kTransB, kVec>, dim3(g.total_tiles), dim3(kThreads),
                x3::kLds, stream, g);
}

gptq_status launch_x3(const GemmGroup &g0, hipStream_t stream, const char *name) {
  GemmGroup g = g0;
  int total = 0;
  bool vec = true;
  int n = 0;
  for (int i = 0; i < g0.count; ++i) {
    const GemmProblem &p = g0.p[i];
    if (p.M <= 0 || p.N <= 0) continue;
    GemmProblem q = p;
    const int tm = (int)cdiv(p.M, x3::kT), tn = (int)cdiv(p.N, x3::kT);
    q.tiles_n = tn;
    q.tile_begin = total;
    total += g.lower_out ? tm * (tm + 1) / 2 : tm * tn;
    vec = vec && vec_ok(p.A, p.lda) && (!g.transB || vec_ok(p.B, p.ldb));
    g.p[n++] = q;
  }
  g.count = n;
  g.total_tiles = total;
  if (n == 0) return GPTQ_OK;
  if (g.transB) return vec ? launch_x3_one<1, true>(g, stream, name) : launch_x3_one<1, false>(g, stream, name);
  return vec ? launch_x3_one<0, true>(g, stream, name) : launch_x3_one<0, false>(g, stream, name);
}

}  // namespace

// Large tiles unless they would leave most of the chip idle: with fewer
// than kSmallLaunch 128 x 128 tiles, 64-row tiles give more workgroups.
// Large launches take the split-bf16 kernel unless a problem has K < 16
// (its stand-in stage reads k = 0..15).
// A product written in place over its A operand (C == A, one column tile
// of N <= 128) keeps whole 128-column rows per workgroup: 64 x 128 tiles.
constexpr int kSmallLaunch = 256;

gptq_status gemm_f32_grouped(const GemmGroup &g0, hipStream_t stream, const char *name) {
  int64_t tiles128 = 0;
  bool inplace = false, short_k = false;
  for (int i = 0; i < g0.count; ++i) {
    const GemmProblem &p = g0.p[i];
    if (p.M <= 0 || p.N <= 0) continue;
    const int64_t tm = cdiv(p.M, 128), tn = cdiv(p.N, 128);
    tiles128 += g0.lower_out ? tm * (tm + 1) / 2 : tm * tn;
    inplace = inplace || p.C == p.A;
    short_k = short_k || p.K < x3::kStep;
  }
  if (inplace) {
    for (int i = 0; i < g0.count; ++i)
      if (g0.p[i].N > 128 || g0.lower_out)
        return fail(GPTQ_ERR_INVALID_ARG, std::string(name) + ": in-place product wider than 128");
    return tiles128 < kSmallLaunch ? launch_grouped<64, 128>(g0, stream, name)
                                   : launch_grouped<128, 128>(g0, stream, name);
  }
  if (tiles128 < kSmallLaunch) return launch_grouped<64, 64>(g0, stream, name);
  if (short_k) return launch_grouped<128, 128>(g0, stream, name);
  return launch_x3(g0, stream, name);
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
