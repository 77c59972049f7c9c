// Hessian accumulation H += 2 X X^T ("GPTQ", section Komponenty) and the
// float64 activation energy hdiag += 2 sum_t x_it^2.
//
// bf16 path: a SYRK on bf16 MFMA, fp32 accumulate.  Only the upper-triangle
// 256x256 tiles of H are computed: diagonal tiles on v_mfma_f32_32x32x16_bf16
// (with the energy), the others on v_mfma_f32_16x16x32_bf16, which holds a
// higher shader clock on gfx950 for the same work.  Most tiles are
// owned by one workgroup that runs the whole token loop, so H is updated by
// one read-modify-write per tile.  The tiles of the last, partly filled
// round may instead be split into `parts` token ranges run by different
// workgroups: part 0 adds into H, parts 1.. store their sums into workspace
// slots, and a second kernel adds the slots into H in part order, so the
// result is deterministic (no split-K atomics).  X is d x n row-major (tokens contiguous), so both MFMA operands
// are K-contiguous rows of X and no transpose is needed anywhere.  X panels
// stream through registers into a double-buffered LDS ring; on diagonal
// tiles the four waves also accumulate the float64 activation energy of the
// tile's rows from the same LDS data, in the shadow of their MFMAs.
#include <type_traits>

#include "common.h"

namespace gptq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int kTile = 256;       // H tile edge
constexpr int kBK = 64;          // tokens per pipeline stage
constexpr int kThreads = 256;    // 4 waves (1 per SIMD), each a 128 x 128 sub-tile
constexpr int kStages = 2;       // LDS ring depth (double buffer)
constexpr int kRowBytes = kBK * 2;                 // 128 B of one X row per stage
constexpr int kChunks = kRowBytes / 16;            // 16-byte chunks per row
constexpr int kPanelBytes = kTile * kRowBytes;     // 32 KB per operand per stage
constexpr int kStageBytes = 2 * kPanelBytes;
constexpr int kGroupRows = 4;    // tile-order band height (panel reuse in L2)

// Wait until at most N vector-memory operations of this wave are in flight
// (the global->LDS copies count as vector-memory operations).
template <int N>
__device__ __forceinline__ void vm_wait() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}

// 16-byte chunk position inside a 128-byte LDS row, XOR-swizzled so that the
// MFMA operand reads (lanes 0-31: rows 0-31 at chunk c, lanes 32-63: the
// same rows at chunk c+1) spread over the LDS banks.  Picked with the LDS
// bank-conflict counter on gfx950 among XOR and rotation candidates: this
// one is conflict-free for all four 16-token steps of a stage.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// A stage (two 256-row x 64-token panels) reaches LDS through registers:
// 16 loads of 16 bytes per lane.  On gfx950 ordinary loads sustained a
// higher per-CU copy rate than direct global->LDS copies (about 56 GB/s per
// CU with every CU streaming), and that rate, not the matrix cores, bounds
// this kernel.  Rows past d are clamped to row d-1 (they only feed outputs
// that are never stored).
constexpr int kLoads = kStageBytes / 16 / kThreads;   // 16 per lane per stage
constexpr int kPanelLoads = kLoads / 2;

// Ragged last stage: register path with element masks (tokens >= n are 0).
__device__ __forceinline__ void tail_panel(const uint16_t *__restrict__ X, int64_t ld, int64_t d,
                                           int64_t n, int64_t row0, int64_t k0, uint8_t *lds,
                                           int tid) {
#pragma unroll
  for (int i = 0; i < kPanelBytes / 16 / kThreads; ++i) {
    const int slot = tid + kThreads * i;
    const int r = slot / kChunks, c = (slot % kChunks) ^ swz(r);
    const int64_t gr = min(row0 + r, d - 1);
    const int64_t gk = k0 + c * 8;
    const uint16_t *p = X + gr * ld + gk;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (gk + e < n) ? p[e] : 0u;
    u32x4_t v;
    v[0] = h[0] | (h[1] << 16);
    v[1] = h[2] | (h[3] << 16);
    v[2] = h[4] | (h[5] << 16);
    v[3] = h[6] | (h[7] << 16);
    *reinterpret_cast<u32x4_t *>(lds + slot * 16) = v;
  }
}

__device__ __forceinline__ bf16x8_t read_frag(const uint8_t *lds, int row, int chunk) {
  return *reinterpret_cast<const bf16x8_t *>(lds + row * kRowBytes + ((chunk ^ swz(row)) << 4));
}

// Upper-triangle tile t (in band order) -> (ti, tj), ti <= tj.  Tiles are
// ordered band by band (kGroupRows tile-rows per band); inside a band by
// column tj, then by row.  Consecutive tiles share X panels.
__device__ __forceinline__ void tile_coords(int t, int nt, int &ti, int &tj) {
  int b0 = 0;
  while (true) {
    const int h = min(kGroupRows, nt - b0);
    const int tri = h * (h + 1) / 2;            // tj in [b0, b0+h)
    const int rect = h * (nt - b0 - h);          // tj in [b0+h, nt)
    if (t < tri + rect) {
      if (t < tri) {
        int c = 0;
        while ((c + 1) * (c + 2) / 2 <= t) ++c;
        tj = b0 + c;
        ti = b0 + (t - c * (c + 1) / 2);
      } else {
        const int u = t - tri;
        tj = b0 + h + u / h;
        ti = b0 + u % h;
      }
      return;
    }
    t -= tri + rect;
    b0 += h;
  }
}

__device__ __forceinline__ double bf16_to_f64(uint32_t bits16) {
  return (double)__uint_as_float(bits16 << 16);
}

// Work of one XCD.  Workgroups are dealt round-robin to the 8 XCDs, so each
// XCD gets a contiguous run of the tile order (tiles that share X panels
// share that XCD's L2): tiles [first, first + full + tail).  Its `cus`
// compute units take the `full` tiles in whole rounds; the `tail` tiles of
// the last, partly filled round are split into token parts.
struct XcdRun {
  int first, full, tail;
};
__host__ __device__ inline XcdRun xcd_run(int x, int ntiles, int cus) {
  const int f = (x * ntiles) / 8, r = ((x + 1) * ntiles) / 8 - f;
  const int full = (r % cus == 0) ? r : (r / cus) * cus;
  return {f, full, r - full};
}

// Workspace slot of a split tile's part p >= 1: its 256 x 256 sums (2 X X^T
// over the part's tokens, row-major), then, for a diagonal tile, the 256
// rows' float64 energies.
constexpr int64_t kSlotFloats = int64_t(kTile) * kTile + 2 * kTile;
constexpr size_t kSlotBytes = size_t(kSlotFloats) * sizeof(float);

// ---- Off-diagonal tiles: 16x16x32 bf16 MFMAs, no energy.  On gfx950 this
// MFMA shape runs at a higher shader clock than 32x32x16 for the same work
// (1.74 against 1.52 GHz in this kernel).  Same LDS ring as the diagonal-tile
// path (two 64-token stages of 128-byte rows, same swizzle, conflict-free
// for the 16-row fragment reads by the bank-conflict counter); each stage
// is two 32-token steps.

// One off-diagonal tile (every entry above the diagonal): each wave owns a
// 128 x 128 sub-tile as 8 x 8 blocks of 16 x 16.  Iteration ks: step 0
// multiplies the first 32 tokens of stage ks with fragment set X while set Y
// (the second 32 tokens) is read, and stores stage ks+1 (loaded one
// iteration earlier) to the ring slot of stage ks-1, re-issuing each
// register's load for stage ks+2; a barrier makes stage ks+1 visible; step 1
// multiplies set Y while set X is read from stage ks+1.  Every read of a ring
// slot precedes the barrier after which that slot is rewritten.  The ragged
// token tail is one more stage whose loads come from clamped addresses and
// whose tokens at or past n are zeroed before they are stored.
__device__ __forceinline__ void syrk_tile16(float *__restrict__ H, const uint16_t *__restrict__ X,
                                            int64_t d, int64_t n, int64_t ld, int64_t I0,
                                            int64_t J0, int part, int nparts,
                                            float *__restrict__ dst_slot, uint8_t *smem,
                                            int tid) {
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  f32x4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Stages of this unit: the ragged token tail first (last part only; its
  // loads are masked), then whole 64-token stages.  Every unit has at least
  // one whole stage (the host checks it), so the loop below only ever
  // touches whole stages.
  const int64_t nfull = n / kBK;
  const int64_t ks0 = nfull * part / nparts;
  const int r = (part == nparts - 1 && nfull * kBK < n) ? 1 : 0;
  const int U = (int)(nfull * (part + 1) / nparts - ks0) + r;
  auto stage_k = [&](int t) {   // first token of stage t (past the last: the last)
    t = min(t, U - 1);
    return t < r ? nfull * kBK : (ks0 + t - r) * kBK;
  };

  // Load q of a lane: row tid/8 + 32 (q%8) of panel q/8 at 16-byte chunk
  // tid%8 (eight lanes read one row's 128 contiguous bytes).  The address is
  // a uniform base (the group's first row, clamped, at the stage's first
  // token) plus a per-lane 32-bit byte offset fixed for the whole loop, so a
  // load costs no vector ALU work.  Rows past d are clamped to row d-1.  The
  // ragged last stage takes the general per-lane path: a chunk wholly past n
  // reads the row's first chunk instead (zeroed when stored).
  const int lrow = tid >> 3, lchunk = tid & 7;
  const int lds_off = lrow * kRowBytes + ((lchunk ^ swz(lrow)) << 4);
  int64_t grow[kLoads];
  uint32_t voff[kLoads];
#pragma unroll
  for (int q = 0; q < kLoads; ++q) {
    const int64_t r0 = (q < kPanelLoads ? I0 : J0) + 32 * (q % kPanelLoads);
    grow[q] = min(r0, d - 1);
    voff[q] = uint32_t((min(r0 + lrow, d - 1) - grow[q]) * ld * 2 + lchunk * 16);
  }
  u32x4_t stg[kLoads];
  // Whole stage: a uniform base plus the lane's fixed offset, no vector ALU
  // work.  General form (the ragged stage, outside the loop): a chunk wholly
  // past n reads the row's first chunk instead, and at the store the tokens
  // at or past n become 0 (a chunk that holds n lies inside the row's
  // storage: ld is a multiple of 8 and at least n).
  auto load_one = [&](int q, int t) {
    const uint8_t *base = reinterpret_cast<const uint8_t *>(X + grow[q] * ld + stage_k(t));
    stg[q] = *reinterpret_cast<const u32x4_t *>(base + voff[q]);
  };
  auto load_any = [&](int q, int t) {
    const int64_t k = stage_k(t);
    const uint16_t *p = X + grow[q] * ld + voff[q] / 2;
    stg[q] = *reinterpret_cast<const u32x4_t *>(p + (k + lchunk * 8 < n ? k : 0));
  };
  auto store_one = [&](int q, int t) {
    *reinterpret_cast<u32x4_t *>(smem + (t & 1) * kStageBytes + lds_off +
                                 (q / kPanelLoads) * kPanelBytes +
                                 (q % kPanelLoads) * 32 * kRowBytes) = stg[q];
  };
  auto store_any = [&](int q, int t) {
    const int64_t valid = n - (stage_k(t) + lchunk * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      stg[q][w] &= (2 * w < valid ? 0xffffu : 0u) | (2 * w + 1 < valid ? 0xffff0000u : 0u);
    store_one(q, t);
  };
  // Set X (step 0): the B fragments and a ring of four A fragments (block
  // row i in slot i % 4), rows 0-2 read during the previous step 1, rows
  // 3-7 three block rows ahead inside step 0 (before the barrier that lets
  // their ring slot be rewritten).  Set Y (step 1, after that barrier) is
  // read whole during step 0.
  bf16x8_t xa[4], xb[8], ya[8], yb[8];
  auto frag_a = [&](int u, int h, int i) {
    return read_frag(smem + (u & 1) * kStageBytes, wm * 128 + 16 * i + (lane & 15),
                     4 * h + (lane >> 4));
  };
  auto frag_b = [&](int u, int h, int j) {
    return read_frag(smem + (u & 1) * kStageBytes + kPanelBytes, wn * 128 + 16 * j + (lane & 15),
                     4 * h + (lane >> 4));
  };
  // Copies: registers 8-15 carry stage u+1 into step 0 of iteration u (then
  // load stage u+2), registers 0-7 carry stage u+2 into step 1 of iteration
  // u (then load stage u+3).  Both land in a ring slot whose last reads came
  // before the previous barrier.
  if (U > 0) {
#pragma unroll
    for (int q = 0; q < kLoads; ++q) load_any(q, 0);
#pragma unroll
    for (int q = 0; q < kLoads; ++q) store_any(q, 0);
#pragma unroll
    for (int q = 0; q < kLoads; ++q) load_any(q, 1);
#pragma unroll
    for (int q = 0; q < kLoads / 2; ++q) {
      store_any(q, 1);
      load_any(q, 2);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int j = 0; j < 8; ++j) xb[j] = frag_b(0, 0, j);
    xa[0] = frag_a(0, 0, 0);
    xa[1] = frag_a(0, 0, 1);
    xa[2] = frag_a(0, 0, 2);
  }
  for (int u = 0; u < U; ++u) {
    // step 0, slot 8i+j: A row i+3 after (i, 1); set Y fragment f (a0 b0 ..
    // b7 a1 .. a7) in slot 4f+2; copy 8+i in slot 8i+5.
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i % 4], xb[j], acc[i][j], 0, 0, 0);
        const int q = 8 * i + j;
        if (j == 1 && i + 3 < 8) xa[(i + 3) % 4] = frag_a(u, 0, i + 3);
        if ((q & 3) == 2) {
          const int f = q >> 2;
          if (f == 0) ya[0] = frag_a(u, 1, 0);
          else if (f < 9) yb[f - 1] = frag_b(u, 1, f - 1);
          else ya[f - 8] = frag_a(u, 1, f - 8);
        }
        if (j == 5) {
          store_one(kLoads / 2 + i, u + 1);
          load_one(kLoads / 2 + i, u + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): stores of u+1, reads of u done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // step 1: set X of the next stage (past the last stage: unused), B
    // fragment i after (i, 2), A rows 0-2 after (i, 6); copy i in slot 8i+5.
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ya[i], yb[j], acc[i][j], 0, 0, 0);
        if (j == 2) xb[i] = frag_b(u + 1, 0, i);
        if (i < 3 && j == 6) xa[i] = frag_a(u + 1, 0, i);
        if (j == 5) {
          store_one(i, u + 2);
          load_one(i, u + 3);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  }
  // 16x16 MFMA result layout: lane l, element v -> row 4*(l/16) + v, col l%16.
  if (dst_slot) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = wn * 128 + 16 * j + (lane & 15);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = wm * 128 + 16 * i + 4 * (lane >> 4) + v;
          dst_slot[r * kTile + c] = 2.f * acc[i][j][v];
        }
      }
    return;
  }
  // H += 2 * acc inside the matrix (every entry of this tile is above the
  // diagonal).  One block row (32 values per lane) at a time: its loads are
  // issued from clamped (valid) addresses before any store.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float hv[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t gc = min(J0 + wn * 128 + 16 * j + (lane & 15), d - 1);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t gr = min(I0 + wm * 128 + 16 * i + 4 * (lane >> 4) + v, d - 1);
        hv[j][v] = H[gr * d + gc];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t gc = J0 + wn * 128 + 16 * j + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t gr = I0 + wm * 128 + 16 * i + 4 * (lane >> 4) + v;
        if (gr < d && gc < d) H[gr * d + gc] = hv[j][v] + 2.f * acc[i][j][v];
      }
    }
  }
}

// One workgroup per CU (128 KB of LDS) and one wave per SIMD: the kernel may
// use the whole register file, so both fragment sets stay in registers.
// Workgroup (xcd, slot): slot < full -> whole tile first + slot; else unit
// u = slot - full, part u / tail of tile first + full + u % tail (parts
// outermost, so that concurrent units read the same token range of
// neighbouring tiles).
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
    syrk_bf16_kernel(float *__restrict__ H, double *__restrict__ hdiag,
                     const uint16_t *__restrict__ X, int64_t d, int64_t n, int64_t ld, int nt,
                     int ntiles, int parts, int xcd_cus, float *__restrict__ slots,
                     int tile16) {
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const XcdRun run = xcd_run(xcd, ntiles, xcd_cus);
  int t, part = 0, nparts = 1;   // this unit: part `part` of `nparts` token ranges
  float *dst_slot = nullptr;
  if (slot < run.full) {
    t = run.first + slot;
  } else {
    nparts = parts;
    const int u = slot - run.full;
    if (u >= run.tail * parts) return;
    part = u / run.tail;
    t = run.first + run.full + u % run.tail;
    if (part > 0) {
      int gi = u % run.tail;             // index among all XCDs' tail tiles
      for (int x = 0; x < xcd; ++x) gi += xcd_run(x, ntiles, xcd_cus).tail;
      dst_slot = slots + (int64_t(gi) * (parts - 1) + part - 1) * kSlotFloats;
    }
  }
  int ti, tj;
  tile_coords(t, nt, ti, tj);
  const bool diag = ti == tj;
  const int64_t I0 = int64_t(ti) * kTile, J0 = int64_t(tj) * kTile;

  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  if (!diag && tile16) {
    syrk_tile16(H, X, d, n, ld, I0, J0, part, nparts, dst_slot, smem, tid);
    return;
  }
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;  // sub-tile rows wm*128.., cols wn*128..
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  // On a diagonal tile every wave also accumulates, in float64, the
  // activation energy of one 64-row quarter of the tile's rows (row
  // I0 + 64 wave + lane per lane) from the same LDS data, spread over its
  // MFMA slots; the lower-left sub-tile is multiplied but never stored.
  double en = 0.0;
  const int erow = 64 * wave + lane;

  // Stage ks is fetched into stg[] with ordinary 16-byte loads and stored to
  // its LDS slot one iteration later.  Load q of a lane is row
  // (tid/8 + 32 (q%8)) of panel q/8 (A: rows I0.., B: rows J0..; on a
  // diagonal tile both are the same rows, which keeps every tile on one
  // branch-free code path) at 16-byte chunk tid%8: eight lanes read one
  // row's 128 contiguous bytes (a whole cache line).  Stages past the last
  // full one re-load that one; that extra copy lands in a slot the tail
  // path overwrites.
  // this unit's full 64-token stages [ks0, ks1); the ragged token tail goes
  // with the last part
  const int64_t nfull = n / kBK;
  const int64_t ks0 = nfull * part / nparts, ks1 = nfull * (part + 1) / nparts;
  const bool has_tail = part == nparts - 1 && nfull * kBK < n;
  const int lrow = tid >> 3, lchunk = tid & 7;
  const int lds_off = lrow * kRowBytes + ((lchunk ^ swz(lrow)) << 4);
  const uint16_t *rp[kLoads];
#pragma unroll
  for (int q = 0; q < kLoads; ++q)
    rp[q] = X + min((q < kPanelLoads ? I0 : J0) + lrow + 32 * (q % kPanelLoads), d - 1) * ld +
            lchunk * 8;
  u32x4_t stg[kLoads];
  auto load_one = [&](int q, int64_t ks) {
    stg[q] = *reinterpret_cast<const u32x4_t *>(rp[q] + min(ks, ks1 - 1) * kBK);
  };
  auto store_one = [&](int q, int64_t ks) {
    *reinterpret_cast<u32x4_t *>(smem + (ks % kStages) * kStageBytes + lds_off +
                                 (q / kPanelLoads) * kPanelBytes +
                                 (q % kPanelLoads) * 32 * kRowBytes) = stg[q];
  };
  // Energy inputs: the two 16-byte chunks (16 tokens) of this lane's row
  // that 16-token step h of stage ks covers.
  auto energy_read = [&](u32x4_t (&e)[2], int64_t ks, int h) {
    const uint8_t *A = smem + (ks % kStages) * kStageBytes + erow * kRowBytes;
    e[0] = *reinterpret_cast<const u32x4_t *>(A + (((2 * h) ^ swz(erow)) << 4));
    e[1] = *reinterpret_cast<const u32x4_t *>(A + (((2 * h + 1) ^ swz(erow)) << 4));
  };
  // Token q of those 16, in token order.
  auto energy_acc = [&](const u32x4_t (&e)[2], int q) {
    const uint32_t w = e[q >> 3][(q >> 1) & 3];
    const double v = bf16_to_f64((q & 1) ? (w >> 16) : (w & 0xffffu));
    en = fma(v, v, en);
  };
  auto energy_stage = [&](int64_t ks) {
    u32x4_t e[2];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      energy_read(e, ks, h);
#pragma unroll
      for (int q = 0; q < 16; ++q) energy_acc(e, q);
    }
  };
  // Fragment f of 16-token step h of stage ks, in the order the MFMAs of a
  // step consume them: a0 b0 b1 b2 b3 a1 a2 a3.
  auto read_one = [&](bf16x8_t (&fa)[4], bf16x8_t (&fb)[4], int64_t ks, int h, int f) {
    const uint8_t *A = smem + (ks % kStages) * kStageBytes;
    const int c = 2 * h + (lane >> 5);
    if (f == 0) fa[0] = read_frag(A, wm * 128 + (lane & 31), c);
    else if (f < 5) fb[f - 1] = read_frag(A + kPanelBytes, wn * 128 + (f - 1) * 32 + (lane & 31), c);
    else fa[f - 4] = read_frag(A, wm * 128 + (f - 4) * 32 + (lane & 31), c);
  };
  auto read_step = [&](bf16x8_t (&fa)[4], bf16x8_t (&fb)[4], int64_t ks, int h) {
#pragma unroll
    for (int f = 0; f < 8; ++f) read_one(fa, fb, ks, h, f);
  };
  // The 16 MFMAs of one step; after MFMA q, hook(q) issues the memory
  // operations planned for that slot, so that fragment reads, stage stores
  // and global loads are spread over the matrix-core work instead of
  // stalling it.
  auto mfma_step = [&](const bf16x8_t (&fa)[4], const bf16x8_t (&fb)[4], auto &&hook) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        hook(4 * i + j);
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  // Pipeline (double-buffered LDS stages of 64 tokens, one more stage in
  // flight in registers).  Iteration ks multiplies stage ks in four 16-token
  // steps; the fragments of step h+1 are read (one per two MFMAs) while the
  // MFMAs of step h run.  Over steps 0-2 every third slot also stores one
  // register of stage ks+1 (loaded one iteration earlier) to the LDS slot
  // that stage ks-1 used (its reads all ended before the previous barrier)
  // and re-issues that register's load for stage ks+2, so the copies stay
  // in flight for a whole iteration and the LDS writes do not crowd the
  // fragment reads of one step (about 3% faster than all 16 in step 2).
  // A barrier then makes stage ks+1 visible (all reads of stage ks have
  // completed by then), and step 0 of stage ks+1 is read while step 3 of
  // stage ks is multiplied.
  // On diagonal tiles each slot also adds one token of the lane's energy
  // row, whose chunks are read one step ahead.
  auto tail = [&]() {
    __syncthreads();
    uint8_t *base = smem + (nfull % kStages) * kStageBytes;
    tail_panel(X, ld, d, n, I0, nfull * kBK, base, tid);
    tail_panel(X, ld, d, n, J0, nfull * kBK, base + kPanelBytes, tid);
    __syncthreads();
  };
  if (ks1 > ks0) {
#pragma unroll
    for (int q = 0; q < kLoads; ++q) load_one(q, ks0);
#pragma unroll
    for (int q = 0; q < kLoads; ++q) store_one(q, ks0);
#pragma unroll
    for (int q = 0; q < kLoads; ++q) load_one(q, ks0 + 1);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  }
  bf16x8_t xa[4], xb[4], ya[4], yb[4];
  auto main_loop = [&](auto energy_tag) {
    constexpr bool kEnergy = decltype(energy_tag)::value;
    u32x4_t ep[2], eq[2];  // energy chunks of even / odd steps
    if (ks1 > ks0) {
      read_step(xa, xb, ks0, 0);
      if (kEnergy) energy_read(ep, ks0, 0);
    }
    for (int64_t ks = ks0; ks < ks1; ++ks) {
      // copy c (0..15) of the stage sits in slot 3 (c % 6) of step c / 6
      auto copy = [&](int step, int q) {
        const int c = 6 * step + q / 3;
        if (q % 3 == 0 && c < kLoads) {
          store_one(c, ks + 1);
          load_one(c, ks + 2);
        }
      };
      mfma_step(xa, xb, [&](int q) {
        copy(0, q);
        if (q & 1) read_one(ya, yb, ks, 1, q >> 1);
        if (kEnergy) {
          if (q == 0) energy_read(eq, ks, 1);
          energy_acc(ep, q);
        }
      });
      mfma_step(ya, yb, [&](int q) {
        copy(1, q);
        if (q & 1) read_one(xa, xb, ks, 2, q >> 1);
        if (kEnergy) {
          if (q == 0) energy_read(ep, ks, 2);
          energy_acc(eq, q);
        }
      });
      mfma_step(xa, xb, [&](int q) {
        copy(2, q);
        if (q & 1) read_one(ya, yb, ks, 3, q >> 1);
        if (kEnergy) {
          if (q == 0) energy_read(eq, ks, 3);
          energy_acc(ep, q);
        }
      });
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): stores of ks+1, reads of ks done
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(ya, yb, [&](int q) {
        if (q & 1) read_one(xa, xb, ks + 1, 0, q >> 1);  // past the last stage: unused
        if (kEnergy) {
          if (q == 0) energy_read(ep, ks + 1, 0);
          energy_acc(eq, q);
        }
      });
    }
  };
  if (diag) main_loop(std::true_type{});
  else main_loop(std::false_type{});
  if (has_tail) {
    auto none = [](int) {};
    tail();
#pragma unroll
    for (int h = 0; h < 4; h += 2) {
      read_step(xa, xb, nfull, h);
      read_step(ya, yb, nfull, h + 1);
      mfma_step(xa, xb, none);
      mfma_step(ya, yb, none);
    }
    if (diag) energy_stage(nfull);
  }
  if (dst_slot) {
    // a later part: its sums go to the workspace slot, all 256 x 256 of
    // them (the folding kernel keeps the upper part inside the matrix)
    double *eslot = reinterpret_cast<double *>(dst_slot + kTile * kTile);
    if (diag) eslot[erow] = 2.0 * en;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = wn * 128 + j * 32 + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          dst_slot[r * kTile + c] = 2.f * acc[i][j][v];
        }
      }
    return;
  }
  if (diag && I0 + erow < d) hdiag[I0 + erow] += 2.0 * en;

  // Epilogue: H[i][j] += 2 * acc for i <= j inside the matrix.  32x32 MFMA
  // result layout: lane l, element v -> row 8*(v/4) + 4*(l/32) + v%4, col l%32.
  // One 32-row band of the sub-tile (64 values per lane) at a time: all its
  // loads are issued from clamped (valid) addresses before any store.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float hv[4][16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gc = min(J0 + wn * 128 + j * 32 + (lane & 31), d - 1);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t gr =
            min(I0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), d - 1);
        hv[j][v] = H[gr * d + gc];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gc = J0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t gr = I0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (gr <= gc && gc < d) H[gr * d + gc] = hv[j][v] + 2.f * acc[i][j][v];
      }
    }
  }
}

// Adds the workspace slots of the split tiles into H, parts in order (one
// workgroup per 16-row strip of a tail tile, four columns per thread; a
// diagonal tile's first strip also adds the parts' energies into hdiag).
__global__ void __launch_bounds__(256)
    syrk_fold_kernel(float *__restrict__ H, double *__restrict__ hdiag, int64_t d, int nt,
                     int ntiles, int parts, int xcd_cus, const float *__restrict__ slots) {
  const int gi = blockIdx.x >> 4, strip = blockIdx.x & 15;
  int x = 0, rest = gi;
  XcdRun run = xcd_run(0, ntiles, xcd_cus);
  while (rest >= run.tail && x < 7) {
    rest -= run.tail;
    run = xcd_run(++x, ntiles, xcd_cus);
  }
  int ti, tj;
  tile_coords(run.first + run.full + rest, nt, ti, tj);
  const int64_t I0 = int64_t(ti) * kTile, J0 = int64_t(tj) * kTile;
  const float *s0 = slots + int64_t(gi) * (parts - 1) * kSlotFloats;
  const bool vec = (d & 3) == 0;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int e = threadIdx.x + 256 * it;      // float4 chunk of the 16 x 256 strip
    const int r = strip * 16 + (e >> 6), c = (e & 63) * 4;
    const int64_t gr = I0 + r, gc = J0 + c;
    if (gr >= d) continue;
    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < parts - 1; ++p) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t *>(s0 + p * kSlotFloats + r * kTile + c);
      if (p == 0) sum = v;
      else sum += v;
    }
    float *h = H + gr * d + gc;
    if (vec && gr <= gc && gc + 3 < d) {
      *reinterpret_cast<f32x4_t *>(h) = *reinterpret_cast<const f32x4_t *>(h) + sum;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (gr <= gc + k && gc + k < d) h[k] += sum[k];
    }
  }
  if (ti == tj && strip == 0 && I0 + threadIdx.x < d) {
    double en = 0.0;
    for (int p = 0; p < parts - 1; ++p)
      en += reinterpret_cast<const double *>(s0 + p * kSlotFloats + kTile * kTile)[threadIdx.x];
    hdiag[I0 + threadIdx.x] += en;
  }
}

// fp32 inputs: plain LDS-tiled FMA SYRK on 64x64 upper tiles (fp32 products
// are not exact in bf16, so this path keeps fp32 operands end to end).
constexpr int kFT = 64;
__global__ void __launch_bounds__(256)
    syrk_f32_kernel(float *__restrict__ H, const float *__restrict__ X, int64_t d, int64_t n,
                    int64_t ld) {
  const int ti = blockIdx.y, tj = blockIdx.x;
  if (ti > tj) return;
  __shared__ float As[16][kFT + 1];
  __shared__ float Bs[16][kFT + 1];
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;  // 4x4 outputs per thread
  const int64_t I0 = int64_t(ti) * kFT, J0 = int64_t(tj) * kFT;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < n; k0 += 16) {
    for (int e = tid; e < kFT * 16; e += 256) {
      const int r = e / 16, k = e % 16;
      const int64_t gk = k0 + k;
      As[k][r] = (I0 + r < d && gk < n) ? X[(I0 + r) * ld + gk] : 0.f;
      Bs[k][r] = (J0 + r < d && gk < n) ? X[(J0 + r) * ld + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] += As[k][tr * 4 + a] * Bs[k][tc * 4 + b];
    __syncthreads();
  }
  for (int a = 0; a < 4; ++a)
    for (int b = 0; b < 4; ++b) {
      const int64_t gr = I0 + tr * 4 + a, gc = J0 + tc * 4 + b;
      if (gr <= gc && gc < d) H[gr * d + gc] += 2.f * acc[a][b];
    }
}

// hdiag[i] += 2 * sum_t x_it^2 in float64, one workgroup per feature row,
// fixed reduction order (deterministic).
template <typename T>
__device__ __forceinline__ double to_f64(T v);
template <>
__device__ __forceinline__ double to_f64<uint16_t>(uint16_t v) {
  return (double)__uint_as_float(uint32_t(v) << 16);
}
template <>
__device__ __forceinline__ double to_f64<float>(float v) {
  return (double)v;
}

template <typename T>
__global__ void __launch_bounds__(256)
    diag_energy_kernel(double *__restrict__ hdiag, const T *__restrict__ X, int64_t n, int64_t ld) {
  const int64_t row = blockIdx.x;
  const T *x = X + row * ld;
  double s = 0.0;
  for (int64_t t = threadIdx.x; t < n; t += 256) {
    const double v = to_f64<T>(x[t]);
    s = fma(v, v, s);
  }
  __shared__ double red[256];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) hdiag[row] += 2.0 * red[0];
}

}  // namespace

// How the bf16 SYRK's tiles are cut: `parts` token parts per tail tile (1 =
// no split), chosen to finish the last round soonest with the workspace at
// hand.  Cost model per XCD, in whole-tile times: full / cus rounds of whole
// tiles, then ceil(tail parts / cus) rounds of 1/parts of a tile, each
// round paying a fixed prologue/epilogue of about four 64-token stages.
struct SyrkPlan {
  int parts, xcd_cus, units, tail_total;
};

SyrkPlan plan_syrk(int ntiles, int cus, int64_t n, size_t ws_bytes, int max_parts) {
  SyrkPlan best{1, std::max(1, cus / 8), 0, 0};
  const int P = best.xcd_cus;
  XcdRun runs[8];
  for (int x = 0; x < 8; ++x) {
    runs[x] = xcd_run(x, ntiles, P);
    best.tail_total += runs[x].tail;
  }
  const double eps = 4.0 / std::max<int64_t>(n / kBK, 1) + 0.005;
  double best_score = 1e30;
  for (int parts = 1; parts <= max_parts; ++parts) {
    if (parts > 1 && (best.tail_total == 0 ||
                      size_t(best.tail_total) * (parts - 1) * kSlotBytes > ws_bytes))
      break;
    double score = 0.0;
    int units = 0;
    for (int x = 0; x < 8; ++x) {
      const int rounds = (runs[x].tail * parts + P - 1) / P;
      score = std::max(score, double(runs[x].full) / P * (1.0 + eps) +
                                  rounds * (1.0 / parts + eps));
      units = std::max(units, runs[x].full + runs[x].tail * parts);
    }
    if (score < best_score - 1e-9) {
      best_score = score;
      best.parts = parts;
      best.units = units;
    }
  }
  return best;
}

size_t hessian_ws_bytes(int64_t d) {
  const int nt = (int)cdiv(d, kTile);
  const SyrkPlan p = plan_syrk(nt * (nt + 1) / 2, device_cu_count(), int64_t(1) << 15,
                               ~size_t(0), 4);
  return align256(size_t(p.tail_total) * (p.parts - 1) * kSlotBytes);
}

gptq_status hessian_accumulate_impl(float *H, double *hdiag, int64_t d, const void *X,
                                    int x_dtype, int64_t n_tok, int64_t ld_x, void *ws,
                                    size_t ws_bytes, hipStream_t stream) {
  if (x_dtype == GPTQ_DT_BF16) {
    const uint16_t *Xb = static_cast<const uint16_t *>(X);
    const int nt = (int)cdiv(d, kTile);
    const int ntiles = nt * (nt + 1) / 2;
    const SyrkPlan p = plan_syrk(ntiles, device_cu_count(), n_tok, ws ? ws_bytes : 0, 16);
    float *slots = static_cast<float *>(ws);
    const size_t lds = size_t(kStages) * kStageBytes;
    GPTQ_TRY(allow_dynamic_lds((const void *)syrk_bf16_kernel, lds));
    // Off-diagonal tiles take the 16x16x32 path when every token part holds a
    // whole 64-token stage and the per-lane row offsets fit in 32 bits.
    const int tile16 = (n_tok / kBK >= p.parts && ld_x < (int64_t(1) << 26)) ? 1 : 0;
    GPTQ_TRY(launch("hessian_syrk_bf16", syrk_bf16_kernel, dim3(8 * p.units), dim3(kThreads), lds,
                    stream, H, hdiag, Xb, d, n_tok, ld_x, nt, ntiles, p.parts, p.xcd_cus, slots,
                    tile16));
    if (p.parts > 1)
      GPTQ_TRY(launch("hessian_fold", syrk_fold_kernel, dim3(16 * p.tail_total), dim3(256), 0,
                      stream, H, hdiag, d, nt, ntiles, p.parts, p.xcd_cus, (const float *)slots));
  } else {
    const float *Xf = static_cast<const float *>(X);
    const unsigned nt = (unsigned)cdiv(d, kFT);
    GPTQ_TRY(launch("hessian_syrk_f32", syrk_f32_kernel, dim3(nt, nt), dim3(256), 0, stream, H,
                    Xf, d, n_tok, ld_x));
    GPTQ_TRY(launch("hessian_diag", diag_energy_kernel<float>, dim3((unsigned)d), dim3(256), 0,
                    stream, hdiag, Xf, n_tok, ld_x));
  }
  return GPTQ_OK;
}

}  // namespace gptq
