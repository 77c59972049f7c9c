// W4A16 product: y = x W^T for a stored 4-bit affine layer, the weights
// rebuilt from their codes inside the product kernel.
//
// ("Hugging Face AutoGPTQ and Transformers Integration", section Mixed
// Precision Scheme: int4 weights with fp16 activations, dequantized on the
// fly in a fused kernel; "GPTQ", section Waskie gardla: in inference the
// cost is reading memory.)
//
// Layout written once by gptq_w4a16_prepare into the caller's buffer:
//  * kperm  kernel position -> original column.  Columns are sorted by group
//           (stable), so every group is a run of `group` consecutive kernel
//           positions and its scale multiplies a partial sum instead of each
//           weight.
//  * wq     codes in tiles of 16 rows x 128 kernel positions (1 KiB), tile
//           (rt, st) at index rt * ksteps + st.  Lane l = 16 kg + n of a wave
//           owns 16 bytes of a tile: row n, positions 32 t + 8 kg + e for the
//           MFMA sub-step t = 0..3 and e = 0..7, one 32-bit word per t, code e
//           at bit 16 (e & 1) + 4 (e >> 1).  A wave reads a tile as one
//           contiguous 1 KiB load.
//  * sc, zp per 16-row tile and group: 16 float scales and 16 zero nibbles.
//
// Exact dequantization in fp16.  OR-ing a code q into the mantissa of the
// fp16 number 1024 (0x6400) gives 1024 + q; a code in mantissa bits 4..7
// gives 1024 + 16 q.  One packed fp16 add of -(1024 + z), or a packed fma
// with 1/16 and -(64 + z), then yields q - z, an integer of at most 15 in
// magnitude and so exact.  The MFMA multiplies it by the fp16 activation
// (exact in fp32) and sums in fp32; the group's scale is applied to that sum.
#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>
#include <string>

#include "common.h"

namespace gptq {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kStep = 128;         // kernel positions per step (one load per lane)
constexpr int kMaxBatch = 64;      // rows of x per product launch
constexpr int kMaxNs = 8;          // steps per workgroup, at most (all loaded up front)
constexpr int kStageChunks = 16;   // 16-byte x chunks staged per thread, at most
constexpr int kNT = 2;             // 16-row tiles per wave

// status words at the start of the layer buffer
constexpr int kStatBadGroup = 1;   // g_idx out of range or a group of wrong size
constexpr int kStatPermuted = 2;   // kperm is not the identity

struct LayerMap {
  int32_t *status;
  int32_t *kperm;
  u4_t *wq;
  float *sc;
  uint32_t *zp;
  size_t bytes;
};

struct Geometry {
  int64_t rows, cols, rows_pad, k_pad, rt16, ksteps, ngroups, ngp;
  int32_t group;
};

Geometry geometry(int64_t rows, int64_t cols, int32_t group) {
  Geometry g;
  g.rows = rows;
  g.cols = cols;
  g.group = group;
  g.rows_pad = cdiv(rows, 16) * 16;
  g.k_pad = cdiv(cols, kStep) * kStep;
  g.rt16 = g.rows_pad / 16;
  g.ksteps = g.k_pad / kStep;
  g.ngroups = cols / group;
  g.ngp = g.k_pad / group;
  return g;
}

LayerMap layer_map(void *mem, const Geometry &g) {
  LayerMap m;
  char *p = static_cast<char *>(mem);
  size_t off = 0;
  auto take = [&](size_t n) {
    char *q = p ? p + off : nullptr;
    off += align256(n);
    return q;
  };
  m.status = reinterpret_cast<int32_t *>(take(256));
  m.kperm = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * g.k_pad));
  m.wq = reinterpret_cast<u4_t *>(take(size_t(g.rows_pad) * g.k_pad / 2));
  m.sc = reinterpret_cast<float *>(take(sizeof(float) * g.rt16 * g.ngp * 16));
  m.zp = reinterpret_cast<uint32_t *>(take(sizeof(uint32_t) * g.rt16 * g.ngp * 2));
  m.bytes = off;
  return m;
}

bool valid_group(int64_t cols, int32_t group) {
  if (group == 32 || group == 64) return cols % group == 0;
  return group >= kStep && group % kStep == 0 && cols % group == 0;
}

// ------------------------------------------------------------ prepare kernels
// Status words cleared, every kernel position marked empty (-1), so that
// positions a malformed g_idx leaves unclaimed never name a column.
__global__ void w4a16_init_kernel(int32_t *status, int32_t *kperm, int32_t k_pad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < 64) status[i] = 0;
  if (i < k_pad) kperm[i] = -1;
}

// One workgroup per group g: the columns with g_idx == g, in increasing
// order, go to kernel positions [g * group, (g + 1) * group).
__global__ __launch_bounds__(kThreads) void w4a16_kperm_kernel(
    const int32_t *__restrict__ g_idx, int32_t cols, int32_t group, int32_t ngroups,
    int32_t k_pad, int32_t *__restrict__ kperm, int32_t *__restrict__ status) {
  __shared__ int32_t wave_cnt[kWaves];
  const int g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t running = 0;
  int bad = 0, moved = 0;
  for (int base = 0; base < cols; base += kThreads) {
    const int c = base + tid;
    int gi = -1;
    if (c < cols) {
      gi = g_idx[c];
      if (g == 0 && (gi < 0 || gi >= ngroups)) bad = 1;
    }
    const bool hit = gi == g;
    const uint64_t mask = __ballot(hit);
    const int before = __popcll(mask & ((uint64_t(1) << lane) - 1));
    if (lane == 0) wave_cnt[wave] = __popcll(mask);
    __syncthreads();
    int off = running;
    for (int w = 0; w < wave; ++w) off += wave_cnt[w];
    int total = 0;
    for (int w = 0; w < kWaves; ++w) total += wave_cnt[w];
    if (hit) {
      const int rank = off + before;
      if (rank < group) {
        const int pos = g * group + rank;
        kperm[pos] = c;
        if (pos != c) moved = 1;
      }
    }
    running += total;
    __syncthreads();
  }
  if (running != group) bad = 1;
  if (g == 0)
    for (int k = cols + tid; k < k_pad; k += kThreads) kperm[k] = -1;
  bad = __any(bad);
  moved = __any(moved);
  if (lane == 0 && bad) atomicOr(status, kStatBadGroup);
  if (lane == 0 && moved) atomicOr(status, kStatPermuted);
}

// One thread per (16-row tile, step, lane): gathers the lane's 32 codes.
__global__ __launch_bounds__(kThreads) void w4a16_repack_kernel(
    const uint32_t *__restrict__ packed, int64_t rows, int64_t cols,
    const int32_t *__restrict__ kperm, int64_t ksteps, int64_t total,
    u4_t *__restrict__ wq) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const int lane = int(i & 63), n = lane & 15, kg = lane >> 4;
  const int64_t st = (i >> 6) % ksteps, rt = (i >> 6) / ksteps;
  const int64_t r = rt * 16 + n;
  const uint32_t *prow = packed + r * (cols / 8);
  u4_t out;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t k = st * kStep + 32 * t + 8 * kg + e;
      const int32_t c = kperm[k];
      uint32_t code = 0;
      if (r < rows && c >= 0 && c < cols) code = (prow[c >> 3] >> (4 * (c & 7))) & 15u;
      w |= code << (16 * (e & 1) + 4 * (e >> 1));
    }
    out[t] = w;
  }
  wq[i] = out;
}

// One thread per (16-row tile, group, row): scale, and for every 8th row the
// word of 8 zero nibbles.
__global__ __launch_bounds__(kThreads) void w4a16_scales_kernel(
    const float *__restrict__ scale, const uint32_t *__restrict__ zero_packed,
    int64_t rows, int64_t ngroups, int64_t ngp, int64_t total, float *__restrict__ sc,
    uint32_t *__restrict__ zp) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const int n = int(i & 15);
  const int64_t g = (i >> 4) % ngp, rt = (i >> 4) / ngp;
  const int64_t r = rt * 16 + n;
  sc[i] = (r < rows && g < ngroups) ? scale[r * ngroups + g] : 0.f;
  if ((n & 7) == 0) {
    uint32_t w = 0;
    for (int e = 0; e < 8; ++e) {
      const int64_t rr = r + e;
      uint32_t z = 0;
      if (rr < rows && g < ngroups) {
        const int64_t t = rr * ngroups + g;  // code index in the zero stream
        z = (zero_packed[t >> 3] >> (4 * (t & 7))) & 15u;
      }
      w |= z << (4 * e);
    }
    zp[((rt * ngp + g) << 1) + (n >> 3)] = w;
  }
}

// x_p[b][k] = x[b][kperm[k]] (0 on padding), 8 positions per thread.
__global__ __launch_bounds__(kThreads) void w4a16_gather_x_kernel(
    const uint16_t *__restrict__ x, int64_t cols, int64_t k_pad, int64_t total,
    const int32_t *__restrict__ kperm, uint16_t *__restrict__ xp) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const int64_t per_row = k_pad / 8;
  const int64_t b = i / per_row, k0 = (i - b * per_row) * 8;
  const uint16_t *xr = x + b * cols;
  uint32_t v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int32_t c0 = kperm[k0 + 2 * e], c1 = kperm[k0 + 2 * e + 1];
    const uint32_t lo = c0 >= 0 ? xr[c0] : 0u, hi = c1 >= 0 ? xr[c1] : 0u;
    v[e] = lo | (hi << 16);
  }
  u4_t o = {v[0], v[1], v[2], v[3]};
  *reinterpret_cast<u4_t *>(xp + b * k_pad + k0) = o;
}

// ------------------------------------------------------------ product kernel
struct W4Args {
  const u4_t *wq;
  const float *sc;
  const uint32_t *zp;
  const uint16_t *x;   // activations in kernel order, row stride ldx halves
  uint16_t *y;
  float *part;         // split-K partial sums: [split][batch][rows_pad]
  int64_t ldx, ldy;
  int32_t batch, cols, rows, rows_pad, rt16, ksteps, ngp, gsteps;
  int32_t splits, base, rem, ns_max;
};

// Masks and the fp16 1024.0 pair held in registers, so that each nibble
// extraction is one v_and_or_b32 (two literal operands cannot be encoded).
struct DqConst {
  uint32_t lo, hi, magic;
};

__device__ inline DqConst dq_const() {
  DqConst c;
  asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(c.lo));
  asm volatile("s_mov_b32 %0, 0x00f000f0" : "=s"(c.hi));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(c.magic));
  return c;
}

// B operand for one sub-step: the 8 codes of word w minus the zero point.
__device__ inline h8_t dequant8(uint32_t w, uint32_t nz1, uint32_t nz2, const DqConst &c) {
  const uint32_t w8 = w >> 8;
  const uint32_t h0 = (w & c.lo) | c.magic;
  const uint32_t h1 = (w & c.hi) | c.magic;
  const uint32_t h2 = (w8 & c.lo) | c.magic;
  const uint32_t h3 = (w8 & c.hi) | c.magic;
  const h2_t sixteenth = {_Float16(0.0625f), _Float16(0.0625f)};
  const h2_t z1 = __builtin_bit_cast(h2_t, nz1), z2 = __builtin_bit_cast(h2_t, nz2);
  const h2_t b01 = __builtin_bit_cast(h2_t, h0) + z1;
  const h2_t b23 = __builtin_elementwise_fma(__builtin_bit_cast(h2_t, h1), sixteenth, z2);
  const h2_t b45 = __builtin_bit_cast(h2_t, h2) + z1;
  const h2_t b67 = __builtin_elementwise_fma(__builtin_bit_cast(h2_t, h3), sixteenth, z2);
  return h8_t{b01[0], b01[1], b23[0], b23[1], b45[0], b45[1], b67[0], b67[1]};
}

// Grid: tiles x splits workgroups of 4 waves.  A workgroup owns 16 * kNT * 4
// rows and one range of steps, walked in chunks of at most ns_max steps; its
// waves take kNT 16-row tiles each and share each chunk's activations,
// staged in LDS.  MT 16-row slabs of x.  SPS scale units per step: 1 for
// group >= 128, 2 for group 64, 4 for group 32.  NS >= the steps of a chunk
// (2, 4 or 8).
template <int MT, int SPS, int NS>
__global__ __launch_bounds__(kThreads) void w4a16_gemm_kernel(W4Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int kSub = 4 / SPS;  // sub-steps per scale unit
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int tile = blockIdx.x / a.splits, split = blockIdx.x - tile * a.splits;
  const int kbeg = split * a.base + min(split, a.rem);  // this split's steps:
  const int nsplit = a.base + (split < a.rem ? 1 : 0);  //   [kbeg, kbeg + nsplit)
  const int rt0 = (tile * kWaves + wave) * kNT;
  const int row_h = a.ns_max * kStep + 8;  // LDS row stride in halves (+16 B)
  uint16_t *xs = reinterpret_cast<uint16_t *>(smem);

  u4_t wb[NS][kNT];
  float sb[NS][kNT][SPS];
  uint32_t zb[NS][kNT][SPS];
  auto issue = [&](int slot, int st) {
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const int64_t rt = min(rt0 + j, a.rt16 - 1);
      wb[slot][j] = a.wq[(rt * a.ksteps + st) * 64 + lane];
#pragma unroll
      for (int u = 0; u < SPS; ++u) {
        const int64_t g = SPS == 1 ? st / a.gsteps : int64_t(st) * SPS + u;
        sb[slot][j][u] = a.sc[(rt * a.ngp + g) * 16 + n];
        zb[slot][j][u] = a.zp[(rt * a.ngp + g) * 2 + (n >> 3)];
      }
    }
  };

  f4_t yacc[MT][kNT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < kNT; ++j) yacc[m][j] = f4_t{0.f, 0.f, 0.f, 0.f};

  const uint16_t *xa = xs + n * row_h + 8 * kg;  // lane's A row (m = n) and k offset
  const DqConst dq = dq_const();

  // The split's steps are walked in chunks of at most a.ns_max (<= NS):
  // each chunk stages its x in LDS and issues all of its weights at once.
  for (int c = 0; c < nsplit; c += a.ns_max) {
    const int k0 = kbeg + c;
    const int ns = min(a.ns_max, nsplit - c);
    if (c > 0) __syncthreads();  // every wave is done with the previous chunk's x

    // ---- stage this chunk of x (rows >= batch and columns >= cols are zero)
    {
      constexpr int kChunks = MT * NS;   // >= 16 MT rows x (16 ns) chunks / 256 threads
      const int cpr = ns * (kStep / 8);  // 16-byte chunks per row, 16..128
      const int db = kThreads / cpr, dc = kThreads - db * cpr;
      int b0 = tid / cpr, c0 = tid - b0 * cpr;
      int bs[kChunks], cs[kChunks];
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        bs[i] = b0;
        cs[i] = c0;
        b0 += db;
        c0 += dc;
        if (c0 >= cpr) {
          c0 -= cpr;
          ++b0;
        }
      }
      u4_t stg[kChunks];
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        const int col = k0 * kStep + cs[i] * 8;
        stg[i] = u4_t{0, 0, 0, 0};
        if (bs[i] < a.batch && col < a.cols)
          stg[i] = *reinterpret_cast<const u4_t *>(a.x + bs[i] * a.ldx + col);
      }
      // weights, scales and zeros of every step of the chunk, after x: loads
      // complete in order, so x can be stored to LDS while the weights are
      // still on their way (slots past the chunk repeat its last step: same
      // cache lines, no branch, so the loads in flight are counted exactly)
#pragma unroll
      for (int p = 0; p < NS; ++p) issue(p, k0 + min(p, ns - 1));
#pragma unroll
      for (int i = 0; i < kChunks; ++i)
        if (bs[i] < 16 * MT) *reinterpret_cast<u4_t *>(xs + bs[i] * row_h + cs[i] * 8) = stg[i];
    }
    __syncthreads();

    // One step: 4 MFMA sub-steps per slab and tile; the scale of each unit
    // is applied to the unit's fp32 sum.
    auto step = [&](const int p) {
      const int s = p;
      f4_t acc[MT][kNT];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        h8_t A[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
          A[m] = *reinterpret_cast<const h8_t *>(xa + m * 16 * row_h + s * kStep + 32 * t);
        const int u = t / kSub;
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
          const uint32_t z = (zb[p][j][u] >> (4 * (n & 7))) & 15u;
          const uint32_t nz1 = (0xE400u | z) * 0x00010001u;
          const uint32_t nz2 = (0xD400u | (z << 4)) * 0x00010001u;
          const h8_t B = dequant8(wb[p][j][t], nz1, nz2, dq);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const f4_t c0 = (t % kSub == 0) ? f4_t{0.f, 0.f, 0.f, 0.f} : acc[m][j];
            acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[m], B, c0, 0, 0, 0);
          }
          if (t % kSub == kSub - 1) {
            const float sc = sb[p][j][u];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
              for (int i = 0; i < 4; ++i) yacc[m][j][i] = fmaf(sc, acc[m][j][i], yacc[m][j][i]);
          }
        }
      }
    };
#pragma unroll
    for (int p = 0; p < NS; ++p)
      if (p < ns) step(p);
  }

  // ---- output.  Lane holds C[m = 4 kg + i][n] of each 16 x 16 block.
  if (a.splits == 1) {
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const int r = (rt0 + j) * 16 + n;
      if (rt0 + j >= a.rt16 || r >= a.rows) continue;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = m * 16 + 4 * kg + i;
          if (b < a.batch)
            a.y[b * a.ldy + r] = __builtin_bit_cast(uint16_t, _Float16(yacc[m][j][i]));
        }
    }
    return;
  }
  float *mine = a.part + int64_t(split) * a.batch * a.rows_pad;
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    if (rt0 + j >= a.rt16) continue;
    const int r = (rt0 + j) * 16 + n;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = m * 16 + 4 * kg + i;
        if (b < a.batch) mine[int64_t(b) * a.rows_pad + r] = yacc[m][j][i];
      }
  }
}


// The same product for splits of many chunks: two chunks of x in LDS and two
// sets of weights in registers.  While chunk c is multiplied, chunk c+1's x
// waits in registers (loaded during chunk c-1) and goes to the other LDS
// buffer after the multiplication; then chunk c+2's x is loaded and its
// weights are issued into the set just freed.  ns_max is a power of two, at
// most 4 steps (2 from three 16-row slabs of x up), so that two workgroups
// fit a CU.
template <int MT, int SPS, int NS>
__global__ __launch_bounds__(kThreads) void w4a16_gemm_pipe_kernel(W4Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int kSub = 4 / SPS;  // sub-steps per scale unit
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int tile = blockIdx.x / a.splits, split = blockIdx.x - tile * a.splits;
  const int kbeg = split * a.base + min(split, a.rem);  // this split's steps:
  const int nsplit = a.base + (split < a.rem ? 1 : 0);  //   [kbeg, kbeg + nsplit)
  const int rt0 = (tile * kWaves + wave) * kNT;
  const int row_h = a.ns_max * kStep + 8;  // LDS row stride in halves (+16 B)
  const int buf_h = 16 * MT * row_h;        // halves per staged chunk of x
  uint16_t *xs = reinterpret_cast<uint16_t *>(smem);

  u4_t wb[2][NS][kNT];
  float sb[2][NS][kNT][SPS];
  uint32_t zb[2][NS][kNT][SPS];
  auto issue = [&](int set, int slot, int st) {
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const int64_t rt = min(rt0 + j, a.rt16 - 1);
      wb[set][slot][j] = a.wq[(rt * a.ksteps + st) * 64 + lane];
#pragma unroll
      for (int u = 0; u < SPS; ++u) {
        const int64_t g = SPS == 1 ? st / a.gsteps : int64_t(st) * SPS + u;
        sb[set][slot][j][u] = a.sc[(rt * a.ngp + g) * 16 + n];
        zb[set][slot][j][u] = a.zp[(rt * a.ngp + g) * 2 + (n >> 3)];
      }
    }
  };

  f4_t yacc[MT][kNT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < kNT; ++j) yacc[m][j] = f4_t{0.f, 0.f, 0.f, 0.f};

  const DqConst dq = dq_const();

  // This thread's 16-byte pieces of a staged chunk of x: piece i is row
  // b0 + i db, piece c0 of the row's cpr = 16 ns_max pieces (ns_max is a
  // power of two, so cpr divides the 256 threads).
  constexpr int kChunks = MT * NS;   // >= 16 MT rows x cpr pieces / 256 threads
  const int cpr = a.ns_max * (kStep / 8);
  const int lg = __builtin_ctz(cpr);
  const int b0 = tid >> lg, c0 = tid & (cpr - 1), db = kThreads >> lg;
  // Chunk c of the split: steps [kbeg + c ns_max, ...) (rows >= batch and
  // columns >= cols are zero; a chunk past the split loads nothing).
  const int nchunks = (nsplit + a.ns_max - 1) / a.ns_max;
  u4_t stg[kChunks];
  auto x_load = [&](int c) {
    const int col = (kbeg + c * a.ns_max) * kStep + c0 * 8;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int b = b0 + i * db;
      stg[i] = u4_t{0, 0, 0, 0};
      if (c < nchunks && b < a.batch && col < a.cols)
        stg[i] = *reinterpret_cast<const u4_t *>(a.x + b * a.ldx + col);
    }
  };
  auto x_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int b = b0 + i * db;
      if (b < 16 * MT) *reinterpret_cast<u4_t *>(xs + buf * buf_h + b * row_h + c0 * 8) = stg[i];
    }
  };
  // the weights of chunk c (slots past its steps repeat its last step, or the
  // split's last step past the split: same cache lines)
  auto w_issue = [&](int set, int c) {
    const int k0 = kbeg + c * a.ns_max;
    const int last = kbeg + nsplit - 1;
#pragma unroll
    for (int p = 0; p < NS; ++p) issue(set, p, min(k0 + min(p, a.ns_max - 1), last));
  };

  // One step of chunk buffer `buf` with weight set `set`: 4 MFMA sub-steps
  // per slab and tile; the scale of each unit is applied to its fp32 sum.
  auto step = [&](auto settag, int buf, const int p) {
    constexpr int set = decltype(settag)::value;
    const uint16_t *xa = xs + buf * buf_h + n * row_h + 8 * kg;  // lane's A row and k offset
    f4_t acc[MT][kNT];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      h8_t A[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m)
        A[m] = *reinterpret_cast<const h8_t *>(xa + m * 16 * row_h + p * kStep + 32 * t);
      const int u = t / kSub;
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const uint32_t z = (zb[set][p][j][u] >> (4 * (n & 7))) & 15u;
        const uint32_t nz1 = (0xE400u | z) * 0x00010001u;
        const uint32_t nz2 = (0xD400u | (z << 4)) * 0x00010001u;
        const h8_t B = dequant8(wb[set][p][j][t], nz1, nz2, dq);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const f4_t c0 = (t % kSub == 0) ? f4_t{0.f, 0.f, 0.f, 0.f} : acc[m][j];
          acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[m], B, c0, 0, 0, 0);
        }
        if (t % kSub == kSub - 1) {
          const float sc = sb[set][p][j][u];
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) yacc[m][j][i] = fmaf(sc, acc[m][j][i], yacc[m][j][i]);
        }
      }
    }
  };
  // Chunk c: multiply buffer c % 2 with weight set c % 2; meanwhile chunk
  // c+1's x waits in registers (loaded during chunk c-1) and is stored to
  // the other buffer after the multiplication, chunk c+2's x is loaded and
  // its weights are issued into the freed set.  The barrier at the end of a
  // chunk orders the other buffer's stores before its reads, and this
  // buffer's reads before its next stores.
  auto chunk = [&](auto settag, int c) {
    constexpr int set = decltype(settag)::value;
    const int ns = min(a.ns_max, nsplit - c * a.ns_max);
#pragma unroll
    for (int p = 0; p < NS; ++p)
      if (p < ns) step(settag, set, p);
    x_store(set ^ 1);
    x_load(c + 2);
    w_issue(set, c + 2);
    __syncthreads();
  };
  x_load(0);
  w_issue(0, 0);
  x_store(0);
  x_load(1);
  w_issue(1, 1);
  __syncthreads();
  for (int c = 0; c < nchunks; c += 2) {
    chunk(std::integral_constant<int, 0>{}, c);
    if (c + 1 < nchunks) chunk(std::integral_constant<int, 1>{}, c + 1);
  }

  // ---- output.  Lane holds C[m = 4 kg + i][n] of each 16 x 16 block.
  if (a.splits == 1) {
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const int r = (rt0 + j) * 16 + n;
      if (rt0 + j >= a.rt16 || r >= a.rows) continue;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = m * 16 + 4 * kg + i;
          if (b < a.batch)
            a.y[b * a.ldy + r] = __builtin_bit_cast(uint16_t, _Float16(yacc[m][j][i]));
        }
    }
    return;
  }
  float *mine = a.part + int64_t(split) * a.batch * a.rows_pad;
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    if (rt0 + j >= a.rt16) continue;
    const int r = (rt0 + j) * 16 + n;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = m * 16 + 4 * kg + i;
        if (b < a.batch) mine[int64_t(b) * a.rows_pad + r] = yacc[m][j][i];
      }
  }
}


// Split-K partials -> y: one thread per output, splits summed in split order.
__global__ __launch_bounds__(kThreads) void w4a16_reduce_kernel(
    const float *__restrict__ part, int32_t splits, int32_t batch, int32_t rows,
    int32_t rows_pad, uint16_t *__restrict__ y, int64_t ldy) {
  const int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= int64_t(batch) * rows) return;
  const int b = int(e / rows), r = int(e - int64_t(b) * rows);
  const float *p = part + int64_t(b) * rows_pad + r;
  const int64_t sstride = int64_t(batch) * rows_pad;
  constexpr int kLoads = 8;   // partials in flight per thread, at most
  float sum = 0.f;
  for (int s0 = 0; s0 < splits; s0 += kLoads) {
    // (s0 + i < splits is the same for every thread: no load past the splits)
    float v[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      v[i] = 0.f;
      if (s0 + i < splits) v[i] = p[int64_t(s0 + i) * sstride];
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      if (s0 + i < splits) sum += v[i];
  }
  y[b * ldy + r] = __builtin_bit_cast(uint16_t, _Float16(sum));
}

// Small batches: one workgroup of W waves per 16-row tile over all of K, so
// no workgroup waits for another.  The `batch` rows of x (kernel order) are
// staged in LDS; wave w takes the steps w, w + W, ... with all of its weights
// loaded up front, and the waves' 16 x 16 partial products are summed through
// LDS in wave order.  NSW >= the steps of any wave.  Layers with many row
// tiles use small workgroups (4 waves), so that several workgroups per CU
// have their loads in flight while others compute.
template <int SPS, int NSW>
struct RowTile {
  u4_t w[NSW];
  float s[NSW][SPS];
  uint32_t z[NSW][SPS];
};

template <int SPS, int NSW>
__global__ __launch_bounds__(NSW > 8 ? 512 : 1024) void w4a16_rows_kernel(W4Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int kSub = 4 / SPS;
  constexpr int kXChunks = 8;   // 16-byte x chunks staged per thread, at most
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x, W = nthr >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int row_h = a.ksteps * kStep + 8;   // LDS row stride in halves (+16 B)
  const int ns = (a.ksteps - wave + W - 1) / W;
  uint16_t *xs = reinterpret_cast<uint16_t *>(smem);
  float *red = reinterpret_cast<float *>(smem + size_t(a.batch) * row_h * 2);

  auto issue = [&](RowTile<SPS, NSW> &T, int rt) {
#pragma unroll
    for (int p = 0; p < NSW; ++p) {
      const int st = wave + min(p, ns - 1) * W;
      T.w[p] = a.wq[(int64_t(rt) * a.ksteps + st) * 64 + lane];
#pragma unroll
      for (int u = 0; u < SPS; ++u) {
        const int64_t g = SPS == 1 ? st / a.gsteps : int64_t(st) * SPS + u;
        T.s[p][u] = a.sc[(int64_t(rt) * a.ngp + g) * 16 + n];
        T.z[p][u] = a.zp[(int64_t(rt) * a.ngp + g) * 2 + (n >> 3)];
      }
    }
  };

  RowTile<SPS, NSW> TA;
  const int rt = blockIdx.x;

  // ---- x (issued first: loads complete in order), then the first tile
  {
    const int cpr = a.ksteps * (kStep / 8);   // 16-byte chunks per row
    const int db = nthr / cpr, dc = nthr - db * cpr;
    int b0 = tid / cpr, c0 = tid - b0 * cpr;
    int bs[kXChunks], cs[kXChunks];
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) {
      bs[i] = b0;
      cs[i] = c0;
      b0 += db;
      c0 += dc;
      if (c0 >= cpr) {
        c0 -= cpr;
        ++b0;
      }
    }
    u4_t stg[kXChunks];
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) {
      stg[i] = u4_t{0, 0, 0, 0};
      if (bs[i] < a.batch && cs[i] * 8 < a.cols)
        stg[i] = *reinterpret_cast<const u4_t *>(a.x + bs[i] * a.ldx + cs[i] * 8);
    }
    issue(TA, rt);
#pragma unroll
    for (int i = 0; i < kXChunks; ++i)
      if (bs[i] < a.batch) *reinterpret_cast<u4_t *>(xs + bs[i] * row_h + cs[i] * 8) = stg[i];
  }
  __syncthreads();

  // Lane's A row m = n.  Rows m >= batch of C are never stored and depend only
  // on row m of A, so those lanes read row batch - 1 instead of zeros.
  const uint16_t *xa = xs + min(n, a.batch - 1) * row_h + 8 * kg;
  const DqConst dq = dq_const();
  auto tile = [&](const RowTile<SPS, NSW> &T, const int rtile) {
    f4_t yacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NSW; ++p) {
      if (p >= ns) break;
      const int st = wave + p * W;
      f4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const h8_t A = *reinterpret_cast<const h8_t *>(xa + st * kStep + 32 * t);
        const int u = t / kSub;
        const uint32_t z = (T.z[p][u] >> (4 * (n & 7))) & 15u;
        const uint32_t nz1 = (0xE400u | z) * 0x00010001u;
        const uint32_t nz2 = (0xD400u | (z << 4)) * 0x00010001u;
        const h8_t B = dequant8(T.w[p][t], nz1, nz2, dq);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            A, B, (t % kSub == 0) ? f4_t{0.f, 0.f, 0.f, 0.f} : acc, 0, 0, 0);
        if (t % kSub == kSub - 1) {
          const float sc = T.s[p][u];
#pragma unroll
          for (int i = 0; i < 4; ++i) yacc[i] = fmaf(sc, acc[i], yacc[i]);
        }
      }
    }
    // sum the waves' partial products in wave order
    *reinterpret_cast<f4_t *>(red + (wave * 64 + lane) * 4) = yacc;
    __syncthreads();
    for (int e = tid; e < 256; e += nthr) {   // 16 x 16 outputs; W may be below 4
      const int l = e >> 2, i = e & 3;
      float sum = 0.f;
      for (int w = 0; w < W; ++w) sum += red[(w * 64 + l) * 4 + i];
      const int b = 4 * (l >> 4) + i, r = rtile * 16 + (l & 15);
      if (b < a.batch && r < a.rows)
        a.y[b * a.ldy + r] = __builtin_bit_cast(uint16_t, _Float16(sum));
    }
    __syncthreads();
  };

  tile(TA, rt);
}

// ------------------------------------------------------------ launch plan
int cu_count() { return device_cu_count(); }

constexpr size_t kRowsLdsMax = 144 * 1024;   // LDS of the rows kernel, at most
constexpr int kRowsMaxBatch = 16;

// Rows kernel (no split of K across workgroups): waves per workgroup and the
// static bound on steps per wave, or waves = 0 when the batch does not fit.
struct RowsPlan {
  int waves, nsw;
  size_t lds;
};

RowsPlan rows_plan(const Geometry &g, int bc, int cus) {
  RowsPlan r{0, 0, 0};
  const size_t xbytes = size_t(bc) * (g.ksteps * kStep + 8) * 2;
  if (bc > kRowsMaxBatch || xbytes + 16 * 1024 > kRowsLdsMax) return r;
  // steps a wave holds in registers: 16 (workgroups of at most 8 waves), 8
  // (128 VGPRs), fewer with more scales per step
  const int64_t max_ns = g.group == 32 ? 4 : g.group == 64 ? 8 : 16;
  // many row tiles: small workgroups, several resident per CU; few: all 16
  // waves of a CU on one tile
  int w = g.rt16 >= 2 * cus ? 4 : 16;
  while (w < 16 && (cdiv(g.ksteps, w) > max_ns || int64_t(bc) * g.k_pad > int64_t(4096) * w))
    w *= 2;
  w = int(std::min<int64_t>(w, g.ksteps));
  const int64_t ns = cdiv(g.ksteps, w);
  if (ns > max_ns || int64_t(bc) * g.k_pad > int64_t(4096) * w) return r;
  if (ns > 8 && w > 8) return r;   // 16 steps per wave: at most 512 threads
  r.waves = w;
  r.nsw = ns <= 2 ? 2 : ns <= 4 ? 4 : ns <= 8 ? 8 : 16;
  r.lds = xbytes + size_t(w) * 64 * 16;   // x, then the cross-wave sums
  return r;
}

// Split kernel: workgroups of 4 waves over 128 rows and a range of steps.
struct W4Plan {
  int mt, ns_t, tiles, splits, base, rem, ns_max;
  size_t lds;
};

W4Plan plan_for(const Geometry &g, int bc, int cus) {
  W4Plan p;
  p.mt = (bc + 15) / 16;
  p.tiles = int(cdiv(g.rt16, kWaves * kNT));
  const int ns_cap = std::min(kMaxNs, kStageChunks / p.mt);  // steps per staged chunk
  // About two workgroups per CU, in one round: a split walks its steps in
  // chunks of ns_cap, so the split count is free of the staging capacity
  // (fewer splits, fewer partial sums written and read back).
  p.splits = int(std::min<int64_t>(g.ksteps, std::max(1, 2 * cus / p.tiles)));
  p.base = int(g.ksteps / p.splits);
  p.rem = int(g.ksteps % p.splits);
  p.ns_max = std::min(p.base + (p.rem ? 1 : 0), ns_cap);
  p.ns_t = p.ns_max <= 2 ? 2 : p.ns_max <= 4 ? 4 : 8;
  p.lds = size_t(16) * p.mt * (size_t(p.ns_max) * kStep + 8) * 2;
  return p;
}

// Pipelined kernel: the same tiles and splits, chunks of a power of two
// steps (at most 4; 2 from three slabs up, and for groups below 128 from two
// slabs down), two of them staged.  Taken when the plain kernel would walk
// three or more chunks per split.
W4Plan plan_pipe(const Geometry &g, int bc, int cus) {
  W4Plan p = plan_for(g, bc, cus);
  int ns_cap = std::min(kMaxNs / 2, kStageChunks / 2 / p.mt);
  if (g.group < kStep && p.mt <= 2) ns_cap = std::min(ns_cap, 2);
  p.ns_max = std::min(p.base + (p.rem ? 1 : 0), ns_cap);
  while (p.ns_max & (p.ns_max - 1)) p.ns_max &= p.ns_max - 1;   // a power of two
  p.ns_t = p.ns_max <= 2 ? 2 : 4;
  p.lds = 2 * size_t(16) * p.mt * (size_t(p.ns_max) * kStep + 8) * 2;
  return p;
}

bool use_pipe(const W4Plan &p) {
  const int steps = p.base + (p.rem ? 1 : 0);
  return (steps + p.ns_max - 1) / p.ns_max >= 3;
}

size_t partial_bytes(const Geometry &g, int bc, int cus) {
  if (rows_plan(g, bc, cus).waves) return 0;
  const W4Plan p = plan_for(g, bc, cus);
  return p.splits > 1 ? align256(sizeof(float) * p.splits * bc * g.rows_pad) : 0;
}

size_t ws_bytes_for(const Geometry &g, bool permuted, int64_t batch, int cus) {
  const int full = int(std::min<int64_t>(batch, kMaxBatch));
  const int tail = int(batch % kMaxBatch);
  size_t part = partial_bytes(g, full, cus);
  if (batch > kMaxBatch && tail) part = std::max(part, partial_bytes(g, tail, cus));
  const size_t xp = permuted ? align256(sizeof(uint16_t) * full * g.k_pad) : 0;
  return xp + part;
}

template <int MT, int SPS, int NS>
gptq_status launch_gemm(const W4Args &a, const W4Plan &p, hipStream_t stream) {
  auto kern = w4a16_gemm_kernel<MT, SPS, NS>;
  GPTQ_TRY(allow_dynamic_lds(reinterpret_cast<const void *>(kern), 96 * 1024));
  return launch("w4a16_gemm", kern, dim3(p.tiles * p.splits), dim3(kThreads), p.lds, stream, a);
}

template <int MT, int SPS>
gptq_status launch_gemm_ns(const W4Args &a, const W4Plan &p, hipStream_t stream) {
  switch (p.ns_t) {
    case 2: return launch_gemm<MT, SPS, 2>(a, p, stream);
    case 4: return launch_gemm<MT, SPS, 4>(a, p, stream);
    default: return launch_gemm<MT, SPS, 8>(a, p, stream);
  }
}

template <int MT>
gptq_status launch_gemm_sps(const W4Args &a, const W4Plan &p, int sps, hipStream_t stream) {
  switch (sps) {
    case 1: return launch_gemm_ns<MT, 1>(a, p, stream);
    case 2: return launch_gemm_ns<MT, 2>(a, p, stream);
    default: return launch_gemm_ns<MT, 4>(a, p, stream);
  }
}

template <int MT, int SPS, int NS>
gptq_status launch_pipe(const W4Args &a, const W4Plan &p, hipStream_t stream) {
  auto kern = w4a16_gemm_pipe_kernel<MT, SPS, NS>;
  GPTQ_TRY(allow_dynamic_lds(reinterpret_cast<const void *>(kern), 96 * 1024));
  return launch("w4a16_gemm", kern, dim3(p.tiles * p.splits), dim3(kThreads), p.lds, stream, a);
}

template <int MT>
gptq_status launch_pipe_sps(const W4Args &a, const W4Plan &p, int sps, hipStream_t stream) {
  const bool n2 = p.ns_t == 2;
  switch (sps) {
    case 1: return n2 ? launch_pipe<MT, 1, 2>(a, p, stream) : launch_pipe<MT, 1, 4>(a, p, stream);
    case 2: return n2 ? launch_pipe<MT, 2, 2>(a, p, stream) : launch_pipe<MT, 2, 4>(a, p, stream);
    default: return n2 ? launch_pipe<MT, 4, 2>(a, p, stream) : launch_pipe<MT, 4, 4>(a, p, stream);
  }
}

template <int SPS, int NSW>
gptq_status launch_rows(const W4Args &a, const RowsPlan &r, hipStream_t stream) {
  auto kern = w4a16_rows_kernel<SPS, NSW>;
  GPTQ_TRY(allow_dynamic_lds(reinterpret_cast<const void *>(kern), kRowsLdsMax));
  return launch("w4a16_gemm", kern, dim3(a.rt16), dim3(64 * r.waves), r.lds, stream, a);
}

// Steps per wave: up to 16 with one scale per step, 8 with two, 4 with four.
template <int SPS>
gptq_status launch_rows_ns(const W4Args &a, const RowsPlan &r, hipStream_t stream) {
  constexpr int k8 = SPS == 4 ? 4 : 8, k16 = SPS == 1 ? 16 : k8;
  switch (r.nsw) {
    case 2: return launch_rows<SPS, 2>(a, r, stream);
    case 4: return launch_rows<SPS, 4>(a, r, stream);
    case 8: return launch_rows<SPS, k8>(a, r, stream);
    default: return launch_rows<SPS, k16>(a, r, stream);
  }
}

gptq_status launch_rows_sps(const W4Args &a, const RowsPlan &r, int sps, hipStream_t stream) {
  switch (sps) {
    case 1: return launch_rows_ns<1>(a, r, stream);
    case 2: return launch_rows_ns<2>(a, r, stream);
    default: return launch_rows_ns<4>(a, r, stream);
  }
}

// ------------------------------------------------- no-allocation product
// Scratch memory of gptq_w4a16_gemm_noalloc: a static device array, one copy
// per GPU the library runs on, held until the process ends.  Its host-side
// name is only a handle: kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept.
constexpr size_t kScratchBytes = GPTQ_W4A16_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void *> g_scratch_ptr;   // device -> address of its `scratch`

gptq_status scratch_address(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(GPTQ_ERR_DEVICE, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return GPTQ_OK;
  }
  void *ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr)
    return fail(GPTQ_ERR_DEVICE, std::string("cannot locate the static scratch on device ") +
                                     std::to_string(dev) + ": " + hipGetErrorString(e));
  g_scratch_ptr[dev] = ptr;
  *out = ptr;
  return GPTQ_OK;
}

// Argument checks shared by both products (host only, before any launch).
gptq_status check_gemm_args(const gptq_w4a16_layer *layer, const uint16_t *x, int64_t batch,
                            const uint16_t *y) {
  if (!layer || !layer->mem) return fail(GPTQ_ERR_INVALID_ARG, "layer is not prepared");
  if (batch < 1 || batch > 4096) return fail(GPTQ_ERR_INVALID_ARG, "batch must be in [1, 4096]");
  if (!x || !y) return fail(GPTQ_ERR_INVALID_ARG, "x and y must not be NULL");
  if (reinterpret_cast<uintptr_t>(x) % 16)
    return fail(GPTQ_ERR_INVALID_ARG, "x must be 16-byte aligned");
  if (!valid_group(layer->cols, layer->group) || layer->rows < 1)
    return fail(GPTQ_ERR_INVALID_ARG, "layer is not prepared");
  return GPTQ_OK;
}

// The product's launches, arguments already checked and `ws` large enough.
gptq_status gemm_launches(const gptq_w4a16_layer *layer, const uint16_t *x, int64_t batch,
                          uint16_t *y, void *ws, hipStream_t s) {
  const Geometry g = geometry(layer->rows, layer->cols, layer->group);
  const LayerMap m = layer_map(layer->mem, g);
  const int cus = cu_count();
  uint16_t *xp = layer->permuted ? static_cast<uint16_t *>(ws) : nullptr;
  float *part = reinterpret_cast<float *>(
      static_cast<char *>(ws) +
      (layer->permuted ? align256(sizeof(uint16_t) * std::min<int64_t>(batch, kMaxBatch) * g.k_pad)
                       : 0));
  const int sps = g.group >= kStep ? 1 : kStep / g.group;
  for (int64_t b0 = 0; b0 < batch; b0 += kMaxBatch) {
    const int bc = int(std::min<int64_t>(kMaxBatch, batch - b0));
    W4Args a;
    a.x = x + b0 * g.cols;
    a.ldx = g.cols;
    if (layer->permuted) {
      const int64_t total = int64_t(bc) * g.k_pad / 8;
      GPTQ_TRY(launch("w4a16_gather_x", w4a16_gather_x_kernel, dim3(cdiv(total, kThreads)),
                      dim3(kThreads), 0, s, a.x, g.cols, g.k_pad, total,
                      (const int32_t *)m.kperm, xp));
      a.x = xp;
      a.ldx = g.k_pad;
    }
    a.wq = m.wq;
    a.sc = m.sc;
    a.zp = m.zp;
    a.y = y + b0 * g.rows;
    a.part = part;
    a.ldy = g.rows;
    a.batch = bc;
    a.cols = int32_t(g.cols);
    a.rows = int32_t(g.rows);
    a.rows_pad = int32_t(g.rows_pad);
    a.rt16 = int32_t(g.rt16);
    a.ksteps = int32_t(g.ksteps);
    a.ngp = int32_t(g.ngp);
    a.gsteps = g.group >= kStep ? g.group / kStep : 1;
    const RowsPlan rp = rows_plan(g, bc, cus);
    if (rp.waves) {
      a.splits = 1;
      a.base = a.rem = a.ns_max = 0;
      GPTQ_TRY(launch_rows_sps(a, rp, sps, s));
      continue;
    }
    W4Plan p = plan_for(g, bc, cus);
    const bool pipe = use_pipe(p);
    if (pipe) p = plan_pipe(g, bc, cus);
    a.splits = p.splits;
    a.base = p.base;
    a.rem = p.rem;
    a.ns_max = p.ns_max;
    switch (p.mt) {
      case 1: GPTQ_TRY(pipe ? launch_pipe_sps<1>(a, p, sps, s) : launch_gemm_sps<1>(a, p, sps, s)); break;
      case 2: GPTQ_TRY(pipe ? launch_pipe_sps<2>(a, p, sps, s) : launch_gemm_sps<2>(a, p, sps, s)); break;
      case 3: GPTQ_TRY(pipe ? launch_pipe_sps<3>(a, p, sps, s) : launch_gemm_sps<3>(a, p, sps, s)); break;
      default: GPTQ_TRY(pipe ? launch_pipe_sps<4>(a, p, sps, s) : launch_gemm_sps<4>(a, p, sps, s)); break;
    }
    if (p.splits > 1) {
      const int64_t total = int64_t(bc) * g.rows;
      GPTQ_TRY(launch("w4a16_reduce", w4a16_reduce_kernel, dim3(cdiv(total, kThreads)),
                      dim3(kThreads), 0, s, (const float *)part, int32_t(p.splits), int32_t(bc),
                      int32_t(g.rows), int32_t(g.rows_pad), a.y, int64_t(g.rows)));
    }
  }
  return GPTQ_OK;
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" {

size_t gptq_w4a16_layer_bytes(int64_t rows, int64_t cols, int32_t group) {
  if (rows < 1 || rows > (int64_t(1) << 24) || cols < 32 || cols > (int64_t(1) << 20) ||
      !valid_group(cols, group))
    return 0;
  return layer_map(nullptr, geometry(rows, cols, group)).bytes;
}

gptq_status gptq_w4a16_prepare(const uint32_t *packed, const int32_t *g_idx,
                               const float *scale, const uint32_t *zero_packed,
                               int64_t rows, int64_t cols, int32_t group, void *mem,
                               size_t mem_bytes, gptq_w4a16_layer *layer, void *stream) {
  if (rows < 1 || rows > (int64_t(1) << 24) || cols < 32 || cols > (int64_t(1) << 20))
    return fail(GPTQ_ERR_INVALID_ARG, "rows and cols must be in [1, 2^24] x [32, 2^20]");
  if (!valid_group(cols, group))
    return fail(GPTQ_ERR_INVALID_ARG,
                "group must be 32, 64 or a multiple of 128, and divide cols");
  if (!packed || !g_idx || !scale || !zero_packed || !mem || !layer)
    return fail(GPTQ_ERR_INVALID_ARG, "packed, g_idx, scale, zero_packed, mem and layer "
                                      "must not be NULL");
  if (reinterpret_cast<uintptr_t>(mem) % 256)
    return fail(GPTQ_ERR_INVALID_ARG, "mem must be 256-byte aligned");
  const Geometry g = geometry(rows, cols, group);
  const LayerMap m = layer_map(mem, g);
  if (mem_bytes < m.bytes)
    return fail(GPTQ_ERR_INVALID_ARG, "mem too small: need " + std::to_string(m.bytes) +
                                          " bytes, got " + std::to_string(mem_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  GPTQ_TRY(launch("w4a16_init", w4a16_init_kernel, dim3(cdiv(g.k_pad, 256)), dim3(256), 0, s,
                  m.status, m.kperm, int32_t(g.k_pad)));
  GPTQ_TRY(launch("w4a16_kperm", w4a16_kperm_kernel, dim3(g.ngroups), dim3(kThreads), 0, s,
                  g_idx, int32_t(cols), group, int32_t(g.ngroups), int32_t(g.k_pad), m.kperm,
                  m.status));
  int32_t st[2] = {0, 0};
  if (hipMemcpyAsync(st, m.status, sizeof(st), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(GPTQ_ERR_DEVICE, "w4a16 prepare: reading the status failed");
  if (st[0] & kStatBadGroup)
    return fail(GPTQ_ERR_INVALID_ARG, "g_idx out of range, or a group does not hold exactly "
                                      "`group` columns");
  const int64_t nw = g.rt16 * g.ksteps * 64;
  GPTQ_TRY(launch("w4a16_repack", w4a16_repack_kernel, dim3(cdiv(nw, kThreads)), dim3(kThreads),
                  0, s, packed, rows, cols, (const int32_t *)m.kperm, g.ksteps, nw, m.wq));
  const int64_t ns = g.rt16 * g.ngp * 16;
  GPTQ_TRY(launch("w4a16_scales", w4a16_scales_kernel, dim3(cdiv(ns, kThreads)), dim3(kThreads),
                  0, s, scale, zero_packed, rows, g.ngroups, g.ngp, ns, m.sc, m.zp));
  if (hipStreamSynchronize(s) != hipSuccess)
    return fail(GPTQ_ERR_DEVICE, "w4a16 prepare: repacking failed");
  layer->rows = rows;
  layer->cols = cols;
  layer->group = group;
  layer->permuted = (st[0] & kStatPermuted) ? 1 : 0;
  layer->rows_pad = g.rows_pad;
  layer->k_pad = g.k_pad;
  layer->mem = mem;
  layer->mem_bytes = mem_bytes;
  return GPTQ_OK;
}

size_t gptq_w4a16_workspace_bytes(const gptq_w4a16_layer *layer, int64_t batch) {
  if (!layer || batch < 1) return 0;
  const Geometry g = geometry(layer->rows, layer->cols, layer->group);
  return ws_bytes_for(g, layer->permuted != 0, batch, cu_count());
}

gptq_status gptq_w4a16_gemm(const gptq_w4a16_layer *layer, const uint16_t *x, int64_t batch,
                            uint16_t *y, void *ws, size_t ws_bytes, void *stream) {
  GPTQ_TRY(check_gemm_args(layer, x, batch, y));
  const Geometry g = geometry(layer->rows, layer->cols, layer->group);
  const size_t need = ws_bytes_for(g, layer->permuted != 0, batch, cu_count());
  if (need) {
    if (!ws) return fail(GPTQ_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % 256)
      return fail(GPTQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
      return fail(GPTQ_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) +
                                          " bytes, got " + std::to_string(ws_bytes));
  }
  return gemm_launches(layer, x, batch, y, ws, static_cast<hipStream_t>(stream));
}

gptq_status gptq_w4a16_gemm_noalloc(const gptq_w4a16_layer *layer, const uint16_t *x,
                                    int64_t batch, uint16_t *y, void *stream) {
  GPTQ_TRY(check_gemm_args(layer, x, batch, y));
  const Geometry g = geometry(layer->rows, layer->cols, layer->group);
  const size_t need = ws_bytes_for(g, layer->permuted != 0, batch, cu_count());
  if (need > kScratchBytes)
    return fail(GPTQ_ERR_WORKSPACE,
                "this product needs " + std::to_string(need) + " bytes of scratch; the static "
                "scratch holds " + std::to_string(kScratchBytes) +
                " (use a smaller batch, or gptq_w4a16_gemm with a workspace)");
  void *ws = nullptr;
  if (need) GPTQ_TRY(scratch_address(&ws));
  return gemm_launches(layer, x, batch, y, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"
