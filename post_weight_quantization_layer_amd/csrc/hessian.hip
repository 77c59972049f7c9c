// Hessian accumulation H += 2 X X^T ("GPTQ", section Komponenty) and the
// float64 activation energy hdiag += 2 sum_t x_it^2.
//
// bf16 path: a SYRK on bf16 MFMA (v_mfma_f32_32x32x16_bf16), fp32 accumulate.
// Only the upper-triangle 256x256 tiles of H are computed.  Each tile is
// owned by one workgroup that runs the whole token loop, so H is updated by
// one read-modify-write per tile and the result is deterministic (no split-K
// atomics).  X is d x n row-major (tokens contiguous), so both MFMA operands
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

// One workgroup per CU (128 KB of LDS) and one wave per SIMD: the kernel may
// use the whole register file, so both fragment sets stay in registers.
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
    syrk_bf16_kernel(float *__restrict__ H, double *__restrict__ hdiag,
                     const uint16_t *__restrict__ X, int64_t d, int64_t n, int64_t ld, int nt,
                     int ntiles, int per_xcd) {
  // XCD-aware mapping: workgroups are dealt round-robin to the 8 XCDs, so
  // give each XCD a contiguous run of the tile order (shared panels stay in
  // that XCD's L2).
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  if (slot >= per_xcd) return;
  const int t = xcd * per_xcd + slot;
  if (t >= ntiles) return;
  int ti, tj;
  tile_coords(t, nt, ti, tj);
  const bool diag = ti == tj;
  const int64_t I0 = int64_t(ti) * kTile, J0 = int64_t(tj) * kTile;

  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
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
  const int64_t nfull = n / kBK;
  const int lrow = tid >> 3, lchunk = tid & 7;
  const int lds_off = lrow * kRowBytes + ((lchunk ^ swz(lrow)) << 4);
  const uint16_t *rp[kLoads];
#pragma unroll
  for (int q = 0; q < kLoads; ++q)
    rp[q] = X + min((q < kPanelLoads ? I0 : J0) + lrow + 32 * (q % kPanelLoads), d - 1) * ld +
            lchunk * 8;
  u32x4_t stg[kLoads];
  auto load_one = [&](int q, int64_t ks) {
    stg[q] = *reinterpret_cast<const u32x4_t *>(rp[q] + min(ks, nfull - 1) * kBK);
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
  if (nfull > 0) {
#pragma unroll
    for (int q = 0; q < kLoads; ++q) load_one(q, 0);
#pragma unroll
    for (int q = 0; q < kLoads; ++q) store_one(q, 0);
#pragma unroll
    for (int q = 0; q < kLoads; ++q) load_one(q, 1);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  }
  bf16x8_t xa[4], xb[4], ya[4], yb[4];
  auto main_loop = [&](auto energy_tag) {
    constexpr bool kEnergy = decltype(energy_tag)::value;
    u32x4_t ep[2], eq[2];  // energy chunks of even / odd steps
    if (nfull > 0) {
      read_step(xa, xb, 0, 0);
      if (kEnergy) energy_read(ep, 0, 0);
    }
    for (int64_t ks = 0; ks < nfull; ++ks) {
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
  if (nfull * kBK < n) {
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

gptq_status hessian_accumulate_impl(float *H, double *hdiag, int64_t d, const void *X,
                                    int x_dtype, int64_t n_tok, int64_t ld_x,
                                    hipStream_t stream) {
  if (x_dtype == GPTQ_DT_BF16) {
    const uint16_t *Xb = static_cast<const uint16_t *>(X);
    const int nt = (int)cdiv(d, kTile);
    const int ntiles = nt * (nt + 1) / 2;
    const int per_xcd = (int)cdiv(ntiles, 8);
    const size_t lds = size_t(kStages) * kStageBytes;
    static bool lds_set = false;
    if (!lds_set) {
      hipError_t e = hipFuncSetAttribute((const void *)syrk_bf16_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess)
        return fail(GPTQ_ERR_DEVICE, std::string("cannot raise LDS limit: ") + hipGetErrorString(e));
      lds_set = true;
    }
    GPTQ_TRY(launch("hessian_syrk_bf16", syrk_bf16_kernel, dim3(8 * per_xcd), dim3(kThreads), lds,
                    stream, H, hdiag, Xb, d, n_tok, ld_x, nt, ntiles, per_xcd));
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
