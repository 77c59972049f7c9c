// C ABI entry points: argument validation (host only, before any launch),
// thread-local error text, and the event-based per-kernel profiler.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "common.h"

namespace gptq {

static thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }

gptq_status fail(gptq_status st, const std::string &msg) {
  g_last_error = msg;
  return st;
}

// ---------------------------------------------------------------- profiler
namespace {
struct Pending {
  int slot;
  hipEvent_t start, stop;
};
struct Profiler {
  bool on = false;
  std::vector<std::string> names;
  std::map<std::string, int> slot_of;
  std::vector<int64_t> launches;
  std::vector<double> ms;
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;

  hipEvent_t get_event() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  int slot(const char *name) {
    auto it = slot_of.find(name);
    if (it != slot_of.end()) return it->second;
    int s = (int)names.size();
    names.push_back(name);
    slot_of[name] = s;
    launches.push_back(0);
    ms.push_back(0.0);
    return s;
  }
  void drain() {
    for (auto &p : pending) {
      float t = 0.f;
      if (hipEventSynchronize(p.stop) == hipSuccess &&
          hipEventElapsedTime(&t, p.start, p.stop) == hipSuccess) {
        launches[p.slot] += 1;
        ms[p.slot] += t;
      }
      pool.push_back(p.start);
      pool.push_back(p.stop);
    }
    pending.clear();
  }
};
Profiler &prof() {
  static Profiler P;
  return P;
}
}  // namespace

ProfileToken profile_begin(const char *name, hipStream_t stream) {
  ProfileToken t;
  Profiler &P = prof();
  if (!P.on) return t;
  t.start = P.get_event();
  if (!t.start) return t;
  t.slot = P.slot(name);
  (void)hipEventRecord(t.start, stream);
  return t;
}

void profile_end(ProfileToken tok, hipStream_t stream) {
  if (tok.slot < 0) return;
  Profiler &P = prof();
  hipEvent_t stop = P.get_event();
  if (!stop) {
    P.pool.push_back(tok.start);
    return;
  }
  (void)hipEventRecord(stop, stream);
  P.pending.push_back({tok.slot, tok.start, stop});
  if (P.pending.size() > (size_t(1) << 18)) P.drain();
}

// ------------------------------------------------------- per-device set-up
namespace {
std::mutex g_setup_mu;
std::map<std::pair<const void *, int>, size_t> g_lds_limit;  // (kernel, device) -> bytes
std::map<int, int> g_cu_count;                               // device -> compute units
}  // namespace

gptq_status allow_dynamic_lds(const void *kernel, size_t bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(GPTQ_ERR_DEVICE, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(g_setup_mu);
  auto key = std::make_pair(kernel, dev);
  auto it = g_lds_limit.find(key);
  if (it != g_lds_limit.end() && it->second >= bytes) return GPTQ_OK;
  hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess)
    return fail(GPTQ_ERR_DEVICE, std::string("cannot raise LDS limit: ") + hipGetErrorString(e));
  g_lds_limit[key] = bytes;
  return GPTQ_OK;
}

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(g_setup_mu);
  auto it = g_cu_count.find(dev);
  if (it != g_cu_count.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  g_cu_count[dev] = n;
  return n;
}

// ------------------------------------------------------------- validation
static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

static gptq_status check_params(const gptq_params *p, int64_t cols) {
  if (!p) return fail(GPTQ_ERR_INVALID_ARG, "params is NULL");
  if (p->grid != GPTQ_GRID_AFFINE && p->grid != GPTQ_GRID_Q4K)
    return fail(GPTQ_ERR_INVALID_ARG, "grid must be GPTQ_GRID_AFFINE or GPTQ_GRID_Q4K");
  if (p->grid == GPTQ_GRID_AFFINE && (p->bits < 2 || p->bits > 8))
    return fail(GPTQ_ERR_INVALID_ARG, "bits must be in [2, 8] for the affine grid");
  if (p->grid == GPTQ_GRID_Q4K && (p->bits < 2 || p->bits > 6))
    return fail(GPTQ_ERR_INVALID_ARG, "bits must be in [2, 6] for the two-level (Q4K) grid");
  if (p->grid == GPTQ_GRID_Q4K && p->group != 256)
    return fail(GPTQ_ERR_INVALID_ARG, "the Q4K grid has 256-weight super-blocks (group = 256)");
  if (p->group < 1) return fail(GPTQ_ERR_INVALID_ARG, "group must be >= 1");
  if (p->block < 1 || p->block > 128)
    return fail(GPTQ_ERR_INVALID_ARG, "block must be in [1, 128]");
  if (p->group % p->block != 0 && p->block % p->group != 0)
    return fail(GPTQ_ERR_INVALID_ARG, "group and block must divide one another");
  if (p->act_order != 0 && p->act_order != 1)
    return fail(GPTQ_ERR_INVALID_ARG, "act_order must be 0 or 1");
  if (!(p->percdamp >= 0.f) || !std::isfinite(p->percdamp))
    return fail(GPTQ_ERR_INVALID_ARG, "percdamp must be finite and >= 0");
  if (cols > 0 && cols % p->group != 0)
    return fail(GPTQ_ERR_INVALID_ARG, "cols must be a multiple of group");
  if (p->search != 0 && p->search != 1)
    return fail(GPTQ_ERR_INVALID_ARG, "search must be 0 or 1");
  if (p->route != GPTQ_ROUTE_INVERSE && p->route != GPTQ_ROUTE_HESSIAN)
    return fail(GPTQ_ERR_INVALID_ARG, "route must be GPTQ_ROUTE_INVERSE or GPTQ_ROUTE_HESSIAN");
  if (p->route == GPTQ_ROUTE_HESSIAN) {
    if (p->block != 128)
      return fail(GPTQ_ERR_INVALID_ARG, "the Hessian-factor route needs block = 128");
    if (p->grid != GPTQ_GRID_AFFINE || 128 % p->group != 0)
      return fail(GPTQ_ERR_INVALID_ARG,
                  "the Hessian-factor route needs the affine grid with group dividing 128");
    if (cols > 0 && cols % 128 != 0)
      return fail(GPTQ_ERR_INVALID_ARG, "the Hessian-factor route needs cols % 128 == 0");
  }
  return GPTQ_OK;
}

static gptq_status check_ws(void *ws, size_t ws_bytes, size_t need) {
  if (need == 0) return GPTQ_OK;
  if (!ws) return fail(GPTQ_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(GPTQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(GPTQ_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) +
                                        " bytes, got " + std::to_string(ws_bytes));
  return GPTQ_OK;
}

static constexpr int64_t kMaxDim = int64_t(1) << 20;  // features / columns
static constexpr int64_t kMaxRows = int64_t(1) << 24;

}  // namespace gptq

using namespace gptq;

extern "C" {

const char *gptq_last_error(void) { return g_last_error.c_str(); }

size_t gptq_workspace_bytes(int64_t rows, int64_t cols, const gptq_params *p) {
  if (rows < 1 || cols < 1 || rows > kMaxRows || cols > kMaxDim) {
    set_error("rows and cols must be in [1, 2^24] x [1, 2^20]");
    return 0;
  }
  if (check_params(p, cols) != GPTQ_OK) return 0;
  const size_t a = prepare_ws_bytes(cols);
  const size_t b = quantize_ws_bytes(rows, cols, *p);
  const size_t h = hessian_ws_bytes(cols);
  return std::max(a, std::max(b, h));
}

gptq_status gptq_hessian_accumulate(float *H, double *hdiag, int64_t d, const void *X,
                                    int32_t x_dtype, int64_t n_tok, int64_t ld_x, void *ws,
                                    size_t ws_bytes, void *stream) {
  if (d < 1 || d > kMaxDim) return fail(GPTQ_ERR_INVALID_ARG, "d must be in [1, 2^20]");
  if (!H || !hdiag) return fail(GPTQ_ERR_INVALID_ARG, "H and hdiag must not be NULL");
  if (x_dtype != GPTQ_DT_F32 && x_dtype != GPTQ_DT_BF16)
    return fail(GPTQ_ERR_INVALID_ARG, "x_dtype must be GPTQ_DT_F32 or GPTQ_DT_BF16");
  if (n_tok < 0) return fail(GPTQ_ERR_INVALID_ARG, "n_tok must be >= 0");
  if (n_tok == 0) return GPTQ_OK;
  if (!X) return fail(GPTQ_ERR_INVALID_ARG, "X must not be NULL");
  if (ld_x < n_tok) return fail(GPTQ_ERR_INVALID_ARG, "ld_x must be >= n_tok");
  if (!aligned(X, 16)) return fail(GPTQ_ERR_INVALID_ARG, "X must be 16-byte aligned");
  if (x_dtype == GPTQ_DT_BF16 && ld_x % 8)
    return fail(GPTQ_ERR_INVALID_ARG, "ld_x must be a multiple of 8 for bf16 X");
  if (x_dtype == GPTQ_DT_F32 && ld_x % 4)
    return fail(GPTQ_ERR_INVALID_ARG, "ld_x must be a multiple of 4 for f32 X");
  if (!aligned(H, 16) || !aligned(hdiag, 8))
    return fail(GPTQ_ERR_INVALID_ARG, "H must be 16-byte and hdiag 8-byte aligned");
  if (ws && !aligned(ws, 256))
    return fail(GPTQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return hessian_accumulate_impl(H, hdiag, d, X, x_dtype, n_tok, ld_x, ws, ws ? ws_bytes : 0,
                                 (hipStream_t)stream);
}

gptq_status gptq_prepare_hinv(const float *H, const double *hdiag, int64_t d,
                              const gptq_params *p, float *U, int32_t *perm, uint8_t *dead,
                              void *ws, size_t ws_bytes, void *stream) {
  if (d < 1 || d > kMaxDim) return fail(GPTQ_ERR_INVALID_ARG, "d must be in [1, 2^20]");
  GPTQ_TRY(check_params(p, 0));
  if (p->route == GPTQ_ROUTE_HESSIAN && d % 128 != 0)
    return fail(GPTQ_ERR_INVALID_ARG, "the Hessian-factor route needs d % 128 == 0");
  if (!H || !hdiag || !U || !perm || !dead)
    return fail(GPTQ_ERR_INVALID_ARG, "H, hdiag, U, perm and dead must not be NULL");
  if (!aligned(H, 16) || !aligned(U, 16))
    return fail(GPTQ_ERR_INVALID_ARG, "H and U must be 16-byte aligned");
  GPTQ_TRY(check_ws(ws, ws_bytes, prepare_ws_bytes(d)));
  return prepare_hinv_impl(H, hdiag, d, *p, U, perm, dead, ws, ws_bytes, (hipStream_t)stream);
}

gptq_status gptq_quantize_layer(float *W, int64_t rows, int64_t cols, const float *U,
                                const int32_t *perm, const uint8_t *dead, const double *hdiag,
                                const gptq_params *p,
                                uint8_t *q, int32_t *g_idx, float *scale, uint8_t *zero,
                                uint16_t *q4k_super_scale, uint16_t *q4k_super_min,
                                uint8_t *q4k_sub_scale, uint8_t *q4k_sub_min, void *ws,
                                size_t ws_bytes, void *stream) {
  if (rows < 1 || rows > kMaxRows || cols < 1 || cols > kMaxDim)
    return fail(GPTQ_ERR_INVALID_ARG, "rows and cols must be in [1, 2^24] x [1, 2^20]");
  GPTQ_TRY(check_params(p, cols));
  if (!W || !U || !perm || !dead || !q || !g_idx)
    return fail(GPTQ_ERR_INVALID_ARG, "W, U, perm, dead, q and g_idx must not be NULL");
  if (p->search && !hdiag)
    return fail(GPTQ_ERR_INVALID_ARG, "the weighted grid search needs hdiag");
  if (p->grid == GPTQ_GRID_AFFINE && (!scale || !zero))
    return fail(GPTQ_ERR_INVALID_ARG, "the affine grid needs scale and zero outputs");
  if (p->grid == GPTQ_GRID_Q4K &&
      (!q4k_super_scale || !q4k_super_min || !q4k_sub_scale || !q4k_sub_min))
    return fail(GPTQ_ERR_INVALID_ARG, "the Q4K grid needs the four q4k_* outputs");
  if (p->grid == GPTQ_GRID_Q4K && cols % 256)
    return fail(GPTQ_ERR_INVALID_ARG, "the Q4K grid needs cols to be a multiple of 256");
  if (!aligned(W, 16) || !aligned(U, 16))
    return fail(GPTQ_ERR_INVALID_ARG, "W and U must be 16-byte aligned");
  GPTQ_TRY(check_ws(ws, ws_bytes, quantize_ws_bytes(rows, cols, *p)));
  return quantize_layer_impl(W, rows, cols, U, perm, dead, hdiag, *p, q, g_idx, scale, zero,
                             q4k_super_scale, q4k_super_min, q4k_sub_scale, q4k_sub_min, ws,
                             ws_bytes, (hipStream_t)stream);
}

gptq_status gptq_pack(const uint8_t *codes, int64_t rows, int64_t cols, int32_t bits,
                      uint32_t *packed, void *stream) {
  if (bits < 1 || bits > 8) return fail(GPTQ_ERR_INVALID_ARG, "bits must be in [1, 8]");
  if (rows < 0 || cols < 0) return fail(GPTQ_ERR_INVALID_ARG, "rows and cols must be >= 0");
  if ((cols * bits) % 32) return fail(GPTQ_ERR_INVALID_ARG, "cols*bits must be a multiple of 32");
  if (rows == 0 || cols == 0) return GPTQ_OK;
  if (!codes || !packed) return fail(GPTQ_ERR_INVALID_ARG, "codes and packed must not be NULL");
  if (!aligned(packed, 4)) return fail(GPTQ_ERR_INVALID_ARG, "packed must be 4-byte aligned");
  return pack_impl(codes, rows, cols, bits, packed, (hipStream_t)stream);
}

void gptq_profile_enable(int on) { prof().on = on != 0; }

void gptq_profile_reset(void) {
  Profiler &P = prof();
  P.drain();
  for (auto &v : P.launches) v = 0;
  for (auto &v : P.ms) v = 0.0;
}

gptq_status gptq_profile_query(const char *name, int64_t *launches, double *total_ms) {
  if (!name || !launches || !total_ms)
    return fail(GPTQ_ERR_INVALID_ARG, "name, launches and total_ms must not be NULL");
  Profiler &P = prof();
  P.drain();
  auto it = P.slot_of.find(name);
  if (it == P.slot_of.end()) {
    *launches = 0;
    *total_ms = 0.0;
    return GPTQ_OK;
  }
  *launches = P.launches[it->second];
  *total_ms = P.ms[it->second];
  return GPTQ_OK;
}

}  // extern "C"
