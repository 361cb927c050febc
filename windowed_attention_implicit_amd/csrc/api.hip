// C ABI of the RIB window-attention library: argument validation, workspace
// layout and the launch sequence of each entry point. Every argument is
// checked before the first launch; nothing here allocates device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <optional>
#include <string>
#include <utility>
#include <vector>

#include "internal.hpp"

namespace rib {
namespace {

thread_local std::string g_last_error;

rib_status_t fail(rib_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
rib_status_t fail(rib_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

rib_status_t ok() {
  g_last_error.clear();
  return RIB_OK;
}

rib_status_t hip_fail(hipError_t e, const char* what) {
  return fail(RIB_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int esize_of(rib_dtype_t dt) { return dt == RIB_F32 ? 4 : 2; }

bool dtype_ok(rib_dtype_t dt) { return dt == RIB_F32 || dt == RIB_BF16; }

int padded_rank(int r) { return r <= 16 ? 16 : 32; }

constexpr int kMaxW = 256;

// Shape checks shared by every attention entry point.
rib_status_t check_shape(const rib_shape_t* s, rib_dtype_t dt, bool need_rank) {
  if (!s) return fail(RIB_ERR_INVALID_ARG, "shape is NULL");
  if (!dtype_ok(dt)) return fail(RIB_ERR_INVALID_ARG, "dtype %d is not RIB_F32 or RIB_BF16", (int)dt);
  if (s->B < 0 || s->H <= 0 || s->W <= 0 || s->heads <= 0 || s->d_c <= 0)
    return fail(RIB_ERR_INVALID_ARG, "B must be >= 0 and H, W, heads, d_c > 0 (got B=%d H=%d W=%d heads=%d d_c=%d)",
                s->B, s->H, s->W, s->heads, s->d_c);
  if (s->w < 2) return fail(RIB_ERR_INVALID_ARG, "window size w=%d must be >= 2", s->w);
  if (s->H % s->w || s->W % s->w)
    return fail(RIB_ERR_INVALID_ARG, "H=%d and W=%d must be multiples of the window size w=%d", s->H, s->W, s->w);
  if (s->w > kMaxW) return fail(RIB_ERR_UNSUPPORTED, "window size w=%d exceeds %d", s->w, kMaxW);
  if (need_rank) {
    if (s->r < 1) return fail(RIB_ERR_INVALID_ARG, "rank r=%d must be >= 1", s->r);
    if (s->r > 32) return fail(RIB_ERR_UNSUPPORTED, "rank r=%d exceeds 32", s->r);
    if (s->d_c != 32 && s->d_c != 64)
      return fail(RIB_ERR_UNSUPPORTED, "d_c=%d: d_c = 32 and 64 are implemented", s->d_c);
  }
  int64_t elems = (int64_t)s->B * s->H * s->W * s->heads * s->d_c;
  if (elems > ((int64_t)1 << 40)) return fail(RIB_ERR_UNSUPPORTED, "feature map too large");
  return RIB_OK;
}

rib_status_t check_ptr(const void* p, const char* name) {
  if (!p) return fail(RIB_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(RIB_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return RIB_OK;
}

#define RIB_TRY(expr)                 \
  do {                                \
    rib_status_t _st = (expr);        \
    if (_st != RIB_OK) return _st;    \
  } while (0)

// Sequential carve-out of a workspace in 256-byte aligned pieces.
struct Carve {
  uintptr_t base;
  size_t off = 0;
  explicit Carve(void* p) : base((uintptr_t)p) {}
  void* take(size_t bytes) {
    void* p = (void*)(base + off);
    off += (size_t)round_up((int64_t)bytes, 256);
    return p;
  }
};

struct FwdLayout {
  void *qw, *kw, *vw, *ow, *qp, *kp;
  float* kmax2;
  float* part;   // split-tail pieces of the bf16 kernel (nullptr: none reserved)
  size_t bytes;
};

// The bf16 MFMA kernels cover d_c = 32; float32 runs and d_c = 64 take the simple kernels
// (windowed rows in and out).
bool mfma_path(const Geom& g, rib_dtype_t dt) { return dt == RIB_BF16 && g.d_c == 32; }

// ... and among them, windows whose side divides 64 (a 64-key tile is whole window rows) with
// one positional K-step: the attention kernels read K_c and V (backward: and dO) in their maps,
// through buffer resources spanning one window (w map rows must fit a 31-bit byte range).
bool mapkv_path(const Geom& g, rib_dtype_t dt) {
  return mfma_path(g, dt) && g.r <= 16 && g.w >= 8 && 64 % g.w == 0 &&
         (int64_t)g.w * g.W * g.heads * 64 < ((int64_t)1 << 31);
}

FwdLayout fwd_layout(const Geom& g, rib_dtype_t dt, void* ws) {
  const int es = esize_of(dt);
  const size_t t = (size_t)g.units * g.n_rows * g.d_c * es;
  const size_t pos = (size_t)g.n_rows * padded_rank(g.r) * es;
  Carve c(ws);
  FwdLayout L;
  // the bf16 MFMA kernel reads Q_c and writes O in the map layout directly
  const bool rows_qo = !mfma_path(g, dt);
  const bool mapkv = mapkv_path(g, dt);
  L.qw = rows_qo ? c.take(t) : nullptr;
  L.kw = mapkv ? nullptr : c.take(t);
  L.vw = mapkv ? nullptr : c.take(t);
  L.ow = rows_qo ? c.take(t) : nullptr;
  // the bf16 kernel reads Q_p, K_p in place when no padding is needed (r = 16 or 32)
  const bool pack = rows_qo || g.r != padded_rank(g.r);
  L.qp = pack ? c.take(pos) : nullptr;
  L.kp = pack ? c.take(pos) : nullptr;
  L.kmax2 = mapkv ? nullptr : (float*)c.take(2 * (size_t)g.units * key_bound_parts(g.N) * sizeof(float));
  const size_t pieces = rows_qo ? 0 : split_region_pieces(g.units, g.N);
  L.part = pieces ? (float*)c.take(pieces * kSplitPieceFloats * sizeof(float)) : nullptr;
  L.bytes = c.off;
  return L;
}

// RPB comparison forward: windowed K (rows) and V^T (kappa), key-norm maxima,
// the fp16 tables, their maxima and the per-key table offsets.
struct RpbLayout {
  void *kw, *vw;
  float* kmax2;
  _Float16* tab16;
  float* tmax;
  int* kidx;
  size_t bytes;
};

RpbLayout rpb_layout(const Geom& g, void* ws) {
  const size_t t = (size_t)g.units * g.n_rows * g.d_c * 2;
  Carve c(ws);
  RpbLayout L;
  L.kw = c.take(t);
  L.vw = c.take(t);
  L.kmax2 = (float*)c.take(2 * (size_t)g.units * key_bound_parts(g.N) * sizeof(float));
  L.tab16 = (_Float16*)c.take((size_t)g.heads * rpb_table_stride(g.w) * 2);
  L.tmax = (float*)c.take((size_t)g.heads * sizeof(float));
  L.kidx = (int*)c.take((size_t)g.n_rows * sizeof(int));
  L.bytes = c.off;
  return L;
}

constexpr size_t kLdsPerCu = 160 * 1024;

rib_status_t check_rpb(const rib_shape_t* s, rib_dtype_t dt) {
  RIB_TRY(check_shape(s, dt, false));
  if (dt != RIB_BF16) return fail(RIB_ERR_UNSUPPORTED, "the RPB kernel is bfloat16 only");
  if (s->d_c != 32) return fail(RIB_ERR_UNSUPPORTED, "d_c=%d: only d_c = 32 is implemented", s->d_c);
  if (rpb_fwd_lds_bytes(s->w) > kLdsPerCu)
    return fail(RIB_ERR_UNSUPPORTED, "window size w=%d: the RPB table and tiles need %zu bytes of LDS (max %zu)", s->w,
                rpb_fwd_lds_bytes(s->w), kLdsPerCu);
  return RIB_OK;
}

struct BwdLayout {
  void *qw, *kw, *vw, *dow, *qp, *kp, *dqw, *dkw, *dvw;
  float *lse2, *dd, *dqp_part, *dkp_part;
  size_t bytes;
};

BwdLayout bwd_layout(const Geom& g, rib_dtype_t dt, void* ws) {
  // bf: the MFMA kernels, which write the map directly
  const int es = esize_of(dt);
  const int rp = padded_rank(g.r);
  const size_t t = (size_t)g.units * g.n_rows * g.d_c * es;
  const size_t pos = (size_t)g.n_rows * rp * es;
  const size_t rowf = (size_t)g.units * g.n_rows * sizeof(float);
  const size_t part = (size_t)g.units * g.n_rows * rp * sizeof(float);
  const bool bf = mfma_path(g, dt);
  const bool mapkv = mapkv_path(g, dt);   // K_c, V read in their maps
  Carve c(ws);
  BwdLayout L;
  L.qw = c.take(t);
  L.kw = mapkv ? nullptr : c.take(t);
  L.vw = mapkv ? nullptr : c.take(t);
  L.dow = c.take(t);
  L.qp = c.take(pos);
  L.kp = c.take(pos);
  // the bf16 kernels write dQ_c, dK_c, dV in the map layout directly
  L.dqw = bf ? nullptr : c.take(t);
  L.dkw = bf ? nullptr : c.take(t);
  L.dvw = bf ? nullptr : c.take(t);
  L.lse2 = (float*)c.take(rowf);
  L.dd = (float*)c.take(rowf);
  L.dqp_part = (float*)c.take(part);
  L.dkp_part = (float*)c.take(part);
  L.bytes = c.off;
  return L;
}

// ---- kernel timing (measurement aid, off by default)
struct TimingState {
  std::mutex mu;
  uint32_t mask = 0;   // bit k: group k is timed
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[RIB_KERNEL_COUNT];
};

TimingState& timing() {
  static TimingState t;
  return t;
}

// Brackets a group of launches with events on `stream` while timing is enabled;
// a group abandoned by an early error return records nothing.
class TimedGroup {
 public:
  TimedGroup(rib_kernel_t k, hipStream_t s) : k_(k), s_(s) {
    TimingState& t = timing();
    {
      std::lock_guard<std::mutex> g(t.mu);
      if (!((t.mask >> (int)k_) & 1u)) return;
    }
    // timing-only events: no system-scope fence (an L2 write-back and invalidate at every
    // record, which would idle the GPU between the launches being timed)
    if (hipEventCreateWithFlags(&a_, hipEventDisableSystemFence) != hipSuccess) return;
    if (hipEventCreateWithFlags(&b_, hipEventDisableSystemFence) != hipSuccess) {
      (void)hipEventDestroy(a_);
      return;
    }
    if (hipEventRecord(a_, s_) != hipSuccess) {
      (void)hipEventDestroy(a_);
      (void)hipEventDestroy(b_);
      return;
    }
    on_ = true;
  }
  void end() {
    if (!on_) return;
    on_ = false;
    if (hipEventRecord(b_, s_) != hipSuccess) {
      (void)hipEventDestroy(a_);
      (void)hipEventDestroy(b_);
      return;
    }
    TimingState& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    t.ev[k_].push_back({a_, b_});
  }
  ~TimedGroup() {
    if (on_) {
      (void)hipEventDestroy(a_);
      (void)hipEventDestroy(b_);
    }
  }
  TimedGroup(const TimedGroup&) = delete;
  TimedGroup& operator=(const TimedGroup&) = delete;

 private:
  rib_kernel_t k_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
  bool on_ = false;
};

// ---- workspace of the allocation-free forward: a file-scope array in device memory, one per
// GPU the library runs on, held until the process ends. In host code `scratch` names a host-side
// stand-in, not the array: kernels get the address hipGetSymbolAddress returns on each device.
static __device__ __align__(256) unsigned char scratch[RIB_NOALLOC_WORKSPACE_BYTES];

struct ScratchTable {
  std::mutex mu;
  void* ptr[64] = {};
};

ScratchTable& scratch_table() {
  static ScratchTable t;
  return t;
}

// The array's address on the device `stream` belongs to, which must be the current device
// (*wrong_device is set otherwise); looked up once per device.
hipError_t scratch_address(hipStream_t stream, void** out, bool* wrong_device, int* devs) {
  *wrong_device = false;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (stream) {
    hipDevice_t sd = 0;
    if ((e = hipStreamGetDevice(stream, &sd)) != hipSuccess) return e;
    if ((int)sd != dev) {
      *wrong_device = true;
      devs[0] = (int)sd;
      devs[1] = dev;
      return hipSuccess;
    }
  }
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  ScratchTable& t = scratch_table();
  std::lock_guard<std::mutex> lk(t.mu);
  if (!t.ptr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    t.ptr[dev] = p;
  }
  *out = t.ptr[dev];
  return hipSuccess;
}

float resolve_scale(float scale, const rib_shape_t* s) {
  return scale > 0.f ? scale : 1.0f / sqrtf((float)(s->d_c + s->r));
}

constexpr float kLog2e = 1.44269504088896340736f;

}  // namespace
}  // namespace rib

using namespace rib;

extern "C" {

const char* rib_status_string(rib_status_t status) {
  switch (status) {
    case RIB_OK: return "RIB_OK";
    case RIB_ERR_INVALID_ARG: return "RIB_ERR_INVALID_ARG";
    case RIB_ERR_UNSUPPORTED: return "RIB_ERR_UNSUPPORTED";
    case RIB_ERR_WORKSPACE: return "RIB_ERR_WORKSPACE";
    case RIB_ERR_HIP: return "RIB_ERR_HIP";
  }
  return "RIB_ERR_UNKNOWN";
}

const char* rib_last_error(void) { return g_last_error.c_str(); }

rib_status_t rib_kernel_timing_enable(int32_t enable) {
  return rib_kernel_timing_select(enable ? (1u << RIB_KERNEL_COUNT) - 1u : 0u);
}

rib_status_t rib_kernel_timing_select(uint32_t mask) {
  if (mask >> RIB_KERNEL_COUNT)
    return fail(RIB_ERR_INVALID_ARG, "timing mask 0x%x names groups past the last (%d)", mask, RIB_KERNEL_COUNT - 1);
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.mask = mask;
  return ok();
}

rib_status_t rib_kernel_timing_read(rib_kernel_t kernel, double* total_ms, int64_t* launches) {
  try {
    if ((int)kernel < 0 || (int)kernel >= RIB_KERNEL_COUNT)
      return fail(RIB_ERR_INVALID_ARG, "kernel group %d out of range", (int)kernel);
    if (!total_ms || !launches) return fail(RIB_ERR_INVALID_ARG, "output pointers are NULL");
    std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
    {
      TimingState& t = timing();
      std::lock_guard<std::mutex> g(t.mu);
      ev.swap(t.ev[kernel]);
    }
    double sum = 0.0;
    hipError_t first = hipSuccess;
    for (auto& p : ev) {
      float ms = 0.f;
      hipError_t e = hipEventSynchronize(p.second);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.first, p.second);
      if (e != hipSuccess && first == hipSuccess) first = e;
      sum += ms;
      (void)hipEventDestroy(p.first);
      (void)hipEventDestroy(p.second);
    }
    *total_ms = sum;
    *launches = (int64_t)ev.size();
    if (first != hipSuccess) return hip_fail(first, "reading kernel timing events");
    return ok();
  } catch (...) {
    return fail(RIB_ERR_HIP, "unexpected C++ exception in rib_kernel_timing_read");
  }
}

// Limits shared by rib_posgen and rib_posgen_bwd.
static rib_status_t check_mlp(int32_t w, const rib_mlp_t* mlp) {
  if (w < 2) return fail(RIB_ERR_INVALID_ARG, "window size w=%d must be >= 2", w);
  if (w > kMaxW) return fail(RIB_ERR_UNSUPPORTED, "window size w=%d exceeds %d", w, kMaxW);
  if (!mlp) return fail(RIB_ERR_INVALID_ARG, "mlp is NULL");
  if (mlp->n_freq < 1 || mlp->n_freq > 16) return fail(RIB_ERR_UNSUPPORTED, "n_freq=%d must be in 1..16", mlp->n_freq);
  if (mlp->hidden < 1 || mlp->hidden > 128) return fail(RIB_ERR_UNSUPPORTED, "hidden=%d must be in 1..128", mlp->hidden);
  if (mlp->rank < 1 || mlp->rank > 32) return fail(RIB_ERR_UNSUPPORTED, "rank=%d must be in 1..32", mlp->rank);
  if (!mlp->w1 || !mlp->w2) return fail(RIB_ERR_INVALID_ARG, "mlp weights are NULL");
  if (((uintptr_t)mlp->w1 | (uintptr_t)mlp->w2 | (uintptr_t)mlp->b1 | (uintptr_t)mlp->b2) & 3u)
    return fail(RIB_ERR_INVALID_ARG, "mlp weights must be 4-byte aligned");
  return RIB_OK;
}

rib_status_t rib_posgen(int32_t w, const rib_mlp_t* mlp, rib_dtype_t out_dtype, void* q_p, void* k_p,
                        rib_stream_t stream) {
  try {
    RIB_TRY(check_mlp(w, mlp));
    if (!dtype_ok(out_dtype)) return fail(RIB_ERR_INVALID_ARG, "out_dtype %d invalid", (int)out_dtype);
    const size_t lds = posgen_lds_bytes(*mlp);
    if (lds > 65536) return fail(RIB_ERR_UNSUPPORTED, "MLP too large for one LDS stage (%zu bytes)", lds);
    if (!q_p || !k_p) return fail(RIB_ERR_INVALID_ARG, "q_p / k_p is NULL");
    if (((uintptr_t)q_p | (uintptr_t)k_p) & (uintptr_t)(esize_of(out_dtype) - 1))
      return fail(RIB_ERR_INVALID_ARG, "q_p / k_p misaligned for their element type");
    TimedGroup tg(RIB_KERNEL_POSGEN, (hipStream_t)stream);
    hipError_t e = launch_posgen(w, *mlp, out_dtype, q_p, k_p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "posgen launch");
    tg.end();
    return ok();
  } catch (...) {
    return fail(RIB_ERR_HIP, "unexpected C++ exception in rib_posgen");
  }
}

size_t rib_posgen_bwd_workspace_size(int32_t w, const rib_mlp_t* mlp) {
  if (check_mlp(w, mlp) != RIB_OK) return 0;
  return posgen_bwd_workspace_bytes(w, *mlp);
}

rib_status_t rib_posgen_bwd(int32_t w, const rib_mlp_t* mlp, const float* dq_p, const float* dk_p, float* dw1,
                            float* db1, float* dw2, float* db2, void* workspace, size_t workspace_bytes,
                            rib_stream_t stream) {
  try {
    RIB_TRY(check_mlp(w, mlp));
    const size_t lds = posgen_bwd_lds_bytes(*mlp);
    if (lds > 65536) return fail(RIB_ERR_UNSUPPORTED, "MLP too large for one LDS stage (%zu bytes)", lds);
    if (!dq_p || !dk_p) return fail(RIB_ERR_INVALID_ARG, "dq_p / dk_p is NULL");
    if (!dw1 || !dw2) return fail(RIB_ERR_INVALID_ARG, "dw1 / dw2 is NULL");
    if (((uintptr_t)dq_p | (uintptr_t)dk_p | (uintptr_t)dw1 | (uintptr_t)db1 | (uintptr_t)dw2 | (uintptr_t)db2 |
         (uintptr_t)workspace) & 3u)
      return fail(RIB_ERR_INVALID_ARG, "float arguments must be 4-byte aligned");
    const size_t need = posgen_bwd_workspace_bytes(w, *mlp);
    if (!workspace || workspace_bytes < need)
      return fail(RIB_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
    TimedGroup tg(RIB_KERNEL_POSGEN_BWD, (hipStream_t)stream);
    hipError_t e = launch_posgen_bwd(w, *mlp, dq_p, dk_p, dw1, db1, dw2, db2, workspace, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "posgen backward launch");
    tg.end();
    return ok();
  } catch (...) {
    return fail(RIB_ERR_HIP, "unexpected C++ exception in rib_posgen_bwd");
  }
}

static rib_status_t partition_common(const rib_shape_t* shape, rib_dtype_t dtype, const void* a, void* b,
                                     bool forward, rib_stream_t stream) {
  try {
    RIB_TRY(check_shape(shape, dtype, false));
    if ((shape->d_c * esize_of(dtype)) % 16)
      return fail(RIB_ERR_UNSUPPORTED, "d_c * element size must be a multiple of 16 bytes");
    if (shape->B == 0) return ok();
    RIB_TRY(check_ptr(a, forward ? "x" : "x_win"));
    RIB_TRY(check_ptr(b, forward ? "x_win" : "x"));
    Geom g = make_geom(*shape);
    hipError_t e = forward ? launch_partition_plain(g, esize_of(dtype), a, b, (hipStream_t)stream)
                           : launch_unpartition_plain(g, esize_of(dtype), a, b, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "partition launch");
    return ok();
  } catch (...) {
    return fail(RIB_ERR_HIP, "unexpected C++ exception in window partition");
  }
}

rib_status_t rib_window_partition(const rib_shape_t* shape, rib_dtype_t dtype, const void* x, void* x_win,
                                  rib_stream_t stream) {
  return partition_common(shape, dtype, x, x_win, true, stream);
}

rib_status_t rib_window_unpartition(const rib_shape_t* shape, rib_dtype_t dtype, const void* x_win, void* x,
                                    rib_stream_t stream) {
  return partition_common(shape, dtype, x_win, x, false, stream);
}

size_t rib_fwd_workspace_size(const rib_shape_t* shape, rib_dtype_t dtype) {
  if (check_shape(shape, dtype, true) != RIB_OK) return 0;
  Geom g = make_geom(*shape);
  // at least 256 bytes: 0 means an invalid shape (the map-addressed windows need nothing)
  return std::max<size_t>(fwd_layout(g, dtype, nullptr).bytes, 256);
}

size_t rib_bwd_workspace_size(const rib_shape_t* shape, rib_dtype_t dtype) {
  if (check_shape(shape, dtype, true) != RIB_OK) return 0;
  Geom g = make_geom(*shape);
  return bwd_layout(g, dtype, nullptr).bytes;
}

// Every argument of a forward call except the workspace (B == 0 skips the pointer checks).
static rib_status_t check_fwd_args(const rib_shape_t* shape, rib_dtype_t dtype, float scale, const void* q_c,
                                   const void* k_c, const void* v, const void* q_p, const void* k_p,
                                   const void* gate, const void* o, const float* lse) {
  RIB_TRY(check_shape(shape, dtype, true));
  if (!(scale == scale) || isinf(scale)) return fail(RIB_ERR_INVALID_ARG, "scale is not finite");
  if (shape->B == 0) return RIB_OK;
  RIB_TRY(check_ptr(q_c, "q_c"));
  RIB_TRY(check_ptr(k_c, "k_c"));
  RIB_TRY(check_ptr(v, "v"));
  RIB_TRY(check_ptr(q_p, "q_p"));
  RIB_TRY(check_ptr(k_p, "k_p"));
  RIB_TRY(check_ptr(o, "o"));
  if (gate) RIB_TRY(check_ptr(gate, "gate"));
  if (lse && ((uintptr_t)lse & 3u)) return fail(RIB_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  return RIB_OK;
}

static rib_status_t attn_fwd_impl(const rib_shape_t* shape, rib_dtype_t dtype, float scale, const void* q_c,
                                  const void* k_c, const void* v, const void* q_p, const void* k_p,
                                  const void* gate, void* o, float* lse, void* workspace, size_t workspace_bytes,
                                  rib_stream_t stream) {
  {
    RIB_TRY(check_fwd_args(shape, dtype, scale, q_c, k_c, v, q_p, k_p, gate, o, lse));
    if (shape->B == 0) return ok();
    Geom g = make_geom(*shape);
    const size_t need = std::max<size_t>(fwd_layout(g, dtype, nullptr).bytes, 256);
    if (!workspace || workspace_bytes < need)
      return fail(RIB_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
    if ((uintptr_t)workspace & 255u) return fail(RIB_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    FwdLayout L = fwd_layout(g, dtype, workspace);
    hipStream_t st = (hipStream_t)stream;
    const int es = esize_of(dtype);
    const int rp = padded_rank(g.r);
    hipError_t e;
    const bool bf = mfma_path(g, dtype);
    const bool mapkv = mapkv_path(g, dtype);
    const void* kp_rows = L.kp ? L.kp : k_p;
    FwdArgs a;
    a.g = g;
    a.c = resolve_scale(scale, shape) * kLog2e;
    a.qw = L.qw; a.kw = L.kw; a.vw = L.vw; a.ow = L.ow;
    a.qp = L.qp ? L.qp : q_p;
    a.kp = kp_rows;
    a.q_map = q_c; a.o_map = o;
    a.k_map = mapkv ? k_c : nullptr;
    a.v_map = mapkv ? v : nullptr;
    a.lse = lse;
    a.kmax2 = L.kmax2;
    a.rp = rp;
    a.gate = gate;
    a.part = L.part;
    // the split plan queries the device (it can fail), so it is made before anything is launched
    if (bf && (e = plan_fwd_split(a)) != hipSuccess) return hip_fail(e, "split plan");
    // the partition group is timed only where it launches something (map-addressed windows with
    // r = 16 or 32 gather nothing)
    std::optional<TimedGroup> t_part;
    if (L.qp || !mapkv) t_part.emplace(RIB_KERNEL_PARTITION, st);
    if (L.qp) {   // positional rows padded to rp (the fused gather below reads K_p)
      if ((e = launch_pack_pos(g.N, g.n_rows, g.r, rp, es, q_p, es, L.qp, st)) != hipSuccess)
        return hip_fail(e, "pack q_p");
      if ((e = launch_pack_pos(g.N, g.n_rows, g.r, rp, es, k_p, es, L.kp, st)) != hipSuccess)
        return hip_fail(e, "pack k_p");
    }
    if (mapkv) {
      // nothing to gather: the attention kernel reads K_c and V in their maps
    } else if (bf) {
      // K_c rows, V^T kappa and the key-norm partial maxima in one pass
      if ((e = launch_gather_kv_bound(g, rp, k_c, v, kp_rows, L.kw, L.vw, L.kmax2, st)) != hipSuccess)
        return hip_fail(e, "partition k, v");
    } else {
      if ((e = launch_partition(g, es, q_c, L.qw, st)) != hipSuccess) return hip_fail(e, "partition q");
      if ((e = launch_partition(g, es, k_c, L.kw, st)) != hipSuccess) return hip_fail(e, "partition k");
      if ((e = launch_partition(g, es, v, L.vw, st)) != hipSuccess) return hip_fail(e, "partition v");
    }
    if (t_part) t_part->end();
    TimedGroup t_attn(RIB_KERNEL_ATTN_FWD, st);
    e = bf ? launch_attn_fwd_bf16(a, st) : launch_attn_fwd_simple(a, es, st);
    if (e != hipSuccess) return hip_fail(e, "attention forward");
    t_attn.end();
    if (bf && a.split_spx) {
      // the pieces of the split tail: O and LSE of those items
      TimedGroup t_comb(RIB_KERNEL_UNPARTITION, st);
      if ((e = launch_fwd_split_combine(a, st)) != hipSuccess) return hip_fail(e, "split combine");
      t_comb.end();
    }
    if (!bf) {
      TimedGroup t_unp(RIB_KERNEL_UNPARTITION, st);
      if ((e = launch_unpartition(g, es, L.ow, o, st)) != hipSuccess) return hip_fail(e, "unpartition o");
      t_unp.end();
    }
    return ok();
  }
}

rib_status_t rib_window_attn_fwd(const rib_shape_t* shape, rib_dtype_t dtype, float scale, const void* q_c,
                                 const void* k_c, const void* v, const void* q_p, const void* k_p, void* o,
                                 float* lse, void* workspace, size_t workspace_bytes, rib_stream_t stream) {
  try {
    return attn_fwd_impl(shape, dtype, scale, q_c, k_c, v, q_p, k_p, nullptr, o, lse, workspace, workspace_bytes,
                         stream);
  } catch (...) {
    return fail(RIB_ERR_HIP, "unexpected C++ exception in rib_window_attn_fwd");
  }
}

rib_status_t rib_window_attn_fwd_gated(const rib_shape_t* shape, rib_dtype_t dtype, float scale, const void* q_c,
                                       const void* k_c, const void* v, const void* q_p, const void* k_p,
                                       const void* gate, void* o, float* lse, void* workspace,
                                       size_t workspace_bytes, rib_stream_t stream) {
  try {
    if (!gate) return fail(RIB_ERR_INVALID_ARG, "gate is NULL (use rib_window_attn_fwd for ungated attention)");
    return attn_fwd_impl(shape, dtype, scale, q_c, k_c, v, q_p, k_p, gate, o, lse, workspace, workspace_bytes,
                         stream);
  } catch (...) {
    return fail(RIB_ERR_HIP, "unexpected C++ exception in rib_window_attn_fwd_gated");
  }
}

rib_status_t rib_window_attn_fwd_noalloc(const rib_shape_t* shape, rib_dtype_t dtype, float scale, const void* q_c,
                                         const void* k_c, const void* v, const void* q_p, const void* k_p, void* o,
                                         float* lse, rib_stream_t stream) {
  try {
    RIB_TRY(check_fwd_args(shape, dtype, scale, q_c, k_c, v, q_p, k_p, nullptr, o, lse));
    const size_t need = fwd_layout(make_geom(*shape), dtype, nullptr).bytes;
    if (need > RIB_NOALLOC_WORKSPACE_BYTES)
      return fail(RIB_ERR_WORKSPACE,
                  "this shape needs %zu bytes of workspace, more than the %zu the allocation-free forward holds "
                  "per GPU; call rib_window_attn_fwd with a caller workspace",
                  need, (size_t)RIB_NOALLOC_WORKSPACE_BYTES);
    if (shape->B == 0) return ok();
    void* ws = nullptr;
    bool wrong = false;
    int devs[2] = {0, 0};
    hipError_t e = scratch_address((hipStream_t)stream, &ws, &wrong, devs);
    if (e != hipSuccess) return hip_fail(e, "allocation-free forward: workspace address");
    if (wrong)
      return fail(RIB_ERR_INVALID_ARG, "stream belongs to device %d but device %d is current", devs[0], devs[1]);
    return attn_fwd_impl(shape, dtype, scale, q_c, k_c, v, q_p, k_p, nullptr, o, lse, ws,
                         RIB_NOALLOC_WORKSPACE_BYTES, stream);
  } catch (...) {
    return fail(RIB_ERR_HIP, "unexpected C++ exception in rib_window_attn_fwd_noalloc");
  }
}

rib_status_t rib_cla_gate(const rib_shape_t* shape, rib_dtype_t dtype, const void* x, const float* w_dw,
                          const float* b_dw, const float* w_pw, const float* b_pw, void* g, rib_stream_t stream) {
  try {
    if (!shape) return fail(RIB_ERR_INVALID_ARG, "shape is NULL");
    if (!dtype_ok(dtype)) return fail(RIB_ERR_INVALID_ARG, "dtype %d is not RIB_F32 or RIB_BF16", (int)dtype);
    if (shape->B < 0 || shape->H <= 0 || shape->W <= 0 || shape->heads <= 0 || shape->d_c <= 0)
      return fail(RIB_ERR_INVALID_ARG, "B must be >= 0 and H, W, heads, d_c > 0");
    const int64_t C64 = (int64_t)shape->heads * shape->d_c;
    if (C64 > 4096 || !cla_channels_supported((int)C64))
      return fail(RIB_ERR_UNSUPPORTED, "C = heads * d_c = %lld: the gate supports multiples of 32 up to 256",
                  (long long)C64);
    if ((int64_t)shape->B * shape->H * shape->W * C64 > ((int64_t)1 << 40))
      return fail(RIB_ERR_UNSUPPORTED, "feature map too large");
    if (shape->B == 0) return ok();
    RIB_TRY(check_ptr(x, "x"));
    RIB_TRY(check_ptr(g, "g"));
    if (!w_dw || ((uintptr_t)w_dw & 3u)) return fail(RIB_ERR_INVALID_ARG, "w_dw is NULL or not 4-byte aligned");
    if (!w_pw || ((uintptr_t)w_pw & 3u)) return fail(RIB_ERR_INVALID_ARG, "w_pw is NULL or not 4-byte aligned");
    if (b_dw && ((uintptr_t)b_dw & 3u)) return fail(RIB_ERR_INVALID_ARG, "b_dw is not 4-byte aligned");
    if (b_pw && ((uintptr_t)b_pw & 3u)) return fail(RIB_ERR_INVALID_ARG, "b_pw is not 4-byte aligned");
    GateArgs a;
    a.x = x; a.w_dw = w_dw; a.b_dw = b_dw; a.w_pw = w_pw; a.b_pw = b_pw; a.g = g;
    a.B = shape->B; a.H = shape->H; a.W = shape->W; a.C = (int)C64;
    hipStream_t st = (hipStream_t)stream;
    TimedGroup t(RIB_KERNEL_CLA_GATE, st);
    hipError_t e = launch_cla_gate(a, esize_of(dtype), st);
    if (e != hipSuccess) return hip_fail(e, "cla gate");
    t.end();
    return ok();
  } catch (...) {
    return fail(RIB_ERR_HIP, "unexpected C++ exception in rib_cla_gate");
  }
}

size_t rib_rpb_fwd_workspace_size(const rib_shape_t* shape, rib_dtype_t dtype) {
  if (check_rpb(shape, dtype) != RIB_OK) return 0;
  Geom g = make_geom(*shape);
  return rpb_layout(g, nullptr).bytes;
}

rib_status_t rib_rpb_window_attn_fwd(const rib_shape_t* shape, rib_dtype_t dtype, float scale, const void* q_c,
                                     const void* k_c, const void* v, const float* table, void* o, float* lse,
                                     void* workspace, size_t workspace_bytes, rib_stream_t stream) {
  try {
    RIB_TRY(check_rpb(shape, dtype));
    if (!(scale == scale) || isinf(scale)) return fail(RIB_ERR_INVALID_ARG, "scale is not finite");
    if (shape->B == 0) return ok();
    RIB_TRY(check_ptr(q_c, "q_c"));
    RIB_TRY(check_ptr(k_c, "k_c"));
    RIB_TRY(check_ptr(v, "v"));
    RIB_TRY(check_ptr(o, "o"));
    if (!table || ((uintptr_t)table & 3u)) return fail(RIB_ERR_INVALID_ARG, "table is NULL or not 4-byte aligned");
    if (lse && ((uintptr_t)lse & 3u)) return fail(RIB_ERR_INVALID_ARG, "lse is not 4-byte aligned");
    Geom g = make_geom(*shape);
    const size_t need = rpb_layout(g, nullptr).bytes;
    if (!workspace || workspace_bytes < need)
      return fail(RIB_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
    if ((uintptr_t)workspace & 255u) return fail(RIB_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    RpbLayout L = rpb_layout(g, workspace);
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    TimedGroup t_part(RIB_KERNEL_PARTITION, st);
    // K_c rows, V^T kappa and the key-norm partial maxima (no positional part) in one pass
    if ((e = launch_gather_kv_bound(g, 0, k_c, v, nullptr, L.kw, L.vw, L.kmax2, st)) != hipSuccess)
      return hip_fail(e, "partition k, v");
    if ((e = launch_rpb_prep(g, table, L.tab16, L.tmax, L.kidx, st)) != hipSuccess) return hip_fail(e, "rpb prep");
    FwdArgs a;
    a.g = g;
    a.c = (scale > 0.f ? scale : 1.0f / sqrtf((float)shape->d_c)) * kLog2e;
    a.qw = nullptr; a.kw = L.kw; a.vw = L.vw; a.qp = nullptr; a.kp = nullptr; a.ow = nullptr;
    a.q_map = q_c; a.o_map = o;
    a.lse = lse;
    a.kmax2 = L.kmax2;
    a.rp = 0;
    a.rpb_tab16 = L.tab16; a.rpb_max = L.tmax; a.rpb_kidx = L.kidx; a.rpb_stride = rpb_table_stride(g.w);
    t_part.end();
    TimedGroup t_attn(RIB_KERNEL_RPB_ATTN_FWD, st);
    if ((e = launch_attn_fwd_rpb(a, st)) != hipSuccess) return hip_fail(e, "rpb attention forward");
    t_attn.end();
    return ok();
  } catch (...) {
    return fail(RIB_ERR_HIP, "unexpected C++ exception in rib_rpb_window_attn_fwd");
  }
}

rib_status_t rib_window_attn_bwd(const rib_shape_t* shape, rib_dtype_t dtype, float scale, const void* q_c,
                                 const void* k_c, const void* v, const void* q_p, const void* k_p, const void* o,
                                 const float* lse, const void* d_o, void* dq_c, void* dk_c, void* dv, float* dq_p,
                                 float* dk_p, void* workspace, size_t workspace_bytes, rib_stream_t stream) {
  try {
    RIB_TRY(check_shape(shape, dtype, true));
    if (!(scale == scale) || isinf(scale)) return fail(RIB_ERR_INVALID_ARG, "scale is not finite");
    RIB_TRY(check_ptr(dq_p, "dq_p"));
    RIB_TRY(check_ptr(dk_p, "dk_p"));
    if (shape->B == 0) {
      // no unit contributes: the positional gradients are an empty sum (zeros)
      Geom g0 = make_geom(*shape);
      const int rp0 = padded_rank(g0.r);
      hipError_t e =
          launch_reduce_pos_grads(0, g0.N, g0.n_rows, g0.r, rp0, nullptr, dq_p, nullptr, dk_p, (hipStream_t)stream);
      if (e != hipSuccess) return hip_fail(e, "zero dq_p / dk_p");
      return ok();
    }
    RIB_TRY(check_ptr(q_c, "q_c"));
    RIB_TRY(check_ptr(k_c, "k_c"));
    RIB_TRY(check_ptr(v, "v"));
    RIB_TRY(check_ptr(q_p, "q_p"));
    RIB_TRY(check_ptr(k_p, "k_p"));
    RIB_TRY(check_ptr(o, "o"));
    RIB_TRY(check_ptr(lse, "lse"));
    RIB_TRY(check_ptr(d_o, "d_o"));
    RIB_TRY(check_ptr(dq_c, "dq_c"));
    RIB_TRY(check_ptr(dk_c, "dk_c"));
    RIB_TRY(check_ptr(dv, "dv"));
    Geom g = make_geom(*shape);
    const size_t need = bwd_layout(g, dtype, nullptr).bytes;
    if (!workspace || workspace_bytes < need)
      return fail(RIB_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
    if ((uintptr_t)workspace & 255u) return fail(RIB_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    BwdLayout L = bwd_layout(g, dtype, workspace);
    hipStream_t st = (hipStream_t)stream;
    const int es = esize_of(dtype);
    const int rp = padded_rank(g.r);
    const bool bf = mfma_path(g, dtype);
    hipError_t e;
#define RIB_LAUNCH(call, what)                        \
  do {                                                \
    if ((e = (call)) != hipSuccess) return hip_fail(e, what); \
  } while (0)
    TimedGroup t_part(RIB_KERNEL_PARTITION, st);
    if (bf) {
      // one pass: Q_c (pre-scaled), K_c, dO and V into windowed rows (map-addressed windows:
      // Q_c and dO only), -D and -LSE2 per row, and the positional rows
      BwdGather ga;
      ga.pm = make_pixel_map(g);
      ga.N = g.N; ga.n_rows = g.n_rows; ga.r = g.r; ga.rp = rp;
      ga.c = resolve_scale(scale, shape) * kLog2e;
      ga.q = (const bf16*)q_c; ga.k = (const bf16*)k_c; ga.v = (const bf16*)v;
      ga.d_o = (const bf16*)d_o; ga.o = (const bf16*)o; ga.lse = lse;
      ga.q_p = (const bf16*)q_p; ga.k_p = (const bf16*)k_p;
      ga.qw = (bf16*)L.qw; ga.kw = (bf16*)L.kw; ga.vw = (bf16*)L.vw; ga.dow = (bf16*)L.dow;
      ga.dd = L.dd; ga.lse2 = L.lse2;
      ga.qp = (bf16*)L.qp; ga.kp = (bf16*)L.kp;
      RIB_LAUNCH(launch_gather_bwd(ga, g.units, st), "backward gather");
      t_part.end();
    } else {
      RIB_LAUNCH(launch_partition(g, es, q_c, L.qw, st), "partition q");
      RIB_LAUNCH(launch_partition(g, es, k_c, L.kw, st), "partition k");
      RIB_LAUNCH(launch_partition(g, es, v, L.vw, st), "partition v");
      RIB_LAUNCH(launch_partition(g, es, d_o, L.dow, st), "partition do");
      RIB_LAUNCH(launch_pack_pos(g.N, g.n_rows, g.r, rp, es, q_p, es, L.qp, st), "pack q_p");
      RIB_LAUNCH(launch_pack_pos(g.N, g.n_rows, g.r, rp, es, k_p, es, L.kp, st), "pack k_p");
      t_part.end();
      TimedGroup t_prep(RIB_KERNEL_BWD_PREP, st);
      RIB_LAUNCH(launch_bwd_prep(g, es, o, d_o, lse, L.dd, L.lse2, st), "bwd prep");
      t_prep.end();
    }
    BwdArgs a;
    a.g = g;
    a.scale = resolve_scale(scale, shape);
    a.c = a.scale * kLog2e;
    a.rp = rp;
    a.qw = L.qw; a.kw = L.kw; a.vw = L.vw; a.dow = L.dow;
    a.qp = L.qp; a.kp = L.kp;
    a.lse2 = L.lse2; a.dd = L.dd;
    a.dqw = L.dqw; a.dkw = L.dkw; a.dvw = L.dvw;
    a.dq_map = dq_c; a.dk_map = dk_c; a.dv_map = dv;
    if (mapkv_path(g, dtype)) { a.k_map = k_c; a.v_map = v; }
    a.dqp_part = L.dqp_part; a.dkp_part = L.dkp_part;
    {
      TimedGroup t_dkv(RIB_KERNEL_ATTN_BWD_DKV, st);
      RIB_LAUNCH(bf ? launch_attn_bwd_dkv_bf16(a, st) : launch_attn_bwd_dkv_simple(a, es, st),
                 "attention backward dK/dV");
      t_dkv.end();
      TimedGroup t_dq(RIB_KERNEL_ATTN_BWD_DQ, st);
      RIB_LAUNCH(bf ? launch_attn_bwd_dq_bf16(a, st) : launch_attn_bwd_dq_simple(a, es, st), "attention backward dQ");
      t_dq.end();
    }
    TimedGroup t_red(RIB_KERNEL_POS_REDUCE, st);
    RIB_LAUNCH(launch_reduce_pos_grads(g.units, g.N, g.n_rows, g.r, rp, L.dqp_part, dq_p, L.dkp_part, dk_p, st),
               "reduce dq_p, dk_p");
    t_red.end();
    if (!bf) {
      TimedGroup t_unp(RIB_KERNEL_UNPARTITION, st);
      RIB_LAUNCH(launch_unpartition(g, es, L.dqw, dq_c, st), "unpartition dq");
      RIB_LAUNCH(launch_unpartition(g, es, L.dkw, dk_c, st), "unpartition dk");
      RIB_LAUNCH(launch_unpartition(g, es, L.dvw, dv, st), "unpartition dv");
      t_unp.end();
    }
#undef RIB_LAUNCH
    return ok();
  } catch (...) {
    return fail(RIB_ERR_HIP, "unexpected C++ exception in rib_window_attn_bwd");
  }
}

}  // extern "C"
