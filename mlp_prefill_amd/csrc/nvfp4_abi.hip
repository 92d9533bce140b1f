// C ABI of libnvfp4.so: host-side validation, workspace sizing and dispatch.
// Every check happens before anything is enqueued; the calls never
// synchronise, copy, allocate or read device memory on the host.
#include "nvfp4.h"

#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "internal.h"

namespace nvfp4 {

static std::atomic<uint64_t> g_launches{0};

// Timing window: at most one open at a time.  `active` is read on every
// launch without the lock; the event pool only changes under the lock.
struct Timing {
  std::mutex mu;
  std::atomic<int> active{-1};
  std::vector<hipEvent_t> ev;  // [start, end] per slot
  int64_t used = 0, dropped = 0, cap = 0;
  bool record_failed = false;
};
static Timing g_timing;

int launch_begin(int kc, hipStream_t st) {
  if (g_timing.active.load(std::memory_order_acquire) != kc) return -1;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (g_timing.active.load(std::memory_order_relaxed) != kc) return -1;
  if (g_timing.used >= g_timing.cap) {
    ++g_timing.dropped;
    return -1;
  }
  const int slot = (int)g_timing.used++;
  if (hipEventRecord(g_timing.ev[2 * slot], st) != hipSuccess) g_timing.record_failed = true;
  return slot;
}

void launch_end(int slot, hipStream_t st) {
  g_launches.fetch_add(1, std::memory_order_relaxed);
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (hipEventRecord(g_timing.ev[2 * slot + 1], st) != hipSuccess) g_timing.record_failed = true;
}

}  // namespace nvfp4

namespace {

using nvfp4::Operand;

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 unusable

// The current device must be a gfx950.  The first call per device reads its
// properties; later calls only ask which device is current.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return NVFP4_ERR_DEVICE;
  }
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return NVFP4_ERR_DEVICE;
    }
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? NVFP4_OK : NVFP4_ERR_DEVICE;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_tensor(const nvfp4_tensor& t) {
  if (!t.codes || !t.scales || !t.gscale) return NVFP4_ERR_NULL;
  if (!aligned(t.codes, 16) || !aligned(t.scales, 16) || !aligned(t.gscale, 4)) return NVFP4_ERR_ALIGN;
  if (t.tiled && !aligned(t.tiled, 256)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

Operand op(const nvfp4_tensor& t) { return Operand{t.codes, t.scales, t.gscale, t.tiled}; }

// Workspace bookkeeping: returns NVFP4_OK and sets *is_query when the call is
// a size query; NVFP4_ERR_WORKSPACE when the given workspace is too small.
int workspace(void* ws, size_t* ws_bytes, size_t need, bool* is_query) {
  *is_query = false;
  if (ws == nullptr && ws_bytes != nullptr) {
    *ws_bytes = need;
    *is_query = true;
    return NVFP4_OK;
  }
  const size_t have = ws_bytes ? *ws_bytes : 0;
  if (need > 0 && (ws == nullptr || have < need)) return NVFP4_ERR_WORKSPACE;
  if (need > 0 && !aligned(ws, 256)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

int elem_size(int dtype) { return dtype == NVFP4_BF16 ? 2 : 4; }
bool dtype_ok(int dtype) { return dtype == NVFP4_F32 || dtype == NVFP4_BF16; }

}  // namespace

extern "C" {

const char* nvfp4_strerror(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid shape";
    case NVFP4_ERR_ALIGN: return "misaligned pointer or row stride";
    case NVFP4_ERR_WORKSPACE: return "workspace too small";
    case NVFP4_ERR_ARG: return "invalid argument";
    case NVFP4_ERR_DEVICE: return "no usable gfx950 device";
    case NVFP4_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

uint64_t nvfp4_launch_count(void) { return nvfp4::g_launches.load(std::memory_order_relaxed); }

int nvfp4_timing_begin(int kernel_class, int64_t max_launches) {
  using nvfp4::g_timing;
  if (kernel_class < 0 || kernel_class >= nvfp4::KC_COUNT) return NVFP4_ERR_ARG;
  if (max_launches <= 0 || max_launches > NVFP4_TIMING_MAX_LAUNCHES) return NVFP4_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (g_timing.active.load(std::memory_order_relaxed) >= 0) return NVFP4_ERR_ARG;
  g_timing.ev.assign((size_t)(2 * max_launches), nullptr);
  for (auto& e : g_timing.ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      (void)hipGetLastError();
      for (auto& d : g_timing.ev)
        if (d) (void)hipEventDestroy(d);
      g_timing.ev.clear();
      return NVFP4_ERR_LAUNCH;
    }
  }
  g_timing.used = g_timing.dropped = 0;
  g_timing.cap = max_launches;
  g_timing.record_failed = false;
  g_timing.active.store(kernel_class, std::memory_order_release);
  return NVFP4_OK;
}

int nvfp4_timing_end(int64_t* launches, int64_t* dropped, double* total_ms) {
  using nvfp4::g_timing;
  if (!launches || !dropped || !total_ms) return NVFP4_ERR_NULL;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (g_timing.active.load(std::memory_order_relaxed) < 0) return NVFP4_ERR_ARG;
  g_timing.active.store(-1, std::memory_order_release);
  int status = g_timing.record_failed ? NVFP4_ERR_LAUNCH : NVFP4_OK;
  double sum = 0.0;
  for (int64_t i = 0; i < g_timing.used && status == NVFP4_OK; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_timing.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]) != hipSuccess) {
      (void)hipGetLastError();
      status = NVFP4_ERR_LAUNCH;
    }
    sum += ms;
  }
  for (auto& e : g_timing.ev) (void)hipEventDestroy(e);
  g_timing.ev.clear();
  *launches = g_timing.used;
  *dropped = g_timing.dropped;
  *total_ms = sum;
  g_timing.used = g_timing.dropped = g_timing.cap = 0;
  return status;
}

int nvfp4_quantize_act(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x, nvfp4_tensor out,
                       int gs_mode, void* ws, size_t* ws_bytes, void* stream) {
  if (!dtype_ok(x_dtype) || (gs_mode != NVFP4_GS_COMPUTE && gs_mode != NVFP4_GS_GIVEN && gs_mode != NVFP4_GS_FROM_AMAX))
    return NVFP4_ERR_ARG;
  if (rows < 0 || cols < 0 || cols % 16 != 0 || ld_x < cols) return NVFP4_ERR_SHAPE;
  if (rows * (cols / 16) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  bool query;
  int rc;
  if (gs_mode == NVFP4_GS_FROM_AMAX) {
    // ws holds the given partial maxima: NVFP4_AMAX_SLOTS float32, 16-byte aligned
    static_assert(NVFP4_AMAX_SLOTS == nvfp4::kAmaxSlots, "slot count");
    query = false;
    if (ws == nullptr && ws_bytes != nullptr) {
      *ws_bytes = NVFP4_AMAX_SLOTS * sizeof(float);
      return NVFP4_OK;
    }
    if (ws == nullptr || ws_bytes == nullptr || *ws_bytes < NVFP4_AMAX_SLOTS * sizeof(float)) return NVFP4_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return NVFP4_ERR_ALIGN;
  } else {
    rc = workspace(ws, ws_bytes, nvfp4::quantize_ws_bytes(rows, cols, gs_mode), &query);
    if (rc != NVFP4_OK || query) return rc;
  }
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (!x) return NVFP4_ERR_NULL;
  if ((rc = check_tensor(out)) != NVFP4_OK) return rc;
  if (!aligned(x, 16) || (ld_x * elem_size(x_dtype)) % 16 != 0) return NVFP4_ERR_ALIGN;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  return nvfp4::quantize_launch(x, x_dtype, rows, cols, ld_x, out.codes, out.scales, out.gscale, gs_mode, ws,
                                reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_quantize_act_noalloc(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                               nvfp4_tensor out, int gs_mode, void* stream) {
  if (!dtype_ok(x_dtype) || (gs_mode != NVFP4_GS_COMPUTE && gs_mode != NVFP4_GS_GIVEN)) return NVFP4_ERR_ARG;
  if (rows < 0 || cols < 0 || cols % 16 != 0 || ld_x < cols) return NVFP4_ERR_SHAPE;
  if (rows * (cols / 16) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  // the scratch array replaces the workspace: it must hold what a workspace would
  if (nvfp4::quantize_ws_bytes(rows, cols, gs_mode) > nvfp4::quantize_scratch_bytes()) return NVFP4_ERR_WORKSPACE;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (!x) return NVFP4_ERR_NULL;
  int rc;
  if ((rc = check_tensor(out)) != NVFP4_OK) return rc;
  if (!aligned(x, 16) || (ld_x * elem_size(x_dtype)) % 16 != 0) return NVFP4_ERR_ALIGN;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  void* ws = nullptr;
  if (nvfp4::quantize_scratch(&ws) != 0) return NVFP4_ERR_DEVICE;
  return nvfp4::quantize_launch(x, x_dtype, rows, cols, ld_x, out.codes, out.scales, out.gscale, gs_mode, ws,
                                reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_rmsnorm_quantize_act(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                               const float* gamma, float eps, nvfp4_tensor out, void* ws, size_t* ws_bytes,
                               void* stream) {
  if (!dtype_ok(x_dtype)) return NVFP4_ERR_ARG;
  if (!(eps >= 0.0f) || !(eps <= 3.0e38f)) return NVFP4_ERR_ARG;   // finite and non-negative (NaN fails)
  if (rows < 0 || cols < 0 || cols % 16 != 0 || ld_x < cols) return NVFP4_ERR_SHAPE;
  if (rows * (cols / 16) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  bool query;
  int rc = workspace(ws, ws_bytes, rows > 0 && cols > 0 ? nvfp4::rmsnorm_quantize_ws_bytes(rows) : 0, &query);
  if (rc != NVFP4_OK || query) return rc;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (!x || !gamma) return NVFP4_ERR_NULL;
  if ((rc = check_tensor(out)) != NVFP4_OK) return rc;
  if (!aligned(x, 16) || (ld_x * elem_size(x_dtype)) % 16 != 0 || !aligned(gamma, 16)) return NVFP4_ERR_ALIGN;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  return nvfp4::rmsnorm_quantize_launch(x, x_dtype, rows, cols, ld_x, gamma, eps, out.codes, out.scales, out.gscale,
                                        ws, reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_gemm(nvfp4_tensor a, nvfp4_tensor b, int64_t M, int64_t N, int64_t K, void* c, int c_dtype,
               int64_t ldc, float* c_amax, void* ws, size_t* ws_bytes, void* stream) {
  if (!dtype_ok(c_dtype)) return NVFP4_ERR_ARG;
  if (M < 0 || N < 0 || K <= 0 || K % 128 != 0 || ldc < N) return NVFP4_ERR_SHAPE;
  if (M * (K / 16) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  bool query;
  int rc = workspace(ws, ws_bytes, (M > 0 && N > 0) ? nvfp4::store_ws_bytes(M, N, K, 1, false) : 0, &query);
  if (rc != NVFP4_OK || query) return rc;
  if (M == 0 || N == 0) return NVFP4_OK;
  if ((rc = check_tensor(a)) != NVFP4_OK || (rc = check_tensor(b)) != NVFP4_OK) return rc;
  if (!c) return NVFP4_ERR_NULL;
  if (!aligned(c, 16) || (ldc * elem_size(c_dtype)) % 16 != 0 || !aligned(c_amax, 16)) return NVFP4_ERR_ALIGN;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  return nvfp4::store_launch(op(a), nullptr, nullptr, 1, M, op(b), N, K, c, c_dtype == NVFP4_BF16, ldc, c_amax, ws,
                             reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_mlp_gu_act(nvfp4_tensor x, nvfp4_tensor w_gate, nvfp4_tensor w_up, int64_t T, int64_t K, int64_t I,
                     nvfp4_tensor h_out, void* ws, size_t* ws_bytes, void* stream) {
  if (T < 0 || K <= 0 || I <= 0 || K % 128 != 0 || I % 128 != 0) return NVFP4_ERR_SHAPE;
  if (T * (I / 16) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  bool query;
  int rc = workspace(ws, ws_bytes, T > 0 ? nvfp4::glu_ws_bytes(T, I, K, 1, false) : 0, &query);
  if (rc != NVFP4_OK || query) return rc;
  if (T == 0) return NVFP4_OK;
  if ((rc = check_tensor(x)) != NVFP4_OK || (rc = check_tensor(w_gate)) != NVFP4_OK ||
      (rc = check_tensor(w_up)) != NVFP4_OK || (rc = check_tensor(h_out)) != NVFP4_OK)
    return rc;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  return nvfp4::glu_launch(op(x), nullptr, nullptr, 1, T, op(w_gate), op(w_up), I, K, h_out.codes, h_out.scales,
                           h_out.gscale, ws, reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_mlp_down(nvfp4_tensor h, nvfp4_tensor w_down, int64_t T, int64_t I, int64_t K, void* y, int y_dtype,
                   int64_t ldy, float* y_amax, void* ws, size_t* ws_bytes, void* stream) {
  if (!dtype_ok(y_dtype)) return NVFP4_ERR_ARG;
  if (T < 0 || I <= 0 || K <= 0 || I % 128 != 0 || ldy < K) return NVFP4_ERR_SHAPE;
  if (T * (I / 16) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  bool query;
  int rc = workspace(ws, ws_bytes, T > 0 ? nvfp4::store_ws_bytes(T, K, I, 1, false) : 0, &query);
  if (rc != NVFP4_OK || query) return rc;
  if (T == 0) return NVFP4_OK;
  if ((rc = check_tensor(h)) != NVFP4_OK || (rc = check_tensor(w_down)) != NVFP4_OK) return rc;
  if (!y) return NVFP4_ERR_NULL;
  if (!aligned(y, 16) || (ldy * elem_size(y_dtype)) % 16 != 0 || !aligned(y_amax, 16)) return NVFP4_ERR_ALIGN;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  return nvfp4::store_launch(op(h), nullptr, nullptr, 1, T, op(w_down), K, I, y, y_dtype == NVFP4_BF16, ldy, y_amax,
                             ws, reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_mlp_gu_act_static(nvfp4_tensor x, nvfp4_tensor w_gate, nvfp4_tensor w_up, int64_t T, int64_t K, int64_t I,
                            nvfp4_tensor h_out, void* ws, size_t* ws_bytes, void* stream) {
  if (T < 0 || K <= 0 || I <= 0 || K % 128 != 0 || I % 128 != 0) return NVFP4_ERR_SHAPE;
  if (T * (I / 16) >= ((int64_t)1 << 31) || T * (K / 16) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  bool query;
  int rc = workspace(ws, ws_bytes, T > 0 ? nvfp4::glu_static_ws_bytes(T, I, K, false) : 0, &query);
  if (rc != NVFP4_OK || query) return rc;
  if (T == 0) return NVFP4_OK;
  if ((rc = check_tensor(x)) != NVFP4_OK || (rc = check_tensor(w_gate)) != NVFP4_OK ||
      (rc = check_tensor(w_up)) != NVFP4_OK || (rc = check_tensor(h_out)) != NVFP4_OK)
    return rc;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  return nvfp4::glu_static_launch(op(x), nullptr, nullptr, 1, T, op(w_gate), op(w_up), I, K, h_out.codes,
                                  h_out.scales, h_out.gscale, ws, reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_mlp_down_quant(nvfp4_tensor h, nvfp4_tensor w_down, int64_t T, int64_t I, int64_t K, nvfp4_tensor y_out,
                         void* ws, size_t* ws_bytes, void* stream) {
  if (T < 0 || I <= 0 || K <= 0 || I % 128 != 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (T * (I / 16) >= ((int64_t)1 << 31) || T * (K / 16) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  bool query;
  int rc = workspace(ws, ws_bytes, T > 0 ? nvfp4::store_ws_bytes(T, K, I, 1, false) : 0, &query);
  if (rc != NVFP4_OK || query) return rc;
  if (T == 0) return NVFP4_OK;
  if ((rc = check_tensor(h)) != NVFP4_OK || (rc = check_tensor(w_down)) != NVFP4_OK ||
      (rc = check_tensor(y_out)) != NVFP4_OK)
    return rc;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  return nvfp4::store_quant_launch(op(h), T, op(w_down), K, I, y_out.codes, y_out.scales, y_out.gscale, ws,
                                   reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_mlp(const void* x, int x_dtype, int64_t ld_x, const float* x_amax, int64_t T, int64_t K, int64_t I,
              nvfp4_tensor w_gate, nvfp4_tensor w_up, nvfp4_tensor w_down, nvfp4_tensor x_q, nvfp4_tensor h_q,
              void* y, int y_dtype, int64_t ldy, float* y_amax, void* ws, size_t* ws_bytes, void* stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return NVFP4_ERR_ARG;
  if (x_amax != nullptr && x_amax == y_amax) return NVFP4_ERR_ARG;   // read and cleared by the same launch
  if (T < 0 || K <= 0 || I <= 0 || K % 128 != 0 || I % 128 != 0 || ld_x < K || ldy < K) return NVFP4_ERR_SHAPE;
  if (T * (I / 16) >= ((int64_t)1 << 31) || T * (K / 16) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  bool query;
  int rc = workspace(ws, ws_bytes, T > 0 ? nvfp4::mlp_ws_bytes(T, K, I) : 0, &query);
  if (rc != NVFP4_OK || query) return rc;
  if (T == 0) return NVFP4_OK;
  if (!x || !y) return NVFP4_ERR_NULL;
  if ((rc = check_tensor(w_gate)) != NVFP4_OK || (rc = check_tensor(w_up)) != NVFP4_OK ||
      (rc = check_tensor(w_down)) != NVFP4_OK || (rc = check_tensor(x_q)) != NVFP4_OK ||
      (rc = check_tensor(h_q)) != NVFP4_OK)
    return rc;
  if (!aligned(x, 16) || (ld_x * elem_size(x_dtype)) % 16 != 0 || !aligned(y, 16) ||
      (ldy * elem_size(y_dtype)) % 16 != 0 || !aligned(x_amax, 16) || !aligned(y_amax, 16))
    return NVFP4_ERR_ALIGN;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  return nvfp4::mlp_launch(x, x_dtype, ld_x, T, K, I, op(w_gate), op(w_up), op(w_down), x_q.codes, x_q.scales,
                           x_q.gscale, h_q.codes, h_q.scales, h_q.gscale, y, y_dtype == NVFP4_BF16, ldy, x_amax, y_amax,
                           ws, reinterpret_cast<hipStream_t>(stream));
}

// Shared by the two one-call expert MLPs: argument checks and the workspace
// query; NVFP4_OK with *go set when the launch should run.
static int moe_mlp_checks(const void* x, int x_dtype, int64_t ld_x, int64_t T, int64_t K, int64_t I, int E,
                          const int32_t* a_rows, const int32_t* group_offsets, int64_t M, const nvfp4_tensor& w_gate,
                          const nvfp4_tensor& w_up, const nvfp4_tensor& w_down, const nvfp4_tensor& x_q,
                          const nvfp4_tensor& h_q, void* y_slots, int y_dtype, int64_t ld_y, void* ws,
                          size_t* ws_bytes, size_t need, bool* go) {
  *go = false;
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return NVFP4_ERR_ARG;
  if (E < 1 || E > 4096) return NVFP4_ERR_ARG;
  if (T < 0 || M < 0 || K <= 0 || I <= 0 || K % 128 != 0 || I % 128 != 0 || ld_x < K || ld_y < K)
    return NVFP4_ERR_SHAPE;
  if (M * (I / 16) >= ((int64_t)1 << 31) || M * (K / 16) >= ((int64_t)1 << 31) ||
      T * (K / 16) >= ((int64_t)1 << 31) || T * K * 2 >= ((int64_t)1 << 31))
    return NVFP4_ERR_SHAPE;
  bool query;
  int rc = workspace(ws, ws_bytes, T > 0 && M > 0 ? need : 0, &query);
  if (rc != NVFP4_OK || query) return rc;
  if (T == 0 || M == 0) return NVFP4_OK;
  if (!x || !y_slots || !a_rows || !group_offsets) return NVFP4_ERR_NULL;
  if ((rc = check_tensor(w_gate)) != NVFP4_OK || (rc = check_tensor(w_up)) != NVFP4_OK ||
      (rc = check_tensor(w_down)) != NVFP4_OK || (rc = check_tensor(x_q)) != NVFP4_OK ||
      (rc = check_tensor(h_q)) != NVFP4_OK)
    return rc;
  if (!aligned(x, 16) || (ld_x * elem_size(x_dtype)) % 16 != 0 || !aligned(y_slots, 16) ||
      (ld_y * elem_size(y_dtype)) % 16 != 0 || !aligned(a_rows, 4) || !aligned(group_offsets, 4))
    return NVFP4_ERR_ALIGN;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  *go = true;
  return NVFP4_OK;
}

int nvfp4_moe_mlp(const void* x, int x_dtype, int64_t ld_x, int64_t T, int64_t K, int64_t I, int E,
                  const int32_t* a_rows, const int32_t* group_offsets, int64_t M, nvfp4_tensor w_gate,
                  nvfp4_tensor w_up, nvfp4_tensor w_down, nvfp4_tensor x_q, nvfp4_tensor h_q, void* y_slots,
                  int y_dtype, int64_t ld_y, void* ws, size_t* ws_bytes, void* stream) {
  bool go;
  const size_t need = T > 0 && M > 0 && K > 0 && I > 0 ? nvfp4::moe_mlp_ws_bytes(T, K, I, E, M) : 0;
  int rc = moe_mlp_checks(x, x_dtype, ld_x, T, K, I, E, a_rows, group_offsets, M, w_gate, w_up, w_down, x_q, h_q,
                          y_slots, y_dtype, ld_y, ws, ws_bytes, need, &go);
  if (rc != NVFP4_OK || !go) return rc;
  return nvfp4::moe_mlp_launch(x, x_dtype, ld_x, T, K, I, E, a_rows, group_offsets, M, op(w_gate), op(w_up),
                               op(w_down), x_q.codes, x_q.scales, x_q.gscale, h_q.codes, h_q.scales, h_q.gscale,
                               y_slots, y_dtype == NVFP4_BF16, ld_y, ws, reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_moe_mlp_static(const void* x, int x_dtype, int64_t ld_x, int64_t T, int64_t K, int64_t I, int E,
                         const int32_t* a_rows, const int32_t* group_offsets, int64_t M, nvfp4_tensor w_gate,
                         nvfp4_tensor w_up, nvfp4_tensor w_down, nvfp4_tensor x_q, nvfp4_tensor h_q, void* y_slots,
                         int y_dtype, int64_t ld_y, void* ws, size_t* ws_bytes, void* stream) {
  bool go;
  const size_t need = T > 0 && M > 0 && K > 0 && I > 0 ? nvfp4::moe_mlp_static_ws_bytes(T, K, I, E, M) : 0;
  int rc = moe_mlp_checks(x, x_dtype, ld_x, T, K, I, E, a_rows, group_offsets, M, w_gate, w_up, w_down, x_q, h_q,
                          y_slots, y_dtype, ld_y, ws, ws_bytes, need, &go);
  if (rc != NVFP4_OK || !go) return rc;
  return nvfp4::moe_mlp_static_launch(x, x_dtype, ld_x, T, K, I, E, a_rows, group_offsets, M, op(w_gate),
                                      op(w_up), op(w_down), x_q.codes, x_q.scales, x_q.gscale, h_q.codes,
                                      h_q.scales, h_q.gscale, y_slots, y_dtype == NVFP4_BF16, ld_y, ws,
                                      reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_moe_route(const float* logits, int64_t T, int E, int k, int64_t ld, int32_t* group_offsets,
                    int32_t* a_rows, int32_t* slot_of, float* weights, void* ws, size_t* ws_bytes, void* stream) {
  if (E < 1 || E > nvfp4::kMaxExperts || k < 1 || k > nvfp4::kMaxTopK || k > E) return NVFP4_ERR_ARG;
  if (T < 0 || ld < E) return NVFP4_ERR_SHAPE;
  if (T * k >= ((int64_t)1 << 31) || T * ld >= ((int64_t)1 << 40)) return NVFP4_ERR_SHAPE;
  bool query;
  int rc = workspace(ws, ws_bytes, T > 0 ? nvfp4::route_ws_bytes(T, E, k) : 0, &query);
  if (rc != NVFP4_OK || query) return rc;
  if (T == 0) return NVFP4_OK;
  if (!logits || !group_offsets || !a_rows || !slot_of || !weights) return NVFP4_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(group_offsets, 4) || !aligned(a_rows, 4) || !aligned(slot_of, 4) ||
      !aligned(weights, 4))
    return NVFP4_ERR_ALIGN;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  return nvfp4::route_launch(logits, T, E, k, ld, group_offsets, a_rows, slot_of, weights, ws,
                             reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_moe_combine(const void* y_slots, int slots_dtype, int64_t ld_slots, const int32_t* slot_of,
                      const float* weights, int64_t T, int k, int64_t N, void* y, int y_dtype, int64_t ldy,
                      void* stream) {
  if (!dtype_ok(slots_dtype) || !dtype_ok(y_dtype) || k < 1 || k > nvfp4::kMaxTopK) return NVFP4_ERR_ARG;
  if (T < 0 || N < 0 || N % 8 != 0 || ld_slots < N || ldy < N) return NVFP4_ERR_SHAPE;
  if (T == 0 || N == 0) return NVFP4_OK;
  if (!y_slots || !slot_of || !weights || !y) return NVFP4_ERR_NULL;
  if (!aligned(y_slots, 16) || !aligned(y, 16) || (ld_slots * elem_size(slots_dtype)) % 16 != 0 ||
      (ldy * elem_size(y_dtype)) % 16 != 0 || !aligned(slot_of, 4) || !aligned(weights, 4))
    return NVFP4_ERR_ALIGN;
  int rc;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  return nvfp4::combine_launch(y_slots, slots_dtype == NVFP4_BF16, ld_slots, slot_of, weights, T, k, N, y,
                               y_dtype == NVFP4_BF16, ldy, reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_tile_weight(nvfp4_tensor w, int64_t experts, int64_t N, int64_t K, uint8_t* tiled,
                      size_t* tiled_bytes, void* stream) {
  if (experts < 1 || experts > 4096) return NVFP4_ERR_ARG;
  if (N < 0 || K <= 0 || K % 128 != 0) return NVFP4_ERR_SHAPE;
  // the contractions address one expert's copy with 32-bit offsets
  if (nvfp4::tile_weight_bytes(1, N, K) >= ((size_t)1 << 31)) return NVFP4_ERR_SHAPE;
  bool query;
  const size_t need = nvfp4::tile_weight_bytes(experts, N, K);
  int rc = workspace(tiled, tiled_bytes, need, &query);
  if (rc != NVFP4_OK || query) return rc;
  if (N == 0) return NVFP4_OK;
  if (!w.codes || !w.scales) return NVFP4_ERR_NULL;
  if (!aligned(w.codes, 16) || !aligned(w.scales, 16)) return NVFP4_ERR_ALIGN;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  return nvfp4::tile_weight_launch(w.codes, w.scales, experts, N, K, tiled, reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_grouped_gemm(nvfp4_tensor a, const int32_t* a_rows, const int32_t* group_offsets, int E, int64_t M,
                       nvfp4_tensor w0, nvfp4_tensor w1, int64_t N, int64_t K, int epilogue, void* out,
                       int out_dtype, int64_t ld_out, nvfp4_tensor out_q, void* ws, size_t* ws_bytes,
                       void* stream) {
  const bool gluq = (epilogue == NVFP4_EPI_SILU_MUL_QUANT_GIVEN);
  const bool glu = (epilogue == NVFP4_EPI_SILU_MUL_REQUANT) || gluq;
  if (epilogue != NVFP4_EPI_STORE && !glu) return NVFP4_ERR_ARG;
  if (!glu && !dtype_ok(out_dtype)) return NVFP4_ERR_ARG;
  if (E < 1 || E > 4096) return NVFP4_ERR_ARG;
  if (M < 0 || N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0) return NVFP4_ERR_SHAPE;
  if (!glu && ld_out < N) return NVFP4_ERR_SHAPE;
  if (M * (N / 16) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  if (M * (K / 16) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  bool query;
  const size_t need = M == 0 ? 0
                              : gluq ? nvfp4::glu_static_ws_bytes(M, N, K, true)
                              : glu  ? nvfp4::glu_ws_bytes(M, N, K, E, true)
                                     : nvfp4::store_ws_bytes(M, N, K, E, true);
  int rc = workspace(ws, ws_bytes, need, &query);
  if (rc != NVFP4_OK || query) return rc;
  if (M == 0) return NVFP4_OK;
  if (!group_offsets) return NVFP4_ERR_NULL;
  if ((rc = check_tensor(a)) != NVFP4_OK || (rc = check_tensor(w0)) != NVFP4_OK) return rc;
  if (glu) {
    if ((rc = check_tensor(w1)) != NVFP4_OK || (rc = check_tensor(out_q)) != NVFP4_OK) return rc;
  } else {
    if (!out) return NVFP4_ERR_NULL;
    if (!aligned(out, 16) || (ld_out * elem_size(out_dtype)) % 16 != 0) return NVFP4_ERR_ALIGN;
  }
  if (!aligned(group_offsets, 4) || (a_rows && !aligned(a_rows, 4))) return NVFP4_ERR_ALIGN;
  if ((rc = check_device()) != NVFP4_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!glu)
    return nvfp4::store_launch(op(a), a_rows, group_offsets, E, M, op(w0), N, K, out, out_dtype == NVFP4_BF16,
                               ld_out, nullptr, ws, st);
  if (gluq)
    return nvfp4::glu_static_launch(op(a), a_rows, group_offsets, E, M, op(w0), op(w1), N, K, out_q.codes,
                                    out_q.scales, out_q.gscale, ws, st);
  return nvfp4::glu_launch(op(a), a_rows, group_offsets, E, M, op(w0), op(w1), N, K, out_q.codes, out_q.scales,
                           out_q.gscale, ws, st);
}

}  // extern "C"
