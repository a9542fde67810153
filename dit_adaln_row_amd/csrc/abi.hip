// C-ABI entry points of libditnorm.so (declared in include/ditnorm.h; the
// measurement copy in include/ditnorm_measure.h).
//
// Every entry point validates its arguments on the host first -- sizes,
// alignment, aliasing -- and only then touches HIP: it looks up the current
// device (checked once per device to be gfx950), fills the kernel argument
// block and enqueues the work on the caller's stream (one kernel; the
// backward one kernel per tree level more).  There is no
// fallback path: anything the kernels do not implement is reported as
// DITNORM_UNSUPPORTED.
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/ditnorm.h"
#include "../../include/ditnorm_measure.h"
#include "launch.hpp"

using namespace ditnorm;

// Scratch memory of ln_modulate_backward_noalloc: the partial token sums that
// ln_modulate_backward keeps in the caller's workspace.  Every device the
// library runs on holds one copy, loaded with the library's code object and
// kept until the process ends.  In host code this name is only a host-side
// stand-in: its device address on each device comes from hipGetSymbolAddress
// (scratch_address below), and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[DITNORM_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 unsupported
DeviceInfo g_dev_info[kMaxDevices];
std::mutex g_dev_mu;

int device_error(hipError_t e) {
  g_last_hip_error = (int)e;
  return DITNORM_DEVICE_ERROR;
}

// Current device, verified to be gfx950 (cached per device).
int current_device(DeviceInfo *out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_error(e);
  if (dev < 0 || dev >= kMaxDevices) return DITNORM_DEVICE_ERROR;
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
      hipDeviceProp_t prop;
      e = hipGetDeviceProperties(&prop, dev);
      if (e != hipSuccess) return device_error(e);
      const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
      g_dev_info[dev].num_cu = prop.multiProcessorCount;
      g_dev_info[dev].device = dev;
      st = ok ? 1 : 2;
      g_dev_state[dev].store(st, std::memory_order_release);
    }
  }
  if (st != 1) return DITNORM_DEVICE_ERROR;
  *out = g_dev_info[dev];
  return DITNORM_OK;
}

// Device address of `scratch` on the current device `dev`, looked up once per
// device (with that device current) and kept.
void *g_scratch_ptr[kMaxDevices];
std::atomic<int> g_scratch_state[kMaxDevices];  // 0 not looked up, 1 g_scratch_ptr valid

int scratch_address(int dev, char **out) {
  if (g_scratch_state[dev].load(std::memory_order_acquire) == 0) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_scratch_state[dev].load(std::memory_order_relaxed) == 0) {
      void *p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return device_error(e);
      if (p == nullptr || ((uintptr_t)p & 255u) != 0) return DITNORM_DEVICE_ERROR;
      g_scratch_ptr[dev] = p;
      g_scratch_state[dev].store(1, std::memory_order_release);
    }
  }
  *out = (char *)g_scratch_ptr[dev];
  return DITNORM_OK;
}

int finish(hipError_t e) {
  if (e != hipSuccess) return device_error(e);
  return DITNORM_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

bool eps_ok(float eps) { return std::isfinite(eps) && eps >= 0.0f; }

// A memory range [p, p + bytes) of one argument.
struct Buf {
  const void *p;
  int64_t bytes;
};

bool overlap(const Buf &a, const Buf &b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + (uintptr_t)a.bytes;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + (uintptr_t)b.bytes;
  return a0 < b1 && b0 < a1;
}

bool same(const Buf &a, const Buf &b) { return a.p == b.p && a.bytes == b.bytes; }

// Outputs must not overlap each other, nor any input -- except that output i
// may coincide exactly with input in_alias[i] (in-place forms).
template <int NI, int NO>
bool aliasing_ok(const Buf (&in)[NI], const Buf (&out)[NO], const int (&in_alias)[NO]) {
  for (int i = 0; i < NO; ++i) {
    for (int j = i + 1; j < NO; ++j)
      if (overlap(out[i], out[j])) return false;
    for (int j = 0; j < NI; ++j) {
      if (!overlap(out[i], in[j])) continue;
      if (in_alias[i] == j && same(out[i], in[j])) continue;
      return false;
    }
  }
  return true;
}

// Bytes spanned by B modulation rows of `cols` bf16 values at row stride `stride`.
int64_t mod_bytes(int64_t nb, int64_t stride, int64_t cols) {
  return ((nb - 1) * stride + cols) * 2;
}

// Shared checks of the row entry points.  Returns a status; DITNORM_OK
// means "valid and supported".
int check_rows(int64_t rows, int64_t cols, int64_t rows_per_batch, int64_t mod_batch_stride,
               float eps) {
  if (rows < 0 || cols <= 0 || rows_per_batch <= 0 || mod_batch_stride < cols || !eps_ok(eps))
    return DITNORM_INVALID_ARGUMENT;
  if (rows % rows_per_batch != 0) return DITNORM_INVALID_ARGUMENT;
  if (cols % 8 != 0 || cols > DITNORM_MAX_COLS || rows > DITNORM_MAX_ROWS ||
      mod_batch_stride > DITNORM_MAX_MOD_STRIDE)
    return DITNORM_UNSUPPORTED;
  const int64_t nb = rows / rows_per_batch;
  if (nb > 1 && mod_batch_stride % 8 != 0) return DITNORM_UNSUPPORTED;
  return DITNORM_OK;
}

// ---- per-entry validation (no HIP calls) -----------------------------------

int validate_ln(const void *x, const void *scale, const void *shift, const void *out,
                int64_t rows, int64_t cols, int64_t rpb, int64_t mbs, float eps,
                const float *mean_out, const float *rstd_out, const void *y_out) {
  int st = check_rows(rows, cols, rpb, mbs, eps);
  if (st != DITNORM_OK || rows == 0) return st;
  if (!x || !scale || !shift || !out) return DITNORM_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(scale) || !aligned16(shift) || !aligned16(out) ||
      !aligned16(y_out) || !aligned4(mean_out) || !aligned4(rstd_out))
    return DITNORM_UNSUPPORTED;
  const int64_t act = rows * cols * 2, nb = rows / rpb;
  const Buf in[] = {{x, act}, {scale, mod_bytes(nb, mbs, cols)}, {shift, mod_bytes(nb, mbs, cols)}};
  const Buf o[] = {{out, act}, {y_out, act}, {mean_out, rows * 4}, {rstd_out, rows * 4}};
  const int alias[] = {0, -1, -1, -1};
  return aliasing_ok(in, o, alias) ? DITNORM_OK : DITNORM_UNSUPPORTED;
}

int validate_gated_ln(const void *x, const void *residual, const void *gate, const void *scale,
                      const void *shift, const void *residual_out, const void *out, int64_t rows,
                      int64_t cols, int64_t rpb, int64_t mbs, float eps, const float *mean_out,
                      const float *rstd_out, const void *y_out) {
  int st = check_rows(rows, cols, rpb, mbs, eps);
  if (st != DITNORM_OK || rows == 0) return st;
  if (!x || !residual || !gate || !scale || !shift || !residual_out || !out)
    return DITNORM_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(residual) || !aligned16(gate) || !aligned16(scale) ||
      !aligned16(shift) || !aligned16(residual_out) || !aligned16(out) || !aligned16(y_out) ||
      !aligned4(mean_out) || !aligned4(rstd_out))
    return DITNORM_UNSUPPORTED;
  const int64_t act = rows * cols * 2, nb = rows / rpb, mb = mod_bytes(nb, mbs, cols);
  const Buf in[] = {{x, act}, {residual, act}, {gate, mb}, {scale, mb}, {shift, mb}};
  const Buf o[] = {{residual_out, act}, {out, act}, {y_out, act}, {mean_out, rows * 4},
                   {rstd_out, rows * 4}};
  const int alias[] = {1, -1, -1, -1, -1};
  return aliasing_ok(in, o, alias) ? DITNORM_OK : DITNORM_UNSUPPORTED;
}

int validate_rms(const void *x, const void *weight, const void *scale, const void *shift,
                 const void *out, const void *residual, const void *gate,
                 const void *residual_out, int64_t rows, int64_t cols, int64_t rpb, int64_t mbs,
                 float eps, const float *rstd_out, const void *y_out) {
  int st = check_rows(rows, cols, rpb, mbs, eps);
  if (st != DITNORM_OK) return st;
  const int gated = residual != nullptr;
  if ((gate != nullptr) != gated || (residual_out != nullptr) != gated)
    return DITNORM_INVALID_ARGUMENT;
  if (rows == 0) return DITNORM_OK;
  if (!x || !weight || !scale || !shift || !out) return DITNORM_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(weight) || !aligned16(scale) || !aligned16(shift) ||
      !aligned16(out) || !aligned16(residual) || !aligned16(gate) || !aligned16(residual_out) ||
      !aligned16(y_out) || !aligned4(rstd_out))
    return DITNORM_UNSUPPORTED;
  const int64_t act = rows * cols * 2, nb = rows / rpb, mb = mod_bytes(nb, mbs, cols);
  const Buf in[] = {{x, act}, {weight, cols * 2}, {scale, mb}, {shift, mb},
                    {residual, gated ? act : 0}, {gate, gated ? mb : 0}};
  const Buf o[] = {{out, act}, {residual_out, gated ? act : 0}, {y_out, act},
                   {rstd_out, rows * 4}};
  // plain site: out may be x; gated site: residual_out may be residual
  const int alias[] = {gated ? -1 : 0, 4, -1, -1};
  return aliasing_ok(in, o, alias) ? DITNORM_OK : DITNORM_UNSUPPORTED;
}

int validate_qk(const void *q, const void *k, const void *q_out, const void *k_out,
                int64_t rows_q, int64_t rows_k, int64_t head_dim, float eps,
                const float *mean_out, const float *rstd_out) {
  if (rows_q < 0 || rows_k < 0 || head_dim <= 0 || !eps_ok(eps)) return DITNORM_INVALID_ARGUMENT;
  if (head_dim % 8 != 0 || head_dim > 128 || rows_q > DITNORM_MAX_ROWS ||
      rows_k > DITNORM_MAX_ROWS - rows_q)
    return DITNORM_UNSUPPORTED;
  if (rows_q + rows_k == 0) return DITNORM_OK;
  if (rows_q > 0 && (!q || !q_out)) return DITNORM_INVALID_ARGUMENT;
  if (rows_k > 0 && (!k || !k_out)) return DITNORM_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_out) || !aligned16(k_out) ||
      !aligned4(mean_out) || !aligned4(rstd_out))
    return DITNORM_UNSUPPORTED;
  const int64_t total = rows_q + rows_k;
  const int64_t rb = head_dim * 2;  // bytes per head row
  const Buf in[] = {{q, rows_q * rb}, {k, rows_k * rb}};
  const Buf o[] = {{q_out, rows_q * rb}, {k_out, rows_k * rb}, {mean_out, total * 4},
                   {rstd_out, total * 4}};
  const int alias[] = {0, 1, -1, -1};
  return aliasing_ok(in, o, alias) ? DITNORM_OK : DITNORM_UNSUPPORTED;
}

int validate_wan(const void *x, const float *bias, const float *gamma, const void *out,
                 int64_t rows, int64_t channels, float eps, const float *rstd_out,
                 const void *xb_out) {
  if (rows < 0 || channels <= 0 || !eps_ok(eps)) return DITNORM_INVALID_ARGUMENT;
  if (channels % 8 != 0 || channels > DITNORM_MAX_CHANNELS || rows > DITNORM_MAX_ROWS)
    return DITNORM_UNSUPPORTED;
  if (rows == 0) return DITNORM_OK;
  if (!x || !gamma || !out) return DITNORM_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(bias) || !aligned16(gamma) || !aligned16(out) ||
      !aligned16(xb_out) || !aligned4(rstd_out))
    return DITNORM_UNSUPPORTED;
  const int64_t act = rows * channels * 2;
  const Buf in[] = {{x, act}, {bias, channels * 4}, {gamma, channels * 4}};
  const Buf o[] = {{out, act}, {xb_out, act}, {rstd_out, rows * 4}};
  const int alias[] = {0, -1, -1};
  return aliasing_ok(in, o, alias) ? DITNORM_OK : DITNORM_UNSUPPORTED;
}

// Element size of a storage type, 0 if the code names none.
int64_t dtype_size(int dtype) {
  return dtype == DITNORM_DTYPE_BF16 || dtype == DITNORM_DTYPE_F16 ? 2
         : dtype == DITNORM_DTYPE_F32                              ? 4
                                                                   : 0;
}

int validate_epilogue(const void *x, const void *bias, const void *h, const void *out,
                      int64_t rows, int64_t channels, int dtype, int bias_dtype) {
  if (rows < 0 || channels <= 0 || dtype_size(dtype) == 0 || dtype_size(bias_dtype) == 0)
    return DITNORM_INVALID_ARGUMENT;
  // the bias is fp32 or of the activation's own type
  if (bias_dtype != DITNORM_DTYPE_F32 && bias_dtype != dtype) return DITNORM_UNSUPPORTED;
  const int64_t es = dtype_size(dtype);
  if (channels % 8 != 0 || channels > DITNORM_MAX_CHANNELS || rows > DITNORM_MAX_ROWS ||
      rows * (channels * es / 16) > DITNORM_MAX_VECTORS)
    return DITNORM_UNSUPPORTED;
  if (rows == 0) return DITNORM_OK;
  if (!x || !bias || !out) return DITNORM_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(bias) || !aligned16(h) || !aligned16(out))
    return DITNORM_UNSUPPORTED;
  const int64_t act = rows * channels * es;
  const Buf in[] = {{x, act}, {bias, channels * dtype_size(bias_dtype)}, {h, h ? act : 0}};
  const Buf o[] = {{out, act}};
  const int alias[] = {0};
  return aliasing_ok(in, o, alias) ? DITNORM_OK : DITNORM_UNSUPPORTED;
}

int validate_backward(const void *x, const void *scale, const void *d_out, const void *d_x,
                      const float *d_scale, const float *d_shift, int64_t rows, int64_t cols,
                      int64_t rpb, int64_t mbs, float eps, const void *ws, int64_t ws_bytes,
                      const float *mean_out, const float *rstd_out, int dtype,
                      bool lib_scratch = false) {
  if (dtype != DITNORM_DTYPE_BF16 && dtype != DITNORM_DTYPE_F32) return DITNORM_INVALID_ARGUMENT;
  int st = check_rows(rows, cols, rpb, mbs, eps);
  if (st != DITNORM_OK || rows == 0) return st;
  if (cols > (dtype == DITNORM_DTYPE_F32 ? DITNORM_MAX_BACKWARD_F32_COLS
                                         : DITNORM_MAX_BACKWARD_COLS))
    return DITNORM_UNSUPPORTED;
  if (!x || !scale || !d_out || !d_x || !d_scale || !d_shift) return DITNORM_INVALID_ARGUMENT;
  const BwdLayout L = bwd_layout(rows, cols, rpb, dtype);
  // one wavefront per row slot of the fused kernel's workgroups
  if ((rows / rpb) * L.chunks * L.rows_per_chunk > DITNORM_MAX_ROWS) return DITNORM_UNSUPPORTED;
  const int64_t need = L.bytes;
  if (lib_scratch) {
    ws = nullptr;  // a static array: it cannot overlap the caller's buffers
    ws_bytes = 0;
  } else if (need > 0 && (!ws || ws_bytes < need)) {
    return DITNORM_INVALID_ARGUMENT;
  }
  if (!aligned16(x) || !aligned16(scale) || !aligned16(d_out) || !aligned16(d_x) ||
      !aligned16(d_scale) || !aligned16(d_shift) || ((uintptr_t)ws & 255u) != 0 ||
      !aligned4(mean_out) || !aligned4(rstd_out))
    return DITNORM_UNSUPPORTED;
  const int64_t es = dtype_size(dtype), act = rows * cols * es, nb = rows / rpb;
  const Buf in[] = {{x, act}, {scale, mod_bytes(nb, mbs, cols) / 2 * es}, {d_out, act}};
  const Buf o[] = {{d_x, act}, {d_scale, nb * cols * 4}, {d_shift, nb * cols * 4},
                   {ws, need}, {mean_out, rows * 4}, {rstd_out, rows * 4}};
  const int alias[] = {-1, -1, -1, -1, -1, -1};
  if (!aliasing_ok(in, o, alias)) return DITNORM_UNSUPPORTED;
  if (lib_scratch && need > DITNORM_NOALLOC_SCRATCH_BYTES) return DITNORM_SCRATCH_EXCEEDED;
  return DITNORM_OK;
}

// The backward on validated arguments, its partial sums in `ws`.
int backward_launch(const void *x, const void *scale, const void *d_out, void *d_x,
                    float *d_scale, float *d_shift, int64_t rows, int64_t cols, int64_t rpb,
                    int64_t mbs, float eps, char *ws, float *mean_out, float *rstd_out,
                    int dtype, void *stream) {
  const BwdLayout L = bwd_layout(rows, cols, rpb, dtype);
  BwdArgs a{};
  a.x = x;
  a.scale = scale;
  a.d_out = d_out;
  a.d_x = d_x;
  a.dtype = dtype;
  a.d_scale = d_scale;
  a.d_shift = d_shift;
  a.mean_out = mean_out;
  a.rstd_out = rstd_out;
  a.rows = rows;
  a.rows_per_batch = rpb;
  a.mod_stride = mbs;
  a.cols = (int32_t)cols;
  a.eps = eps;
  return finish(launch_backward(a, L, (float *)(ws + L.part0_off), (float *)(ws + L.part1_off),
                                (hipStream_t)stream));
}

int validate_elementwise(int op, const void *a, const void *b, const void *m0, const void *m1,
                         const void *out, int64_t rows, int64_t cols, int64_t rpb, int64_t mbs,
                         int dtype) {
  if (dtype != DITNORM_DTYPE_BF16 && dtype != DITNORM_DTYPE_F16) return DITNORM_INVALID_ARGUMENT;
  int st = check_rows(rows, cols, rpb, mbs, 0.0f);
  if (st != DITNORM_OK || rows == 0) return st;
  if (rows * (cols / 8) > DITNORM_MAX_VECTORS) return DITNORM_UNSUPPORTED;
  if (!a || !m0 || !out || (op == 0 && !m1) || (op == 1 && !b)) return DITNORM_INVALID_ARGUMENT;
  if (!aligned16(a) || !aligned16(b) || !aligned16(m0) || !aligned16(m1) || !aligned16(out))
    return DITNORM_UNSUPPORTED;
  const int64_t act = rows * cols * 2, mb = mod_bytes(rows / rpb, mbs, cols);
  const Buf in[] = {{a, act}, {b, op == 1 ? act : 0}, {m0, mb}, {m1, op == 0 ? mb : 0}};
  const Buf o[] = {{out, act}};
  const int alias[] = {op == 0 ? 0 : 1};  // modulate: out may be x; gate add: out may be residual
  return aliasing_ok(in, o, alias) ? DITNORM_OK : DITNORM_UNSUPPORTED;
}

int launch_ew(int op, const void *a, const void *b, const void *m0, const void *m1, void *out,
              int64_t rows, int64_t cols, int64_t rpb, int64_t mbs, int dtype, void *stream) {
  int st = validate_elementwise(op, a, b, m0, m1, out, rows, cols, rpb, mbs, dtype);
  if (st != DITNORM_OK || rows == 0) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != DITNORM_OK) return st;
  ElementwiseArgs e{};
  e.a = (const uint16_t *)a;
  e.b = (const uint16_t *)b;
  e.m0 = (const uint16_t *)m0;
  e.m1 = (const uint16_t *)m1;
  e.out = (uint16_t *)out;
  e.rows = rows;
  e.cols = (int32_t)cols;
  e.rows_per_batch = rpb;
  e.mod_stride = mbs;
  return finish(launch_elementwise(e, op, dtype, dev, (hipStream_t)stream));
}

}  // namespace

// ===========================================================================
// exported
// ===========================================================================

extern "C" {

const char *ditnorm_status_string(int status) {
  switch (status) {
    case DITNORM_OK: return "DITNORM_OK";
    case DITNORM_INVALID_ARGUMENT: return "DITNORM_INVALID_ARGUMENT";
    case DITNORM_UNSUPPORTED: return "DITNORM_UNSUPPORTED";
    case DITNORM_DEVICE_ERROR: return "DITNORM_DEVICE_ERROR";
    case DITNORM_SCRATCH_EXCEEDED: return "DITNORM_SCRATCH_EXCEEDED";
    default: return "DITNORM_UNKNOWN_STATUS";
  }
}

int ditnorm_last_hip_error(void) { return g_last_hip_error; }

int ditnorm_version(void) { return 100; }

namespace {
int ln_common(const void *x, const void *scale, const void *shift, void *out, int64_t rows,
              int64_t cols, int64_t rows_per_batch, int64_t mod_batch_stride, float eps,
              float *mean_out, float *rstd_out, void *y_out, bool fold, void *stream) {
  int st = validate_ln(x, scale, shift, out, rows, cols, rows_per_batch, mod_batch_stride, eps,
                       mean_out, rstd_out, y_out);
  if (st != DITNORM_OK || rows == 0) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != DITNORM_OK) return st;
  RowArgs a{};
  a.x = (const uint16_t *)x;
  a.scale = (const uint16_t *)scale;
  a.shift = (const uint16_t *)shift;
  a.out = (uint16_t *)out;
  a.mean_out = mean_out;
  a.rstd_out = rstd_out;
  a.y_out = (uint16_t *)y_out;
  a.rows = rows;
  a.cols = (int32_t)cols;
  a.rows_per_batch = rows_per_batch;
  a.mod_stride = mod_batch_stride;
  a.eps = eps;
  return finish(launch_row(a, false, false, fold, dev, (hipStream_t)stream));
}
}  // namespace

int ln_modulate(const void *x, const void *scale, const void *shift, void *out, int64_t rows,
                int64_t cols, int64_t rows_per_batch, int64_t mod_batch_stride, float eps,
                float *mean_out, float *rstd_out, void *y_out, void *stream) {
  return ln_common(x, scale, shift, out, rows, cols, rows_per_batch, mod_batch_stride, eps,
                   mean_out, rstd_out, y_out, false, stream);
}

int ln_modulate_folded(const void *x, const void *scale, const void *shift, void *out,
                       int64_t rows, int64_t cols, int64_t rows_per_batch,
                       int64_t mod_batch_stride, float eps, float *mean_out, float *rstd_out,
                       void *stream) {
  return ln_common(x, scale, shift, out, rows, cols, rows_per_batch, mod_batch_stride, eps,
                   mean_out, rstd_out, nullptr, true, stream);
}

int gated_ln_modulate(const void *x, const void *residual, const void *gate, const void *scale,
                      const void *shift, void *residual_out, void *out, int64_t rows,
                      int64_t cols, int64_t rows_per_batch, int64_t mod_batch_stride, float eps,
                      float *mean_out, float *rstd_out, void *y_out, void *stream) {
  int st = validate_gated_ln(x, residual, gate, scale, shift, residual_out, out, rows, cols,
                             rows_per_batch, mod_batch_stride, eps, mean_out, rstd_out, y_out);
  if (st != DITNORM_OK || rows == 0) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != DITNORM_OK) return st;
  RowArgs a{};
  a.x = (const uint16_t *)x;
  a.residual = (const uint16_t *)residual;
  a.gate = (const uint16_t *)gate;
  a.scale = (const uint16_t *)scale;
  a.shift = (const uint16_t *)shift;
  a.residual_out = (uint16_t *)residual_out;
  a.out = (uint16_t *)out;
  a.mean_out = mean_out;
  a.rstd_out = rstd_out;
  a.y_out = (uint16_t *)y_out;
  a.rows = rows;
  a.cols = (int32_t)cols;
  a.rows_per_batch = rows_per_batch;
  a.mod_stride = mod_batch_stride;
  a.eps = eps;
  return finish(launch_row(a, false, true, false, dev, (hipStream_t)stream));
}

int rms_modulate(const void *x, const void *weight, const void *scale, const void *shift,
                 void *out, const void *residual, const void *gate, void *residual_out,
                 int64_t rows, int64_t cols, int64_t rows_per_batch, int64_t mod_batch_stride,
                 float eps, float *rstd_out, void *y_out, void *stream) {
  int st = validate_rms(x, weight, scale, shift, out, residual, gate, residual_out, rows, cols,
                        rows_per_batch, mod_batch_stride, eps, rstd_out, y_out);
  if (st != DITNORM_OK || rows == 0) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != DITNORM_OK) return st;
  RowArgs a{};
  a.x = (const uint16_t *)x;
  a.weight = (const uint16_t *)weight;
  a.scale = (const uint16_t *)scale;
  a.shift = (const uint16_t *)shift;
  a.out = (uint16_t *)out;
  a.residual = (const uint16_t *)residual;
  a.gate = (const uint16_t *)gate;
  a.residual_out = (uint16_t *)residual_out;
  a.rstd_out = rstd_out;
  a.y_out = (uint16_t *)y_out;
  a.rows = rows;
  a.cols = (int32_t)cols;
  a.rows_per_batch = rows_per_batch;
  a.mod_stride = mod_batch_stride;
  a.eps = eps;
  return finish(launch_row(a, true, residual != nullptr, false, dev, (hipStream_t)stream));
}

int qk_layernorm(const void *q, const void *k, void *q_out, void *k_out, int64_t rows_q,
                 int64_t rows_k, int64_t head_dim, float eps, float *mean_out, float *rstd_out,
                 void *stream) {
  int st = validate_qk(q, k, q_out, k_out, rows_q, rows_k, head_dim, eps, mean_out, rstd_out);
  if (st != DITNORM_OK || rows_q + rows_k == 0) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != DITNORM_OK) return st;
  QkArgs a{};
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.q_out = (uint16_t *)q_out;
  a.k_out = (uint16_t *)k_out;
  a.mean_out = mean_out;
  a.rstd_out = rstd_out;
  a.rows_q = rows_q;
  a.rows_k = rows_k;
  a.head_dim = (int32_t)head_dim;
  a.eps = eps;
  return finish(launch_qk(a, dev, (hipStream_t)stream));
}

int rmsnorm_silu_bias(const void *x, const float *bias, const float *gamma, void *out,
                      int64_t rows, int64_t channels, float eps, float *rstd_out, void *xb_out,
                      void *stream) {
  int st = validate_wan(x, bias, gamma, out, rows, channels, eps, rstd_out, xb_out);
  if (st != DITNORM_OK || rows == 0) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != DITNORM_OK) return st;
  WanArgs a{};
  a.x = (const uint16_t *)x;
  a.bias = bias;
  a.gamma = gamma;
  a.out = (uint16_t *)out;
  a.rstd_out = rstd_out;
  a.xb_out = (uint16_t *)xb_out;
  a.rows = rows;
  a.channels = (int32_t)channels;
  a.eps = eps;
  return finish(launch_wan(a, dev, (hipStream_t)stream));
}

int conv_bias_epilogue(const void *x, const void *bias, const void *h, void *out, int64_t rows,
                       int64_t channels, int dtype, int bias_dtype, void *stream) {
  int st = validate_epilogue(x, bias, h, out, rows, channels, dtype, bias_dtype);
  if (st != DITNORM_OK || rows == 0) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != DITNORM_OK) return st;
  EpilogueArgs a{};
  a.x = x;
  a.bias = bias;
  a.h = h;
  a.out = out;
  a.rows = rows;
  a.channels = (int32_t)channels;
  a.dtype = dtype;
  a.bias_dtype = bias_dtype;
  return finish(launch_epilogue(a, dev, (hipStream_t)stream));
}

int ln_modulate_supported(const void *x, const void *scale, const void *shift, const void *out,
                          int64_t rows, int64_t cols, int64_t rows_per_batch,
                          int64_t mod_batch_stride, float eps, const float *mean_out,
                          const float *rstd_out, const void *y_out) {
  return validate_ln(x, scale, shift, out, rows, cols, rows_per_batch, mod_batch_stride, eps,
                     mean_out, rstd_out, y_out) == DITNORM_OK;
}

int ln_modulate_folded_supported(const void *x, const void *scale, const void *shift,
                                 const void *out, int64_t rows, int64_t cols,
                                 int64_t rows_per_batch, int64_t mod_batch_stride, float eps,
                                 const float *mean_out, const float *rstd_out) {
  return validate_ln(x, scale, shift, out, rows, cols, rows_per_batch, mod_batch_stride, eps,
                     mean_out, rstd_out, nullptr) == DITNORM_OK;
}

int gated_ln_modulate_supported(const void *x, const void *residual, const void *gate,
                                const void *scale, const void *shift, const void *residual_out,
                                const void *out, int64_t rows, int64_t cols,
                                int64_t rows_per_batch, int64_t mod_batch_stride, float eps,
                                const float *mean_out, const float *rstd_out,
                                const void *y_out) {
  return validate_gated_ln(x, residual, gate, scale, shift, residual_out, out, rows, cols,
                           rows_per_batch, mod_batch_stride, eps, mean_out, rstd_out,
                           y_out) == DITNORM_OK;
}

int rms_modulate_supported(const void *x, const void *weight, const void *scale,
                           const void *shift, const void *out, const void *residual,
                           const void *gate, const void *residual_out, int64_t rows,
                           int64_t cols, int64_t rows_per_batch, int64_t mod_batch_stride,
                           float eps, const float *rstd_out, const void *y_out) {
  return validate_rms(x, weight, scale, shift, out, residual, gate, residual_out, rows, cols,
                      rows_per_batch, mod_batch_stride, eps, rstd_out, y_out) == DITNORM_OK;
}

int qk_layernorm_supported(const void *q, const void *k, const void *q_out, const void *k_out,
                           int64_t rows_q, int64_t rows_k, int64_t head_dim, float eps,
                           const float *mean_out, const float *rstd_out) {
  return validate_qk(q, k, q_out, k_out, rows_q, rows_k, head_dim, eps, mean_out, rstd_out) ==
         DITNORM_OK;
}

int rmsnorm_silu_bias_supported(const void *x, const float *bias, const float *gamma,
                                const void *out, int64_t rows, int64_t channels, float eps,
                                const float *rstd_out, const void *xb_out) {
  return validate_wan(x, bias, gamma, out, rows, channels, eps, rstd_out, xb_out) == DITNORM_OK;
}

int conv_bias_epilogue_supported(const void *x, const void *bias, const void *h,
                                 const void *out, int64_t rows, int64_t channels, int dtype,
                                 int bias_dtype) {
  return validate_epilogue(x, bias, h, out, rows, channels, dtype, bias_dtype) == DITNORM_OK;
}

int modulate_scale_shift(const void *x, const void *scale, const void *shift, void *out,
                         int64_t rows, int64_t cols, int64_t rows_per_batch,
                         int64_t mod_batch_stride, int dtype, void *stream) {
  return launch_ew(0, x, nullptr, scale, shift, out, rows, cols, rows_per_batch,
                   mod_batch_stride, dtype, stream);
}

int residual_gate_add(const void *update, const void *residual, const void *gate, void *out,
                      int64_t rows, int64_t cols, int64_t rows_per_batch,
                      int64_t mod_batch_stride, int dtype, void *stream) {
  return launch_ew(1, update, residual, gate, nullptr, out, rows, cols, rows_per_batch,
                   mod_batch_stride, dtype, stream);
}

int modulate_scale_shift_supported(const void *x, const void *scale, const void *shift,
                                   const void *out, int64_t rows, int64_t cols,
                                   int64_t rows_per_batch, int64_t mod_batch_stride, int dtype) {
  return validate_elementwise(0, x, nullptr, scale, shift, out, rows, cols, rows_per_batch,
                              mod_batch_stride, dtype) == DITNORM_OK;
}

int residual_gate_add_supported(const void *update, const void *residual, const void *gate,
                                const void *out, int64_t rows, int64_t cols,
                                int64_t rows_per_batch, int64_t mod_batch_stride, int dtype) {
  return validate_elementwise(1, update, residual, gate, nullptr, out, rows, cols,
                              rows_per_batch, mod_batch_stride, dtype) == DITNORM_OK;
}

int64_t ln_modulate_backward_workspace_bytes(int64_t rows, int64_t cols,
                                             int64_t rows_per_batch, int dtype) {
  if (rows < 0 || cols <= 0 || rows_per_batch <= 0 || rows % rows_per_batch != 0) return -1;
  if (dtype != DITNORM_DTYPE_BF16 && dtype != DITNORM_DTYPE_F32) return -1;
  if (rows > DITNORM_MAX_ROWS ||
      cols > (dtype == DITNORM_DTYPE_F32 ? DITNORM_MAX_BACKWARD_F32_COLS
                                         : DITNORM_MAX_BACKWARD_COLS))
    return -1;  // the call rejects them
  if (rows == 0) return 0;
  return bwd_layout(rows, cols, rows_per_batch, dtype).bytes;
}

int ln_modulate_backward(const void *x, const void *scale, const void *d_out, void *d_x,
                         float *d_scale, float *d_shift, int64_t rows, int64_t cols,
                         int64_t rows_per_batch, int64_t mod_batch_stride, float eps,
                         void *workspace, int64_t workspace_bytes, float *mean_out,
                         float *rstd_out, int dtype, void *stream) {
  int st = validate_backward(x, scale, d_out, d_x, d_scale, d_shift, rows, cols, rows_per_batch,
                             mod_batch_stride, eps, workspace, workspace_bytes, mean_out,
                             rstd_out, dtype);
  if (st != DITNORM_OK || rows == 0) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != DITNORM_OK) return st;
  return backward_launch(x, scale, d_out, d_x, d_scale, d_shift, rows, cols, rows_per_batch,
                         mod_batch_stride, eps, (char *)workspace, mean_out, rstd_out, dtype,
                         stream);
}

int ln_modulate_backward_noalloc(const void *x, const void *scale, const void *d_out, void *d_x,
                                 float *d_scale, float *d_shift, int64_t rows, int64_t cols,
                                 int64_t rows_per_batch, int64_t mod_batch_stride, float eps,
                                 float *mean_out, float *rstd_out, int dtype, void *stream) {
  int st = validate_backward(x, scale, d_out, d_x, d_scale, d_shift, rows, cols, rows_per_batch,
                             mod_batch_stride, eps, nullptr, 0, mean_out, rstd_out, dtype, true);
  if (st != DITNORM_OK || rows == 0) return st;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != DITNORM_OK) return st;
  char *ws = nullptr;
  if ((st = scratch_address(dev.device, &ws)) != DITNORM_OK) return st;
  return backward_launch(x, scale, d_out, d_x, d_scale, d_shift, rows, cols, rows_per_batch,
                         mod_batch_stride, eps, ws, mean_out, rstd_out, dtype, stream);
}

int ln_modulate_backward_supported(const void *x, const void *scale, const void *d_out,
                                   const void *d_x, const float *d_scale, const float *d_shift,
                                   int64_t rows, int64_t cols, int64_t rows_per_batch,
                                   int64_t mod_batch_stride, float eps, const void *workspace,
                                   int64_t workspace_bytes, const float *mean_out,
                                   const float *rstd_out, int dtype) {
  return validate_backward(x, scale, d_out, d_x, d_scale, d_shift, rows, cols, rows_per_batch,
                           mod_batch_stride, eps, workspace, workspace_bytes, mean_out,
                           rstd_out, dtype) == DITNORM_OK;
}

int ditnorm_copy(const void *src, void *dst, int64_t bytes, void *stream) {
  if (bytes < 0 || (bytes > 0 && (!src || !dst))) return DITNORM_INVALID_ARGUMENT;
  if (bytes % 16 != 0 || bytes / 16 > DITNORM_MAX_VECTORS - 255 || !aligned16(src) ||
      !aligned16(dst))
    return DITNORM_UNSUPPORTED;
  if (overlap(Buf{src, bytes}, Buf{dst, bytes})) return DITNORM_UNSUPPORTED;
  if (bytes == 0) return DITNORM_OK;
  DeviceInfo dev;
  int st = current_device(&dev);
  if (st != DITNORM_OK) return st;
  return finish(launch_copy(src, dst, bytes, dev, (hipStream_t)stream));
}

}  // extern "C"
