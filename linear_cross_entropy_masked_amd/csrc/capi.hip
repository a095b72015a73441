// extern "C" entry points of liblce_masked.so: argument validation, workspace carving and
// the launch schedule. Every error that can be detected from the arguments is returned
// before any HIP call, so these checks run (and are tested) on a machine without a GPU.
#include <atomic>
#include <cstring>
#include <limits>
#include <mutex>

#include "common.h"
#include "flce.h"
#include "lce_masked.h"

namespace {

using lce::CeWorkspace;

constexpr int64_t kI64Max = std::numeric_limits<int64_t>::max();

bool mul_overflows(int64_t a, int64_t b) { return a != 0 && b > kI64Max / a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Per-device cache: 0 = unknown, 1 = gfx950, 2 = other.
std::atomic<int> g_arch_ok[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LCE_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    int c = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (c) return c == 1 ? LCE_OK : LCE_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LCE_ERR_HIP;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? LCE_OK : LCE_ERR_DEVICE;
}

int ce_check_shape(int64_t n, int64_t v, int64_t ld, int64_t chunk_size) {
  if (n < 0 || v < 1 || ld < v) return LCE_ERR_BAD_SHAPE;
  if (n > int64_t(std::numeric_limits<int32_t>::max())) return LCE_ERR_BAD_SHAPE;  // grid.x
  if (mul_overflows(n, ld) || mul_overflows(n * ld, 2)) return LCE_ERR_BAD_SHAPE;
  if (chunk_size <= 0) return LCE_ERR_BAD_CHUNK;
  return LCE_OK;
}

// Byte range [lo, hi) a call reads or writes; empty for a NULL pointer or no bytes.
struct Span {
  uintptr_t lo, hi;
};
Span span(const void* p, int64_t bytes) {
  if (!p || bytes <= 0) return Span{0, 0};
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + uintptr_t(bytes)};
}
// Bytes of a row-major [n, ld] matrix whose first `cols` columns are used.
int64_t matrix_bytes(int64_t n, int64_t ld, int64_t cols, int64_t elem) {
  return n > 0 ? ((n - 1) * ld + cols) * elem : 0;
}
bool spans_meet(Span a, Span b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}
// Every written range must be disjoint from every read range and from the other written
// ranges (inputs may share memory with each other).
template <size_t NW, size_t NR>
int check_disjoint(const Span (&wr)[NW], const Span (&rd)[NR]) {
  for (size_t i = 0; i < NW; ++i) {
    for (size_t j = 0; j < NR; ++j)
      if (spans_meet(wr[i], rd[j])) return LCE_ERR_OVERLAP;
    for (size_t j = i + 1; j < NW; ++j)
      if (spans_meet(wr[i], wr[j])) return LCE_ERR_OVERLAP;
  }
  return LCE_OK;
}

#define LCE_TRY_HIP(expr)                        \
  do {                                           \
    if ((expr) != hipSuccess) return LCE_ERR_HIP; \
  } while (0)

// ---- static scratch of the allocation-free CE step -------------------------------------
//
// The CE step's workspace is a 256-byte header (the label count) and one fp32 term per row.
// ce_chunked_fwd_bwd_inplace_noalloc keeps it in this device array instead of a caller's
// allocation: every GPU the library runs on holds its own copy, for the life of the process.
// The kernels overwrite every word of it they later read (the count, each row's term), so
// nothing is cleared between calls. In host code `scratch` names a host-side stand-in: its
// device address comes from hipGetSymbolAddress, once per device, and only that address is
// ever handed to a kernel.
constexpr size_t kScratchBytes = 256 + size_t(LCE_NOALLOC_MAX_ROWS) * sizeof(float);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device (NULL: not yet)

// The current device's address of `scratch`, looked up on the first call on that device.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LCE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LCE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LCE_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return LCE_OK;
}

// Argument checks of the single-pass CE step (everything but the workspace).
int ce_fused_check(const uint16_t* logits_inout, int64_t n, int64_t v, int64_t ld,
                   const int32_t* labels, int64_t chunk_size, const float* grad_output,
                   const float* loss_out, const float* lse_out, const int32_t* status_out) {
  int rc = ce_check_shape(n, v, ld, chunk_size);
  if (rc != LCE_OK) return rc;
  if (!loss_out || (n > 0 && (!logits_inout || !labels))) return LCE_ERR_NULL_ARG;
  if (!aligned(logits_inout, 2) || !aligned(labels, 4) || !aligned(grad_output, 4) ||
      !aligned(loss_out, 4) || !aligned(lse_out, 4) || !aligned(status_out, 4))
    return LCE_ERR_ALIGNMENT;
  return LCE_OK;
}

// The single-pass CE step's launches with its workspace at `workspace`.
int ce_fused_launch(uint16_t* logits_inout, int64_t n, int64_t v, int64_t ld,
                    const int32_t* labels, int32_t ignore_index, int64_t num_label_tokens,
                    const float* grad_output, float* loss_out, float* lse_out,
                    int32_t* status_out, void* workspace, hipStream_t s) {
  CeWorkspace ws = lce::ce_workspace_carve(workspace, n);
  const long long th = num_label_tokens >= 0 ? num_label_tokens : -1;
  LCE_TRY_HIP(lce::launch_label_prep(labels, n, v, ignore_index, ws.count, status_out, s));
  if (lce::ce_fused_fits(v)) {
    LCE_TRY_HIP(lce::launch_ce_fused_rows(logits_inout, n, v, ld, labels, ignore_index, ws.count,
                                          th, grad_output, ws.row_loss, lse_out, s));
  } else {
    // rows too long to hold in registers: the forward pass, then the in-place backward (which
    // reads each row again, and once more to rebuild its lse when lse_out is NULL)
    LCE_TRY_HIP(lce::launch_ce_fwd_rows(logits_inout, n, v, ld, labels, ignore_index,
                                        ws.row_loss, lse_out, s));
    LCE_TRY_HIP(lce::launch_ce_bwd_rows(logits_inout, ld, logits_inout, ld, n, v, labels,
                                        ignore_index, lse_out, ws.count, th, grad_output,
                                        nullptr, s));
  }
  LCE_TRY_HIP(lce::launch_loss_reduce(ws.row_loss, n, ws.count, th, loss_out, s));
  return LCE_OK;
}

}  // namespace

extern "C" {

const char* lce_status_str(int status) {
  switch (status) {
    case LCE_OK: return "ok";
    case LCE_ERR_NULL_ARG: return "a required pointer is NULL";
    case LCE_ERR_BAD_SHAPE: return "bad shape (n < 0, v < 1, h < 1, ld < v, h % 8 != 0, or size overflow)";
    case LCE_ERR_BAD_CHUNK: return "chunk_size must be > 0";
    case LCE_ERR_WORKSPACE: return "workspace is NULL or smaller than the size query's answer";
    case LCE_ERR_HIP: return "a HIP call or kernel launch failed";
    case LCE_ERR_DEVICE: return "the current device is not gfx950 (MI355X)";
    case LCE_ERR_BAD_FLAGS: return "unknown flag bits";
    case LCE_ERR_ALIGNMENT: return "a pointer is not aligned to its element size";
    case LCE_ERR_OVERLAP: return "an output or the workspace overlaps another buffer of the call";
    case LCE_ERR_SCRATCH_LIMIT:
      return "n exceeds LCE_NOALLOC_MAX_ROWS, the rows the allocation-free call's static scratch holds";
    default: return "unknown status";
  }
}

const char* flce_status_str(int status) { return lce_status_str(status); }

int ce_chunked_workspace_size(int64_t n, int64_t v, int64_t chunk_size, size_t* bytes) {
  if (!bytes) return LCE_ERR_NULL_ARG;
  const int rc = ce_check_shape(n, v, v, chunk_size);
  if (rc != LCE_OK) return rc;
  *bytes = lce::ce_workspace_bytes(n);
  return LCE_OK;
}

int ce_chunked_fwd(const uint16_t* logits, int64_t n, int64_t v, int64_t ld,
                   const int32_t* labels, int32_t ignore_index, int64_t chunk_size,
                   int64_t num_label_tokens, float* loss_out, float* lse_out,
                   int32_t* status_out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = ce_check_shape(n, v, ld, chunk_size);
  if (rc != LCE_OK) return rc;
  if (!loss_out || (n > 0 && (!logits || !labels))) return LCE_ERR_NULL_ARG;
  if (!workspace || workspace_bytes < lce::ce_workspace_bytes(n)) return LCE_ERR_WORKSPACE;
  if (!aligned(logits, 2) || !aligned(labels, 4) || !aligned(loss_out, 4) ||
      !aligned(lse_out, 4) || !aligned(status_out, 4) || !aligned(workspace, 256))
    return LCE_ERR_ALIGNMENT;
  {
    const Span wr[] = {span(workspace, int64_t(lce::ce_workspace_bytes(n))), span(loss_out, 4),
                       span(lse_out, 4 * n), span(status_out, 4)};
    const Span rd[] = {span(logits, matrix_bytes(n, ld, v, 2)), span(labels, 4 * n)};
    if ((rc = check_disjoint(wr, rd)) != LCE_OK) return rc;
  }
  if ((rc = check_device()) != LCE_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  CeWorkspace ws = lce::ce_workspace_carve(workspace, n);
  LCE_TRY_HIP(lce::launch_label_prep(labels, n, v, ignore_index, ws.count, status_out, s));
  LCE_TRY_HIP(lce::launch_ce_fwd_rows(logits, n, v, ld, labels, ignore_index, ws.row_loss,
                                      lse_out, s));
  LCE_TRY_HIP(lce::launch_loss_reduce(ws.row_loss, n, ws.count,
                                      num_label_tokens >= 0 ? num_label_tokens : -1, loss_out, s));
  return LCE_OK;
}

int ce_chunked_bwd(const uint16_t* logits, int64_t n, int64_t v, int64_t ld, uint16_t* grad,
                   int64_t ldg, const int32_t* labels, int32_t ignore_index, int64_t chunk_size,
                   int64_t num_label_tokens, const float* grad_output, const float* lse,
                   int32_t* status_out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = ce_check_shape(n, v, ld, chunk_size);
  if (rc != LCE_OK) return rc;
  if (ldg < v || mul_overflows(n, ldg) || mul_overflows(n * ldg, 2)) return LCE_ERR_BAD_SHAPE;
  if (n > 0 && (!logits || !grad || !labels)) return LCE_ERR_NULL_ARG;
  if (!workspace || workspace_bytes < lce::ce_workspace_bytes(n)) return LCE_ERR_WORKSPACE;
  if (!aligned(logits, 2) || !aligned(grad, 2) || !aligned(labels, 4) ||
      !aligned(grad_output, 4) || !aligned(lse, 4) || !aligned(status_out, 4) ||
      !aligned(workspace, 256))
    return LCE_ERR_ALIGNMENT;
  {
    // grad == logits with ldg == ld is the in-place case; any other overlap is refused
    const bool inplace = grad == logits && ldg == ld;
    const Span wr[] = {span(workspace, int64_t(lce::ce_workspace_bytes(n))), span(status_out, 4),
                       span(grad, matrix_bytes(n, ldg, v, 2))};
    const Span rd[] = {span(inplace ? nullptr : logits, matrix_bytes(n, ld, v, 2)),
                       span(labels, 4 * n), span(grad_output, 4), span(lse, 4 * n)};
    if ((rc = check_disjoint(wr, rd)) != LCE_OK) return rc;
  }
  if ((rc = check_device()) != LCE_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  CeWorkspace ws = lce::ce_workspace_carve(workspace, n);
  LCE_TRY_HIP(lce::launch_label_prep(labels, n, v, ignore_index, ws.count, status_out, s));
  LCE_TRY_HIP(lce::launch_ce_bwd_rows(logits, ld, grad, ldg, n, v, labels, ignore_index, lse,
                                      ws.count, num_label_tokens >= 0 ? num_label_tokens : -1,
                                      grad_output, nullptr, s));
  return LCE_OK;
}

int ce_chunked_bwd_inplace(uint16_t* logits_inout, int64_t n, int64_t v, int64_t ld,
                           const int32_t* labels, int32_t ignore_index, int64_t chunk_size,
                           int64_t num_label_tokens, const float* grad_output, const float* lse,
                           int32_t* status_out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return ce_chunked_bwd(logits_inout, n, v, ld, logits_inout, ld, labels, ignore_index,
                        chunk_size, num_label_tokens, grad_output, lse, status_out, workspace,
                        workspace_bytes, stream);
}

int ce_chunked_fwd_bwd_inplace(uint16_t* logits_inout, int64_t n, int64_t v, int64_t ld,
                               const int32_t* labels, int32_t ignore_index, int64_t chunk_size,
                               int64_t num_label_tokens, const float* grad_output,
                               float* loss_out, float* lse_out, int32_t* status_out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  int rc = ce_fused_check(logits_inout, n, v, ld, labels, chunk_size, grad_output, loss_out,
                          lse_out, status_out);
  if (rc != LCE_OK) return rc;
  if (!workspace || workspace_bytes < lce::ce_workspace_bytes(n)) return LCE_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return LCE_ERR_ALIGNMENT;
  {
    const Span wr[] = {span(workspace, int64_t(lce::ce_workspace_bytes(n))), span(loss_out, 4),
                       span(lse_out, 4 * n), span(status_out, 4),
                       span(logits_inout, matrix_bytes(n, ld, v, 2))};
    const Span rd[] = {span(labels, 4 * n), span(grad_output, 4)};
    if ((rc = check_disjoint(wr, rd)) != LCE_OK) return rc;
  }
  if ((rc = check_device()) != LCE_OK) return rc;
  return ce_fused_launch(logits_inout, n, v, ld, labels, ignore_index, num_label_tokens,
                         grad_output, loss_out, lse_out, status_out, workspace,
                         static_cast<hipStream_t>(stream));
}

int ce_chunked_fwd_bwd_inplace_noalloc(uint16_t* logits_inout, int64_t n, int64_t v, int64_t ld,
                                       const int32_t* labels, int32_t ignore_index,
                                       int64_t chunk_size, int64_t num_label_tokens,
                                       const float* grad_output, float* loss_out,
                                       float* lse_out, int32_t* status_out, void* stream) {
  int rc = ce_fused_check(logits_inout, n, v, ld, labels, chunk_size, grad_output, loss_out,
                          lse_out, status_out);
  if (rc != LCE_OK) return rc;
  if (n > LCE_NOALLOC_MAX_ROWS) return LCE_ERR_SCRATCH_LIMIT;
  {
    const Span wr[] = {span(loss_out, 4), span(lse_out, 4 * n), span(status_out, 4),
                       span(logits_inout, matrix_bytes(n, ld, v, 2))};
    const Span rd[] = {span(labels, 4 * n), span(grad_output, 4)};
    if ((rc = check_disjoint(wr, rd)) != LCE_OK) return rc;
  }
  if ((rc = check_device()) != LCE_OK) return rc;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws)) != LCE_OK) return rc;
  return ce_fused_launch(logits_inout, n, v, ld, labels, ignore_index, num_label_tokens,
                         grad_output, loss_out, lse_out, status_out, ws,
                         static_cast<hipStream_t>(stream));
}

int ce_rows_fwd(const uint16_t* logits, int64_t n, int64_t v, int64_t ld, const int32_t* labels,
                int32_t ignore_index, int64_t chunk_size, float* row_loss_out, float* lse_out,
                int32_t* status_out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = ce_check_shape(n, v, ld, chunk_size);
  if (rc != LCE_OK) return rc;
  if (n > 0 && (!logits || !labels || !row_loss_out)) return LCE_ERR_NULL_ARG;
  if (!workspace || workspace_bytes < lce::ce_workspace_bytes(n)) return LCE_ERR_WORKSPACE;
  if (!aligned(logits, 2) || !aligned(labels, 4) || !aligned(row_loss_out, 4) ||
      !aligned(lse_out, 4) || !aligned(status_out, 4) || !aligned(workspace, 256))
    return LCE_ERR_ALIGNMENT;
  {
    const Span wr[] = {span(workspace, int64_t(lce::ce_workspace_bytes(n))),
                       span(row_loss_out, 4 * n), span(lse_out, 4 * n), span(status_out, 4)};
    const Span rd[] = {span(logits, matrix_bytes(n, ld, v, 2)), span(labels, 4 * n)};
    if ((rc = check_disjoint(wr, rd)) != LCE_OK) return rc;
  }
  if ((rc = check_device()) != LCE_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  CeWorkspace ws = lce::ce_workspace_carve(workspace, n);
  LCE_TRY_HIP(lce::launch_label_prep(labels, n, v, ignore_index, ws.count, status_out, s));
  LCE_TRY_HIP(lce::launch_ce_fwd_rows(logits, n, v, ld, labels, ignore_index, row_loss_out,
                                      lse_out, s));
  return LCE_OK;
}

int ce_rows_bwd(const uint16_t* logits, int64_t n, int64_t v, int64_t ld, uint16_t* grad,
                int64_t ldg, const int32_t* labels, int32_t ignore_index, int64_t chunk_size,
                const float* grad_rows, const float* lse, int32_t* status_out, void* workspace,
                size_t workspace_bytes, void* stream) {
  int rc = ce_check_shape(n, v, ld, chunk_size);
  if (rc != LCE_OK) return rc;
  if (ldg < v || mul_overflows(n, ldg) || mul_overflows(n * ldg, 2)) return LCE_ERR_BAD_SHAPE;
  if (n > 0 && (!logits || !grad || !labels || !grad_rows)) return LCE_ERR_NULL_ARG;
  if (!workspace || workspace_bytes < lce::ce_workspace_bytes(n)) return LCE_ERR_WORKSPACE;
  if (!aligned(logits, 2) || !aligned(grad, 2) || !aligned(labels, 4) || !aligned(grad_rows, 4) ||
      !aligned(lse, 4) || !aligned(status_out, 4) || !aligned(workspace, 256))
    return LCE_ERR_ALIGNMENT;
  {
    const bool inplace = grad == logits && ldg == ld;
    const Span wr[] = {span(workspace, int64_t(lce::ce_workspace_bytes(n))), span(status_out, 4),
                       span(grad, matrix_bytes(n, ldg, v, 2))};
    const Span rd[] = {span(inplace ? nullptr : logits, matrix_bytes(n, ld, v, 2)),
                       span(labels, 4 * n), span(grad_rows, 4 * n), span(lse, 4 * n)};
    if ((rc = check_disjoint(wr, rd)) != LCE_OK) return rc;
  }
  if ((rc = check_device()) != LCE_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  CeWorkspace ws = lce::ce_workspace_carve(workspace, n);
  LCE_TRY_HIP(lce::launch_label_prep(labels, n, v, ignore_index, ws.count, status_out, s));
  LCE_TRY_HIP(lce::launch_ce_bwd_rows(logits, ld, grad, ldg, n, v, labels, ignore_index, lse,
                                      ws.count, -1, nullptr, grad_rows, s));
  return LCE_OK;
}

int flce_workspace_size(int64_t n, int64_t h, int64_t v, int64_t chunk_size, uint32_t flags,
                        size_t* bytes) {
  if (!bytes) return LCE_ERR_NULL_ARG;
  const int rc = lce::flce_check_shape(n, h, v, chunk_size, flags);
  if (rc != LCE_OK) return rc;
  *bytes = lce::flce_workspace_bytes(n, h, v, chunk_size, flags);
  return LCE_OK;
}

int flce_fwd_bwd(const uint16_t* hidden, const uint16_t* weight, const float* bias,
                 const int32_t* labels, int64_t n, int64_t h, int64_t v, int32_t ignore_index,
                 int64_t chunk_size, int64_t num_label_tokens, uint32_t flags,
                 const float* grad_output, float* loss_out, float* lse_out,
                 uint16_t* grad_hidden, float* grad_weight, float* grad_bias,
                 int32_t* status_out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = lce::flce_check_shape(n, h, v, chunk_size, flags);
  if (rc != LCE_OK) return rc;
  if (!loss_out || !weight || (n > 0 && (!hidden || !labels)) || (grad_bias && !bias))
    return LCE_ERR_NULL_ARG;
  if (!workspace || workspace_bytes < lce::flce_workspace_bytes(n, h, v, chunk_size, flags))
    return LCE_ERR_WORKSPACE;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(bias, 4) || !aligned(labels, 4) ||
      !aligned(grad_output, 4) || !aligned(loss_out, 4) || !aligned(lse_out, 4) ||
      !aligned(grad_hidden, 16) || !aligned(grad_weight, 16) || !aligned(grad_bias, 4) ||
      !aligned(status_out, 4) || !aligned(workspace, 256))
    return LCE_ERR_ALIGNMENT;
  {
    // grad_hidden and the workspace are scratch during the call: nothing may share them
    const Span wr[] = {span(workspace, int64_t(lce::flce_workspace_bytes(n, h, v, chunk_size, flags))),
                       span(grad_hidden, 2 * n * h), span(grad_weight, 4 * v * h),
                       span(grad_bias, 4 * v), span(loss_out, 4), span(lse_out, 4 * n),
                       span(status_out, 4)};
    const Span rd[] = {span(hidden, 2 * n * h), span(weight, 2 * v * h), span(bias, 4 * v),
                       span(labels, 4 * n), span(grad_output, 4)};
    if ((rc = check_disjoint(wr, rd)) != LCE_OK) return rc;
  }
  if ((rc = check_device()) != LCE_OK) return rc;
  lce::FlceArgs a{hidden, weight, bias, labels, n, h, v, ignore_index, chunk_size,
                  num_label_tokens, flags, grad_output, loss_out, lse_out, grad_hidden,
                  grad_weight, grad_bias, status_out, workspace, lce::kFwdBwd, nullptr};
  return lce::flce_run(a, static_cast<hipStream_t>(stream)) == hipSuccess ? LCE_OK : LCE_ERR_HIP;
}

int flce_fwd(const uint16_t* hidden, const uint16_t* weight, const float* bias,
             const int32_t* labels, int64_t n, int64_t h, int64_t v, int32_t ignore_index,
             int64_t chunk_size, int64_t num_label_tokens, float* loss_out, float* lse_out,
             int32_t* status_out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = lce::flce_check_shape(n, h, v, chunk_size, 0);
  if (rc != LCE_OK) return rc;
  if (!loss_out || !weight || (n > 0 && (!hidden || !labels || !lse_out))) return LCE_ERR_NULL_ARG;
  if (!workspace || workspace_bytes < lce::flce_workspace_bytes(n, h, v, chunk_size, 0))
    return LCE_ERR_WORKSPACE;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(bias, 4) || !aligned(labels, 4) ||
      !aligned(loss_out, 4) || !aligned(lse_out, 4) || !aligned(status_out, 4) ||
      !aligned(workspace, 256))
    return LCE_ERR_ALIGNMENT;
  {
    const Span wr[] = {span(workspace, int64_t(lce::flce_workspace_bytes(n, h, v, chunk_size, 0))),
                       span(loss_out, 4), span(lse_out, 4 * n), span(status_out, 4)};
    const Span rd[] = {span(hidden, 2 * n * h), span(weight, 2 * v * h), span(bias, 4 * v),
                       span(labels, 4 * n)};
    if ((rc = check_disjoint(wr, rd)) != LCE_OK) return rc;
  }
  if ((rc = check_device()) != LCE_OK) return rc;
  lce::FlceArgs a{hidden, weight, bias, labels, n, h, v, ignore_index, chunk_size,
                  num_label_tokens, 0, nullptr, loss_out, lse_out, nullptr, nullptr, nullptr,
                  status_out, workspace, lce::kFwdOnly, nullptr};
  return lce::flce_run(a, static_cast<hipStream_t>(stream)) == hipSuccess ? LCE_OK : LCE_ERR_HIP;
}

int flce_bwd(const uint16_t* hidden, const uint16_t* weight, const float* bias,
             const int32_t* labels, const float* lse, int64_t n, int64_t h, int64_t v,
             int32_t ignore_index, int64_t chunk_size, int64_t num_label_tokens, uint32_t flags,
             const float* grad_output, uint16_t* grad_hidden, float* grad_weight,
             float* grad_bias, int32_t* status_out, void* workspace, size_t workspace_bytes,
             void* stream) {
  if (flags & FLCE_RECOMPUTE) return LCE_ERR_BAD_FLAGS;  // the backward always recomputes
  int rc = lce::flce_check_shape(n, h, v, chunk_size, flags);
  if (rc != LCE_OK) return rc;
  if (!weight || (n > 0 && (!hidden || !labels || !lse)) || (grad_bias && !bias))
    return LCE_ERR_NULL_ARG;
  if (!workspace || workspace_bytes < lce::flce_workspace_bytes(n, h, v, chunk_size, flags))
    return LCE_ERR_WORKSPACE;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(bias, 4) || !aligned(labels, 4) ||
      !aligned(lse, 4) || !aligned(grad_output, 4) || !aligned(grad_hidden, 16) ||
      !aligned(grad_weight, 16) || !aligned(grad_bias, 4) || !aligned(status_out, 4) ||
      !aligned(workspace, 256))
    return LCE_ERR_ALIGNMENT;
  {
    const Span wr[] = {span(workspace, int64_t(lce::flce_workspace_bytes(n, h, v, chunk_size, flags))),
                       span(grad_hidden, 2 * n * h), span(grad_weight, 4 * v * h),
                       span(grad_bias, 4 * v), span(status_out, 4)};
    const Span rd[] = {span(hidden, 2 * n * h), span(weight, 2 * v * h), span(bias, 4 * v),
                       span(labels, 4 * n), span(lse, 4 * n), span(grad_output, 4)};
    if ((rc = check_disjoint(wr, rd)) != LCE_OK) return rc;
  }
  if ((rc = check_device()) != LCE_OK) return rc;
  lce::FlceArgs a{hidden, weight, bias, labels, n, h, v, ignore_index, chunk_size,
                  num_label_tokens, flags, grad_output, nullptr, nullptr, grad_hidden,
                  grad_weight, grad_bias, status_out, workspace, lce::kBwdOnly, lse};
  return lce::flce_run(a, static_cast<hipStream_t>(stream)) == hipSuccess ? LCE_OK : LCE_ERR_HIP;
}

}  // extern "C"
