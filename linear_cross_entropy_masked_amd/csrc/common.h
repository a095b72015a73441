// Shared device helpers for the gfx950 kernels (bf16 unpacking, wave reductions) and the
// host-side launch declarations used by the C ABI in capi.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 is the upper half of an fp32: widening is a shift (low element) or a mask (high).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Merge two (max, sum of exp(x - max)) pairs.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  s = s * fast_exp2((m - mn) * kLog2e) + s2 * fast_exp2((m2 - mn) * kLog2e);
  m = mn;
}

// Reduce (m, s) over a 64-lane wavefront; every lane ends with the result.
__device__ __forceinline__ void wave_lse_reduce(float& m, float& s) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float m2 = __shfl_xor(m, off, 64);
    float s2 = __shfl_xor(s, off, 64);
    lse_merge(m, s, m2, s2);
  }
}

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace lce

// ---- host launchers (defined in the kernel files, called from capi.hip) ----
namespace lce {

struct CeWorkspace {
  long long* count;  // device int64: number of labelled rows
  float* row_loss;   // device fp32 [n]
};

size_t ce_workspace_bytes(int64_t n);
CeWorkspace ce_workspace_carve(void* base, int64_t n);

hipError_t launch_label_prep(const int32_t* labels, int64_t n, int64_t v, int32_t ignore_index,
                             long long* count_out, int32_t* status_out, hipStream_t stream);
hipError_t launch_ce_fwd_rows(const uint16_t* logits, int64_t n, int64_t v, int64_t ld,
                              const int32_t* labels, int32_t ignore_index, float* row_loss,
                              float* lse_out, hipStream_t stream);
hipError_t launch_loss_reduce(const float* row_loss, int64_t n, const long long* count_dev,
                              long long count_host, float* loss_out, hipStream_t stream);
// One pass per row (forward and in-place backward); rows up to 16 · 1024 aligned vectors
// (ce_fused_fits). Returns hipErrorInvalidValue for longer rows without launching.
bool ce_fused_fits(int64_t v);
hipError_t launch_ce_fused_rows(uint16_t* logits, int64_t n, int64_t v, int64_t ld,
                                const int32_t* labels, int32_t ignore_index,
                                const long long* count_dev, long long count_host,
                                const float* grad_output, float* row_loss, float* lse_out,
                                hipStream_t stream);
hipError_t launch_ce_bwd_rows(const uint16_t* logits, int64_t ld, uint16_t* grad, int64_t ldg,
                              int64_t n, int64_t v, const int32_t* labels, int32_t ignore_index,
                              const float* lse, const long long* count_dev, long long count_host,
                              const float* grad_output, const float* grad_rows,
                              hipStream_t stream);

}  // namespace lce

// ---- opt-in launch timing (lce_timing_enable / lce_timing_read in the C ABI) ----
namespace lce {

enum KernelId {
  K_LABEL_PREP = 0,
  K_CE_FWD_ROWS,
  K_LOSS_REDUCE,
  K_CE_BWD_ROWS,
  K_FLCE_GEMM_LOGITS,
  K_FLCE_ROW_LSE,
  K_FLCE_BIAS_GRAD,
  K_FLCE_TO_PROBS,
  K_FLCE_GEMM_GRAD_HIDDEN,
  K_FLCE_GEMM_GRAD_WEIGHT,
  K_FLCE_ONEHOT_FIX,
  K_FILL,
  K_FLCE_GRAD_HIDDEN_REDUCE,
  K_FLCE_GEMM_PROBS,
  K_FLCE_LABEL_SORT,
  K_CE_FUSED_ROWS,
  K_FLCE_LOSS_ACC,
  K_FLCE_PROBS_TRANSPOSED,
  K_COUNT
};

const char* kernel_name(int id);
bool timing_on();
// Record a start/stop event pair around a launch on `stream` (no-ops unless enabled).
void timing_start(hipStream_t stream, int id);
void timing_stop(hipStream_t stream, int id);

// RAII helper: brackets one launch.
struct TimedLaunch {
  hipStream_t s;
  int id;
  TimedLaunch(hipStream_t s_, int id_) : s(s_), id(id_) { timing_start(s, id); }
  ~TimedLaunch() { timing_stop(s, id); }
};

}  // namespace lce
