// Internal interface of the fused linear cross-entropy schedule (flce_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

struct FlceArgs {
  const uint16_t* hidden;
  const uint16_t* weight;
  const float* bias;
  const int32_t* labels;
  int64_t n, h, v;
  int32_t ignore_index;
  int64_t chunk_size;
  int64_t num_label_tokens;
  uint32_t flags;
  const float* grad_output;
  float* loss_out;
  float* lse_out;
  uint16_t* grad_hidden;
  float* grad_weight;
  float* grad_bias;
  int32_t* status_out;
  void* workspace;
  int pass;             // kFwdBwd, kFwdOnly (loss and lse, no gradients) or kBwdOnly
  const float* lse_in;  // kBwdOnly: the lse kFwdOnly returned
};
constexpr int kFwdBwd = 0, kFwdOnly = 1, kBwdOnly = 2;

int flce_check_shape(int64_t n, int64_t h, int64_t v, int64_t chunk_size, uint32_t flags);
size_t flce_workspace_bytes(int64_t n, int64_t h, int64_t v, int64_t chunk_size, uint32_t flags);
hipError_t flce_run(const FlceArgs& a, hipStream_t stream);

}  // namespace lce
