// step.h - internal interface of the one-launch decode step (M = 1).
#pragma once
#include <hip/hip_runtime.h>

#include "attn.h"
#include "i4d_internal.h"
#include "proj.h"

namespace i4d {

struct StepInputs {
  const i4d_layer* layer;
  ProjArgs qkv, o, gu, down;  // as for the stage kernels (M = 1)
  AttnArgs attn;              // S = step_m1_splits(...)
  unsigned* sync;             // kStepSyncBytes, zero before the first launch (the step keeps it usable)
  uint64_t* stamps = nullptr;  // optional timeline, kStepStamps per workgroup
};

constexpr int kStepStamps = I4D_STEP_STAMPS;

bool step_m1_supported(const i4d_layer_shape* s);

// Argument checks of a decode step (everything but the workspace) and the
// workspace layout it needs.
i4d_status check_decode_step(const i4d_layer* layer, const i4d_kv_cache* cache, const uint16_t* x_in,
                             const uint16_t* x_out, const int32_t* ctx_len, int M, int max_ctx_len,
                             int num_splits, const float* attn_f32, i4d_workspace_layout* wl);
// Enqueue a checked decode step (weights in the WeightFormat fmt) whose intermediates live at the offsets of
// `wl` from `ws` (the projections' K-split partials take split_part_bytes
// from wl.split_part); the counters at wl.sync and wl.split_cnt must be zero
// and are left at zero.
i4d_status run_decode_step(const i4d_layer* layer, const i4d_kv_cache* cache, const uint16_t* x_in,
                           uint16_t* x_out, const int32_t* ctx_len, int M, int max_ctx_len, int num_splits,
                           char* ws, const i4d_workspace_layout& wl, size_t split_part_bytes, float* attn_f32,
                           hipStream_t st, int fmt, uint64_t* stamps = nullptr);
// zero `bytes` (a multiple of 16) at the 16-byte aligned device address p
i4d_status launch_zero_fill(void* p, size_t bytes, hipStream_t st);
i4d_status launch_step_m1(const StepInputs& in, hipStream_t st);

}  // namespace i4d
