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
  unsigned* sync;             // kStepSyncBytes, zero on entry; left zero on exit
};

bool step_m1_supported(const i4d_layer_shape* s);
i4d_status launch_step_m1(const StepInputs& in, hipStream_t st);

}  // namespace i4d
