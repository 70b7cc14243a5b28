// lmhead.h - internal interface of the LM head kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "i4d_internal.h"

namespace i4d {

struct LmArgs {
  const uint16_t* w;  // bf16 [V][d]
  const uint16_t* h;  // bf16 [M][d]
  int V, d, M, nwaves;
  float eps;
  float* logits;      // optional fp32 [M][V]
  float* part_val;    // [nwaves][M]
  int32_t* part_idx;  // [nwaves][M]
  int32_t* token;     // [M]
};

i4d_status launch_lm_head(const LmArgs& a, hipStream_t st);

}  // namespace i4d
