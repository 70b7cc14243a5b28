// proj.h - internal interface of the INT4 projection kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "i4d_internal.h"

namespace i4d {

enum Epi { EPI_QKV = 0, EPI_O = 1, EPI_GU = 2, EPI_DOWN = 3 };

// weight formats: INT4 codes (1 KiB atoms) or E4M3 codes (2 KiB atoms), both
// with fp16 scales per (row, 128-group)
enum WeightFormat { kFmtInt4 = 0, kFmtE4M3 = 1 };

struct ProjArgs {
  const uint8_t* codes;    // packed atoms [Np/16][K/128][64][16]
  const uint16_t* scales;  // fp16 [Np/16][G][16]
  const uint16_t* x;       // bf16 input [M][K]
  int Np, K, G, G8, M;
  float eps;
  // QKV epilogue
  float* q_out;
  uint16_t* k_out;
  uint16_t* v_out;
  const int32_t* ctx_len;
  int n_q, n_kv, hd;
  float theta;
  double rope_ratio;  // theta^(-2/hd), fp64 (RoPE frequency of pair i = ratio^i)
  // O epilogue
  const uint16_t* resid_bf16;
  float* h_f32;
  uint16_t* h_bf16;
  // gate/up epilogue
  uint16_t* a_out;
  // down epilogue
  const float* resid_f32;
  uint16_t* out_bf16;
  // split of K across workgroups (M > 1; NULL: none): partial tiles and one
  // arrival counter per strip set, zero between launches
  float* split_part;
  unsigned* split_cnt;
  size_t split_bytes;
  int fmt;  // WeightFormat of codes/scales
  // one-launch step (M = 1): the QKV epilogue also writes q, k, v as
  // flagged words (coherent.h) whose flag is *epoch + 1 (the launch's
  // epoch, read from LDS once the workgroup has passed a barrier)
  uint64_t* q_ll;
  uint64_t* k_ll;
  uint64_t* v_ll;
  const unsigned* epoch;
};


i4d_status launch_projection(int epi, const ProjArgs& a, hipStream_t st);
// E4M3 weights (a.fmt == kFmtE4M3), any M in [1, 32]
i4d_status launch_projection_e4m3(int epi, const ProjArgs& a, hipStream_t st);
// the launch plan of launch_projection for `a` (host only, nothing launched)
i4d_status projection_plan_of(int epi, const ProjArgs& a, i4d_projection_plan* out);

}  // namespace i4d
