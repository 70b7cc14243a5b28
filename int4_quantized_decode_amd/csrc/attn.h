// attn.h - internal interface of the KV-append and attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "i4d_internal.h"

namespace i4d {

struct KvArgs {
  uint8_t* k_codes;
  uint32_t* v_codes;
  uint16_t* k_scales;
  uint16_t* v_scales;
  const int64_t* row_base;
  int n_rows, n_kv, hd;
  int32_t* err_word;
};

struct AppendArgs {
  KvArgs kv;
  const uint16_t* k;  // bf16 [T][n_kv][hd]
  const uint16_t* v;
  const int32_t* row_idx;  // NULL = identity
  const int32_t* pos;      // position per token, or NULL when len is given
  const int32_t* len;      // if non-NULL: position = len[t] - 1 (decode step)
  int T;
};

struct AttnArgs {
  KvArgs kv;
  const float* q;          // fp32 [M][n_q][hd], not rotated
  const int32_t* ctx_len;  // [M]
  const uint16_t* k_new;   // optional bf16 [M][n_kv][hd]: appended at ctx_len-1 first
  const uint16_t* v_new;
  int M, n_q, G, S;
  int bps;                 // 32-token blocks per split: split s = blocks [s bps, (s+1) bps)
  float score_scale;       // log2(e) / (hd * sqrt(hd))
  float* part_ml;          // [M][n_q][S][2]
  float* part_o;           // [M][n_q][S][hd]
  float* attn_f32;         // optional [M][n_q*hd]
  uint16_t* attn_bf16;     // [M][n_q*hd]
  // Inside the one-launch step (M = 1) the query [n_q][hd] (fp32 bits) and
  // the new key and value [n_kv][hd] (bf16 bits) arrive as flagged words
  // (coherent.h) with flag `flag`.
  const uint64_t* q_ll;
  const uint64_t* k_ll;
  const uint64_t* v_ll;
  uint32_t flag;
  unsigned* sync_err;  // set (with I4D_DEVERR_SYNC in kv.err_word) by a poll that times out
};

KvArgs kv_args(const i4d_kv_cache* c);

i4d_status launch_kv_append(const AppendArgs& a, hipStream_t st);
// nwa = waves per workgroup (4, 8 or 16).  With S > 1 the launch writes
// per-split partials; combine = true adds the kernel that merges them into
// attn_bf16 / attn_f32 (otherwise the consumer merges them itself).
i4d_status launch_attention(const AttnArgs& a, int nwa, bool combine, hipStream_t st);

}  // namespace i4d
