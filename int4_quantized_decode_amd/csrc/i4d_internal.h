// i4d_internal.h - host-side helpers shared by the C-ABI translation units.
#pragma once
#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/i4d.h"
#include "i4d_layout.h"

namespace i4d {

// split buffer a projection of Np x K at M rows uses when one is at hand
// (0 bytes: it does not split K): partial tiles and strip-set counters
struct SplitNeed {
  size_t part_bytes;
  size_t counters;
};
SplitNeed projection_split_need(int Np, int K, int M);


// records the message for i4d_last_error() and returns `st`
i4d_status fail(i4d_status st, const char* fmt, ...);
i4d_status ok();

bool aligned16(const void* p);

// validates a layer shape (returns I4D_OK or the error, message set)
i4d_status check_shape(const i4d_layer_shape* s);

// a required device pointer: non-NULL and 16-byte aligned
i4d_status need(const void* p, const char* what);
// a cache that matches the shape `s` (may be NULL) and holds at least M rows
i4d_status check_cache(const i4d_kv_cache* c, const i4d_layer_shape* s, int M);

// launch plan of the attention kernel: KV splits per (row, kv head) and
// waves per workgroup
struct AttnPlan {
  int S;
  int nwa;
};
AttnPlan attn_plan(const i4d_layer_shape* s, int M, int max_ctx_len, int num_splits);

// KV splits of the one-launch decode step (M = 1): one attention unit per
// (kv head, split), about 256 units, at least one 32-token block each
int step_m1_splits(const i4d_layer_shape* s, int max_ctx_len, int num_splits);

// size of the sync region of the decode-step workspace (zero before first use)
constexpr size_t kStepSyncBytes = 16384;
// The decode-step workspace starts with the counters, at the same offsets
// for every shape, M and split count: the one-launch step's sync region
// (kStepSyncBytes), then the projections' K-split arrival counters
// (kSplitCntBytes).  One zero-filled workspace can then serve steps of any
// shape: counters a step relies on are never where another layout keeps
// its data.
constexpr size_t kSplitCntBytes = 8192;

struct AttnWs {
  size_t ml;      // fp32 [M][n_q][S][2]   (running max in log2 units, sum)
  size_t o;       // fp32 [M][n_q][S][hd]  unnormalised rotated output
  size_t total;
};
AttnWs attn_ws_layout(const i4d_layer_shape* s, int M, int S);

// Flagged exchange words (8 bytes each) of the one-launch step (M = 1),
// byte offsets from the end of the step's attention partials in the
// attention workspace: query [n_q][hd], new key and value [n_kv][hd].
struct StepLl {
  size_t q, k, v, total;
};
StepLl step_ll_layout(const i4d_layer_shape* s);

struct LmWs {
  size_t val;   // fp32 [nwaves][M]
  size_t idx;   // int32 [nwaves][M]
  size_t total;
  int nwaves;
};
constexpr int kLmStripsPerWave = 2;
constexpr int kLmWavesPerBlock = 4;
LmWs lm_ws_layout(int V, int M);

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace i4d
