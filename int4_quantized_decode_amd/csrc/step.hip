// step.hip - the whole decode step of one layer for one row (M = 1) in one
// persistent launch (gfx950).
//
// At M = 1 the step is a chain of five memory-bound stages (QKV, attention,
// O, gate/up, down) whose data are small but whose every stage depends on
// all of the previous one.  As separate kernels each boundary costs a
// launch (about 1.8 us here), the drain of the previous stage and the first
// load latency of the next.  Here one workgroup of 8 waves per CU runs all
// stages.  A stage's weights do not depend on the activations, yet QKV's
// follow x and those of gate/up are requested only after the wait for the
// previous stage and the x loads: a wave's loads complete in order, and
// weight loads ahead of a short wait or of x measured slower than the
// latency they would hide.  O (behind the attention chain) and down (behind
// a grid barrier after the gate/up stream) wait long enough: they request
// their first atoms before the wait.
//
// Stages and hand-offs (counters in the sync region of the workspace; data
// exchanged with agent-coherent stores and loads, except the query, key and
// value, which travel as flagged words (coherent.h) tagged with the
// launch's epoch + 1: the attention units poll them directly, so the QKV
// workgroups neither wait for their stores nor count them):
//   1. QKV strips (+ rho1, RoPE): q, k, v stored as flagged words.
//   2. Attention unit (kv head j, split s): polls its query heads (and, in
//      the unit that owns position L-1, the new key and value, which it
//      appends); writes a partial; the last unit of kv head j
//      merges the splits, undoes the rotation and counts head j done.
//   3. O strips (+ residual): wait for all kv heads; then a grid barrier.
//   4. gate/up strips (+ rho2, SwiGLU): after the barrier; barrier again.
//   5. down strips (+ residual) -> x_out.
// The counters sit in one of two banks that alternate between launches; the
// first workgroup clears the other bank and, at its end, advances the epoch
// that selects the bank.
// Every wait is bounded: a timeout sets I4D_DEVERR_SYNC and the step runs
// on (with wrong results) instead of hanging.
#include <math.h>

#include "attn.h"
#include "attn_core.h"
#include "coherent.h"
#include "gemv.h"
#include "i4d_internal.h"
#include "proj.h"
#include "step.h"

namespace i4d {

// word offsets in the sync region (one 128-byte line per counter).  The
// counters come in two banks used by alternate launches (the launch's
// epoch selects one): the first workgroup clears the other bank, which the
// previous launch has finished with, while this launch runs, so no launch
// ends with a barrier of all its workgroups to clear its own counters.
constexpr int kLine = 32;
constexpr int kSyncAttn = 0;              // [n_kv] finished attention splits per kv head
constexpr int kSyncAttnDone = 16 * kLine; // kv heads whose attention output is written
constexpr int kSyncBar1 = 17 * kLine;     // 8 group counters (after O)
constexpr int kSyncBar2 = 26 * kLine;     // 8 group counters (after gate/up)
constexpr int kBankLines = 35;            // counter lines of one bank
constexpr int kBankWords = 36 * kLine;    // bank stride
constexpr int kSyncErr = 2 * kBankWords;          // sticky timeout flag (never cleared)
constexpr int kSyncEpoch = 2 * kBankWords + kLine; // completed launches (selects the bank)
static_assert((kSyncEpoch + 1) * 4 <= (int)kStepSyncBytes, "sync region");

// waves per workgroup: 8 (one workgroup per CU, 256 registers per lane)
constexpr int kStepWaves = 8;

// Timeline of a workgroup (optional): the 100 MHz real-time counter at
// entry, QKV stored, attention units done, O's wait passed, O
// stored, gate/up's wait passed, gate/up stored, down's wait passed, down
// stored; read by thread 0 (in the wait hooks after their barrier), stored
// by a vector store.
static_assert(kStepStamps == 10, "stamp slots");
__device__ __forceinline__ void stamp(uint64_t* stamps, int slot) {
  if (stamps && threadIdx.x == 0)
    stamps[(size_t)blockIdx.x * kStepStamps + slot] = __builtin_amdgcn_s_memrealtime();
}

struct StepArgs {
  ProjArgs qkv, o, gu, down;
  GemvPlan pq, po, pg, pd;
  AttnArgs at;
  unsigned* sync;
  uint64_t* stamps;  // optional: kStepStamps timestamps per workgroup
  int32_t* err_word;  // optional (the cache's)
  int n_kv, G, hd, Sf;
};

__device__ __forceinline__ void strip_range(int N, int wg, int nwg, int& s0, int& ns) {
  s0 = (int)((long)wg * N / nwg);
  ns = (int)((long)(wg + 1) * N / nwg) - s0;
}

__device__ __forceinline__ void flag_error(unsigned* err, int32_t* err_word) {
  atomicOr(err, 1u);
  if (err_word) atomicOr(err_word, I4D_DEVERR_SYNC);
}

// all of this workgroup's stores are complete and visible device-wide
__device__ __forceinline__ void stores_done() {
  wait_vmem();
  __builtin_amdgcn_s_barrier();
}

// grid barrier on 8 group counters (workgroup w counts in group w % 8, so
// arrivals spread over 8 addresses); the waiter polls the 8 counters at once
__device__ __forceinline__ void bar_arrive(unsigned* bar, int wg) {
  atomic_add_agent(&bar[(wg & 7) * kLine], 1u);
}
__device__ __forceinline__ bool bar_wait(unsigned* bar, int nwg, unsigned* err) {
  for (int it = 0; it < (1 << 21); ++it) {
    bool all = true;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const unsigned gs = (unsigned)((nwg - g + 7) / 8);
      all &= __hip_atomic_load(&bar[g * kLine], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= gs;
    }
    if (all) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  atomicOr(err, 1u);
  return false;
}

template <int HD, int GQ, int GD>
__global__ __launch_bounds__(kStepWaves * 64) void step_m1_kernel(StepArgs sa) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NW = kStepWaves;
  // Shallow rings (4 atoms per wave): a wave's loads complete in order, so
  // every atom in flight when a stage waits for its producers delays that
  // wave's x loads behind it; deeper rings measured slower at every stage.
  constexpr int UQ = 4;                                  // gate/up
  constexpr int UO = GQ == 0 ? 8 : (GQ > 4 ? GQ : 4);  // O: one strip per workgroup
  constexpr int UD = 4;
  const int tid = threadIdx.x;
  const int wg = blockIdx.x, nwg = gridDim.x;
  stamp(sa.stamps, 0);
  // The epoch (which selects this launch's counter bank) is read by one
  // thread per workgroup into LDS: every wave of every workgroup reading
  // the one word would queue 2048 requests on it at the start, and a
  // wave's loads complete in order, so its first x loads would wait behind
  // them.  Other threads read it after a workgroup barrier; thread 0 uses
  // its own copy.
  __shared__ unsigned epoch_s;
  if (tid == 0) epoch_s = ld_coh(&sa.sync[kSyncEpoch]);
  auto bank_of = [&]() { return sa.sync + (epoch_s & 1u) * kBankWords; };
  unsigned* const err = sa.sync + kSyncErr;
  // the attention units' row metadata (one row), read now so that its
  // latency overlaps the QKV stage, by one thread (as the epoch) into LDS;
  // the attention stage reads it after its first workgroup barrier
  __shared__ RowMeta meta;
  if (tid == 0) {
    const int64_t b0 = sa.at.kv.row_base[0];
    meta.base = b0;
    meta.cap = sa.at.kv.row_base[1] - b0;
    meta.L = sa.at.ctx_len[0];
  }

  // ---- 1. QKV
  {
    const StepArgs* A = &sa;
    ProjArgs pa = A->qkv;
    pa.epoch = &epoch_s;  // read by the epilogue, after the staging barrier
    const GemvPlan pl = A->pq;
    int s0, ns;
    strip_range(pa.Np / kStrip, wg, nwg, s0, ns);
    if (ns > 0) gemv_body<EPI_QKV, NW, 4, GQ, true>(pa, pl, s0, ns, smem, NoWait());
    stamp(A->stamps, 1);
  }

  // ---- 2. attention units (kv head j, split s), head-interleaved
  {
    const StepArgs* A = &sa;
    AttnArgs at = A->at;
    at.sync_err = err;
    unsigned* sync = bank_of();  // thread 0 only (its own read)
    const int n_kv = A->n_kv, G = A->G, Sf = A->Sf;
    const int units = n_kv * Sf;
    for (int u = wg; u < units; u += nwg) {
      const int j = u % n_kv, s = u / n_kv;
      __syncthreads();  // LDS reuse (and epoch_s is visible to every thread)
      at.flag = epoch_s + 1u;
      // the unit polls its query heads (and the new key and value) itself
      attn_body<HD, NW, true>(at, 0, j, s, reinterpret_cast<float*>(smem), NoWait(), &meta);
      stores_done();
      if (Sf > 1) {
        __shared__ int last;
        if (tid == 0) last = (atomic_add_agent(&sync[kSyncAttn + kLine * j], 1u) == (unsigned)(Sf - 1));
        __syncthreads();
        if (last) {
          const int lane = tid & 63, wave = tid >> 6;
          for (int g = wave; g < G; g += NW) {
            float lsum, o0, o1;
            const size_t head_row = (size_t)j * G + g;
            combine_head<HD, true>(at, head_row, lane, lsum, o0, o1);
            finish_head<HD, true>(at, head_row, lsum, o0, o1, lane);
          }
          stores_done();
          if (tid == 0) atomic_add_agent(&sync[kSyncAttnDone], 1u);
        }
      } else if (tid == 0) {
        atomic_add_agent(&sync[kSyncAttnDone], 1u);
      }
    }
    stamp(A->stamps, 2);
  }

  // ---- 3. O + residual (waits for every kv head's attention output)
  {
    const StepArgs* A = &sa;
    const ProjArgs pa = A->o;
    const GemvPlan pl = A->po;
    int32_t* err_word = A->err_word;
    const int n_kv = A->n_kv;
    int s0, ns;
    strip_range(pa.Np / kStrip, wg, nwg, s0, ns);
    auto wait_attn = [&] {
      if (tid == (NW - 1) * 64 && !spin_geq(&bank_of()[kSyncAttnDone], (unsigned)n_kv, err, 1u))
        flag_error(err, err_word);
      lds_barrier();
      stamp(A->stamps, 3);
    };
    __syncthreads();
    // (every thread reads epoch_s only after this barrier) the first
    // workgroup clears the other bank, which the previous launch used
    if (wg == 0 && tid < kBankLines) st_coh(&sa.sync[((epoch_s & 1u) ^ 1u) * kBankWords + tid * kLine], 0u);
    // the first ring of atoms (with one strip per workgroup, the whole O
    // stream) is requested before the wait for the attention heads
    if (ns > 0) gemv_body<EPI_O, NW, UO, GQ, true, true>(pa, pl, s0, ns, smem, wait_attn);
    stores_done();
    if (tid == 0) bar_arrive(&bank_of()[kSyncBar1], wg);
    stamp(A->stamps, 4);
  }

  // ---- 4. gate/up + SwiGLU (after every O strip)
  {
    const StepArgs* A = &sa;
    const ProjArgs pa = A->gu;
    const GemvPlan pl = A->pg;
    int32_t* err_word = A->err_word;
    int s0, ns;
    strip_range(pa.Np / kStrip, wg, nwg, s0, ns);
    auto wait_o = [&] {
      if (tid == (NW - 1) * 64 && !bar_wait(&bank_of()[kSyncBar1], nwg, err)) flag_error(err, err_word);
      lds_barrier();
      stamp(A->stamps, 5);
    };
    __syncthreads();
    if (ns > 0) gemv_body<EPI_GU, NW, UQ, GQ, true>(pa, pl, s0, ns, smem, wait_o);
    stores_done();
    if (tid == 0) bar_arrive(&bank_of()[kSyncBar2], wg);
    stamp(A->stamps, 6);
  }

  // ---- 5. down + residual (after every gate/up strip)
  {
    const StepArgs* A = &sa;
    const ProjArgs pa = A->down;
    const GemvPlan pl = A->pd;
    int32_t* err_word = A->err_word;
    int s0, ns;
    strip_range(pa.Np / kStrip, wg, nwg, s0, ns);
    auto wait_gu = [&] {
      if (tid == (NW - 1) * 64 && !bar_wait(&bank_of()[kSyncBar2], nwg, err)) flag_error(err, err_word);
      lds_barrier();
      stamp(A->stamps, 7);
    };
    __syncthreads();
    // the first ring of atoms is requested before the barrier: gate/up
    // strips finish over about 2 us and every poll of the barrier is a
    // round trip of about 1 us behind the gate/up stream, so the atoms have
    // arrived when the wait ends (on the gate/up stage the same measured
    // slower: its wait is short)
    if (ns > 0) gemv_body<EPI_DOWN, NW, UD, GD, true, true>(pa, pl, s0, ns, smem, wait_gu);
    if (A->stamps) {  // timeline only: every wave's down strips stored
      __syncthreads();
      stamp(A->stamps, 8);
    }
  }

  // ---- exit: the first workgroup advances the epoch (every workgroup read
  // it at entry, before the barrier after O that this one has passed)
  if (wg == 0 && tid == 0) st_coh(&sa.sync[kSyncEpoch], epoch_s + 1u);
}

// ---------------------------------------------------------------------------

namespace {

int gpw_template(int G) {
  // groups per wave of the workgroup: 1, 2, 4 kept in registers, else 0
  const int gpw = G / kStepWaves;
  return (G % kStepWaves == 0 && (gpw == 1 || gpw == 2 || gpw == 4)) ? gpw : 0;
}

GemvPlan step_plan(int nstrips, int G, int nwg) {
  GemvPlan p;
  p.NW = kStepWaves;
  p.GPW = (G + kStepWaves - 1) / kStepWaves;
  p.SP = (nstrips + nwg - 1) / nwg;
  return p;
}

template <int HD, int GQ, int GD>
hipError_t launch_t(const StepArgs& sa, int nwg, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((step_m1_kernel<HD, GQ, GD>), dim3(nwg), dim3(kStepWaves * 64), lds, st, sa);
  return hipGetLastError();
}

template <int HD, int GQ, int GD>
int occupancy_t(size_t lds) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, step_m1_kernel<HD, GQ, GD>, kStepWaves * 64, lds) !=
      hipSuccess)
    return 0;
  return n;
}

template <int HD>
int dispatch_occ(int gq, int gd, size_t lds) {
#define I4D_OCC(Q, D) \
  if (gq == Q && gd == D) return occupancy_t<HD, Q, D>(lds);
  I4D_OCC(1, 4) I4D_OCC(1, 0) I4D_OCC(2, 0) I4D_OCC(2, 4) I4D_OCC(4, 0) I4D_OCC(4, 4) I4D_OCC(0, 0)
  I4D_OCC(0, 4)
#undef I4D_OCC
  return 0;
}

template <int HD>
hipError_t dispatch_launch(int gq, int gd, const StepArgs& sa, int nwg, size_t lds, hipStream_t st) {
#define I4D_LAUNCH(Q, D) \
  if (gq == Q && gd == D) return launch_t<HD, Q, D>(sa, nwg, lds, st);
  I4D_LAUNCH(1, 4) I4D_LAUNCH(1, 0) I4D_LAUNCH(2, 0) I4D_LAUNCH(2, 4) I4D_LAUNCH(4, 0) I4D_LAUNCH(4, 4)
  I4D_LAUNCH(0, 0) I4D_LAUNCH(0, 4)
#undef I4D_LAUNCH
  return hipErrorInvalidValue;
}

size_t attn_lds_bytes(int hd) {
  return (size_t)(hd == 128 ? attn_lds_floats<128, kStepWaves>() : attn_lds_floats<64, kStepWaves>()) * 4;
}

}  // namespace

bool step_m1_supported(const i4d_layer_shape* s) {
  const int gq = gpw_template(s->d_model / kGroup);
  const int go = gpw_template(s->n_q_heads * s->head_dim / kGroup);
  const int G = s->n_q_heads / s->n_kv_heads;
  // one kernel variant for QKV, O and gate/up; every K within the x staging
  // of one workgroup (4 chunks of 8 per thread); at most 16 kv heads
  const int kmax = 4 * 8 * kStepWaves * 64;
  return gq == go && G <= 8 && s->n_kv_heads <= 16 && s->d_model <= kmax &&
         s->n_q_heads * s->head_dim <= kmax && s->d_ffn <= kmax;
}

i4d_status launch_step_m1(const StepInputs& in, hipStream_t st) {
  const i4d_layer_shape& s = in.layer->shape;
  const int gq = gpw_template(s.d_model / kGroup);
  const int gd = gpw_template(s.d_ffn / kGroup) == 4 ? 4 : 0;

  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(I4D_ERR_HIP, "device query failed");

  StepArgs sa = {};
  sa.qkv = in.qkv;
  sa.o = in.o;
  sa.gu = in.gu;
  sa.down = in.down;
  sa.at = in.attn;
  sa.sync = in.sync;
  sa.stamps = in.stamps;
  sa.err_word = in.attn.kv.err_word;
  sa.n_kv = s.n_kv_heads;
  sa.G = s.n_q_heads / s.n_kv_heads;
  sa.hd = s.head_dim;
  sa.Sf = in.attn.S;

  // LDS: the largest stage (attention, or a projection)
  const int nwg_guess = cus;
  sa.pq = step_plan(sa.qkv.Np / kStrip, sa.qkv.G, nwg_guess);
  sa.po = step_plan(sa.o.Np / kStrip, sa.o.G, nwg_guess);
  sa.pg = step_plan(sa.gu.Np / kStrip, sa.gu.G, nwg_guess);
  sa.pd = step_plan(sa.down.Np / kStrip, sa.down.G, nwg_guess);
  size_t lds = attn_lds_bytes(s.head_dim);
  lds = std::max(lds, gemv_lds_bytes(sa.qkv.K, sa.pq));
  lds = std::max(lds, gemv_lds_bytes(sa.o.K, sa.po));
  lds = std::max(lds, gemv_lds_bytes(sa.gu.K, sa.pg));
  lds = std::max(lds, gemv_lds_bytes(sa.down.K, sa.pd));

  // every workgroup must be resident at once (they wait on each other)
  const int occ = s.head_dim == 128 ? dispatch_occ<128>(gq, gd, lds) : dispatch_occ<64>(gq, gd, lds);
  if (occ < 1) return fail(I4D_ERR_UNSUPPORTED, "one-launch step does not fit a CU (LDS %zu)", lds);
  const int nwg = cus;  // one workgroup per CU
  hipError_t e = s.head_dim == 128 ? dispatch_launch<128>(gq, gd, sa, nwg, lds, st)
                                   : dispatch_launch<64>(gq, gd, sa, nwg, lds, st);
  if (e != hipSuccess) return fail(I4D_ERR_HIP, "one-launch step: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace i4d
