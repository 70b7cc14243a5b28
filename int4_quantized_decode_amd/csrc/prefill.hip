// prefill.hip - FP8 (E4M3) prefill of the QKV projection, with the keys and
// values placed straight into the INT4 cache (gfx950).
//
// The "how it works" section of the onedev.kr summary describes the prefill
// as an FP8 GEMM whose QKV epilogue writes K and V at offset(request, head,
// position, channel) of the cache (no dense K/V tensor, no scatter kernel),
// with the RMSNorm gain folded into the weights and rho applied in the
// epilogue, FP8 outputs written by the producing epilogue under delayed
// per-tensor scaling (this call's maximum sets the next call's scale), and
// packed requests tracked by prefix sums instead of padding rows.
//
// Launches:
//   prep   one workgroup per (16-token tile, chunk of 8 weight groups of d):
//          the token map (request by binary search of the prefix sums,
//          position), the RoPE rotation of every token, partial sums of
//          squares for rho, max |x| (atomic max), and x8 = E4M3(x / s_x)
//          stored in the FP8 MFMA operand order;
//   gemm   one workgroup per (two heads = 256 output rows, 128 tokens):
//          v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales.  A is
//          the E4M3 weight atom exactly as stored for the decode variant
//          (lane 16j + r: row r, bytes 8kb + e = k 32kb + 8j + e), B the x8
//          tile in the same byte order, so the 128-term dot product of a
//          group comes out of one instruction.  Each group's product is
//          scaled by its fp16 weight scale and added to the fp32 tile.
//          Epilogue through LDS per 32 tokens: s_x * rho, RoPE, then q ->
//          E4M3(q / s_q) (max |q| atomic), k and v -> bf16 -> Hadamard
//          rotation -> INT4 with one fp16 scale -> cache slot;
//   update (own entry point) next scale = max / 448, maxima reset.
//
// Every (token, head) of the cache is written by exactly one workgroup.
// A value dword holds 8 tokens of one channel: it is stored whole when its 8
// tokens are in one workgroup's tile and request, else each token sets its
// nibble with an atomic and/or (the tile edges and request ends).
#include <math.h>

#include "attn.h"
#include "device_common.h"
#include "gemv.h"
#include "i4d_internal.h"

namespace i4d {

namespace {

constexpr int kHd = 128;            // head_dim this path takes
constexpr int kWaves = 8;           // gemm workgroup: 4 row quarters x 2 token halves
constexpr int kThreads = 64 * kWaves;
constexpr int kTilesPerWg = 16;     // 16-token tiles per gemm workgroup
constexpr int kTokPerWg = 16 * kTilesPerWg;
constexpr int kTilesPerWave = 8;    // a wave's token half
constexpr int kRowsPerWg = 256;     // two heads
constexpr int kStripsPerWave = 4;   // 64 rows per wave
constexpr int kChunkTok = 32;       // epilogue tokens per LDS pass
constexpr int kYPitch = kHd + 4;    // fp32 words per (head, token) row of the epilogue tile
constexpr int kPrepGroups = 8;      // weight groups of d per prep workgroup

typedef int i32x8_t __attribute__((ext_vector_type(8)));

struct PrefillArgs {
  const uint8_t* codes;   // E4M3 QKV atoms [strip][group][64 lanes][32 B]
  const uint8_t* scales;  // E8M0 bytes [strip][group][16 rows]
  int N, K, G;
  int n_q, n_kv;
  float eps;
  double rope_ratio;
  const uint16_t* x;  // bf16 [T][K]
  int T, Tpad, R, nch;
  const int32_t* cu;     // [R + 1]
  const int32_t* start;  // [R]
  i4d_fp8_scales* sc;
  uint8_t* q8;  // [T][n_q * 128]
  uint16_t* k_bf16;
  uint16_t* v_bf16;
  KvArgs kv;
  uint8_t* x8;    // [Tpad / 16][G][2 halves][64 lanes][16 B]
  float* sumsq;   // [nch][Tpad]
  int2* map;      // [Tpad] (cache row, position; -1 = no cache write)
  float2* rope;   // [Tpad][64] (cos, sin)
};

// OCP E4M3 codes of four finite fp32 values (nearest, ties to even, the sign
// kept on zero), bytes 0..3 of the result: gfx950's v_cvt_pk_fp8_f32 on
// inputs clamped to +-448, which gives the saturating encoding (checked
// against the format's definition on every fp16 value, on random values
// and on every midpoint between neighbouring codes and its neighbours)
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  c = fminf(fmaxf(c, -448.0f), 448.0f);
  d = fminf(fmaxf(d, -448.0f), 448.0f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// rint(x / s) clamped to [-8, 7], plus 8, where x / s is the correctly
// rounded fp32 quotient: q = x * (1/s) with one residual correction is
// within one ulp of it, which decides the same integer except next to a
// half-integer, where the quotient is recomputed with the rounded division
__device__ __forceinline__ uint32_t int4_code(float x, float s, float rs) {
  const float q0 = x * rs;
  float q = fmaf(fmaf(-q0, s, x), rs, q0);
  const float fr = fabsf(q - truncf(q));
  if (fabsf(fr - 0.5f) < 1.0e-5f) q = __fdiv_rn(x, s);
  return (uint32_t)((int)fminf(7.f, fmaxf(-8.f, rintf(q))) + 8);
}

// a per-tensor scale the caller supplied: a positive finite value, else 1
// with I4D_DEVERR_SCALE raised
__device__ __forceinline__ float checked_scale(float s, int32_t* err, bool report) {
  if (s > 0.f && s <= 3.4e38f) return s;
  if (report && err) atomicOr(err, I4D_DEVERR_SCALE);
  return 1.0f;
}

__device__ __forceinline__ void atomic_max_pos(float* p, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(p), __float_as_uint(v));
}

// ---------------------------------------------------------------------------
// prep
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void prefill_prep_kernel(PrefillArgs a) {
  __shared__ float red_sq[4][16];
  __shared__ float red_max[4];
  __shared__ int tok_pos[16];
  const int tile = blockIdx.x, ch = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, j = lane >> 4;
  const int t = tile * 16 + r;
  const bool live = t < a.T;
  const float sx = checked_scale(a.sc->x_scale, a.kv.err_word, tile == 0 && ch == 0 && tid == 0);

  float sq = 0.f, amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + 256 * i;
    const int g = ch * kPrepGroups + (u >> 7), h = (u >> 6) & 1;
    if (g >= a.G) break;
    uint32_t out[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k0 = 128 * g + 32 * (2 * h + half) + 8 * j;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (live) v = load16(a.x + (size_t)t * a.K + k0);
      float q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
        sq = fmaf(f, f, sq);
        amax = fmaxf(amax, fabsf(f));
        q[e] = __fdiv_rn(f, sx);
      }
      out[2 * half] = e4m3x4(q[0], q[1], q[2], q[3]);
      out[2 * half + 1] = e4m3x4(q[4], q[5], q[6], q[7]);
    }
    const u32x4_t o = {out[0], out[1], out[2], out[3]};
    *reinterpret_cast<u32x4_t*>(a.x8 + ((((size_t)tile * a.G + g) * 2 + h) * 64 + lane) * 16) = o;
  }
  // the thread's token is r in every unit: sum over j (lanes), then waves
  sq += lane_xor(sq, 16, lane);
  sq += lane_xor(sq, 32, lane);
  float m = amax;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, lane_xor(m, o, lane));
  if (j == 0) red_sq[wave][r] = sq;
  if (lane == 0) red_max[wave] = m;
  if (ch == 0 && tid < 16) {
    // token map: request rr with cu[rr] <= t < cu[rr + 1]
    const int tt = tile * 16 + tid;
    int row = 0, cpos = -1, rpos = 0;
    if (tt < a.T) {
      int lo = 0, hi = a.R;  // cu[lo] <= tt < cu[hi] when tt is inside the batch
      if (a.cu[0] <= tt && tt < a.cu[a.R]) {
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (a.cu[mid] <= tt) lo = mid; else hi = mid;
        }
        row = lo;
        rpos = a.start[lo] + (tt - a.cu[lo]);
        const int64_t cap = a.kv.row_base[lo + 1] - a.kv.row_base[lo];
        cpos = (rpos >= 0 && rpos < cap) ? rpos : -1;
      }
      if (cpos < 0 && a.kv.err_word) atomicOr(a.kv.err_word, I4D_DEVERR_APPEND_POS);
      rpos = max(rpos, 0);
    }
    a.map[tt] = make_int2(row, cpos);
    tok_pos[tid] = rpos;
  }
  __syncthreads();
  if (tid < 16) {
    const float s = red_sq[0][tid] + red_sq[1][tid] + red_sq[2][tid] + red_sq[3][tid];
    a.sumsq[(size_t)ch * a.Tpad + tile * 16 + tid] = s;
  }
  if (tid == 0) {
    const float mm = fmaxf(fmaxf(red_max[0], red_max[1]), fmaxf(red_max[2], red_max[3]));
    if (mm > 0.f) atomic_max_pos(&a.sc->x_amax, mm);
  }
  if (ch == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;  // token idx / 64 of the tile, pair c = idx % 64
      const int tl = idx >> 6, c = idx & 63;
      float cs, sn;
      rope_angle(a.rope_ratio, tok_pos[tl], c, cs, sn);
      a.rope[(size_t)(tile * 16 + tl) * 64 + c] = make_float2(cs, sn);
    }
  }
}

// ---------------------------------------------------------------------------
// gemm + epilogue
// ---------------------------------------------------------------------------

struct TokInfo {
  int64_t base;  // first slot of the token's cache row (row_base * n_kv)
  int cap;       // capacity of that row
  int row, pos;  // cache row, position (-1: no cache write)
  int lo, hi;    // the token's request as a local token range of this tile
  float rho;
};

// LDS.  Main loop: a ring of two stages, each holding one weight group's A
// operands [16 strips][2 halves][64 lanes][16 B], the B operands of the
// workgroup's tokens [16 tiles][2 halves][64 lanes][16 B] and the group
// scales [16 strips][16 rows] (E8M0 bytes).  Epilogue (after the loop, over
// the same bytes): fp32 tile [2 heads][32 tokens][kYPitch] and one region
// that holds either the RoPE rotations of half the tile's tokens [128]
// [kRopePitch] (tiles with a q or k head) and after them the value codes
// [256 tokens][v heads][128] (tiles with a v head).  Token info [256] sits
// after both.
constexpr int kStages = 2;
constexpr size_t kStageA = 16 * 2048;
constexpr size_t kStageB = kTilesPerWg * 2048;
constexpr size_t kStageS = 16 * 16;
constexpr size_t kStageBytes = kStageA + kStageB + kStageS;
constexpr size_t kRingBytes = kStages * kStageBytes;
constexpr size_t kYBytes = (size_t)2 * kChunkTok * kYPitch * 4;
constexpr int kRopePitch = 72;  // float2 per token row: 64 pairs + 64 B so that 4 rows read at once hit distinct banks
constexpr int kRopeTok = 128;   // tokens whose rotations are in LDS at a time
constexpr size_t kRopeBytes = (size_t)kRopeTok * kRopePitch * 8;
constexpr size_t kVcodeBytes = (size_t)kTokPerWg * 2 * kHd;
// a tile has RoPE rows and one v head's codes, or two v heads' codes
constexpr size_t kRegionBytes =
    kRopeBytes + kVcodeBytes / 2 > kVcodeBytes ? kRopeBytes + kVcodeBytes / 2 : kVcodeBytes;
constexpr size_t kEpiBytes = kYBytes + kRegionBytes;
constexpr size_t kShared = kRingBytes > kEpiBytes ? kRingBytes : kEpiBytes;
constexpr size_t kGemmLds = kShared + kTokPerWg * sizeof(TokInfo);  // token info after the shared region
static_assert(kGemmLds <= 160 * 1024, "LDS");
static_assert(kTokPerWg <= 256, "representative entries keep the token in 8 bits");

__device__ __forceinline__ i32x8_t cat8(const u32x4_t& lo, const u32x4_t& hi) {
  return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per active lane from global memory straight into LDS at
// lds + 16 * lane.  Issued from asm (M0 saved and restored) so that the
// compiler does not drain it before every LDS read; the ring waits for it
// with an explicit vmcnt.  lds must be wave-uniform.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(lds)
      : "memory");
}

// The two heads of gemm tile n: the q heads paired with the k and v heads
// first (q_i with kv head i, kv heads in k | v order), then the remaining
// heads two by two, so that the tiles with the heavier k / v epilogue also
// hold a q head and the epilogues even out.  Heads are numbered in the
// packed QKV order (q | k | v), head h owns strips 8h .. 8h + 7.
__device__ __forceinline__ int2 tile_heads(int n, int n_q, int n_kv) {
  const int P = min(n_q, 2 * n_kv);
  if (n < P) return make_int2(n, n_q + n);
  // the rest in order: q heads P .. n_q - 1, then kv heads P .. 2 n_kv - 1
  const int i = 2 * (n - P);
  auto rest = [&](int k) { return k < n_q - P ? P + k : n_q + P + (k - (n_q - P)); };
  return make_int2(rest(i), rest(i + 1));
}

// every vector-memory operation of the wave has completed
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8)); }

__global__ __launch_bounds__(kThreads) void prefill_gemm_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 3, wt = wave >> 2;  // row quarter (4 strips), token half (8 tiles)
  const int r = lane & 15, j = lane >> 4;
  const int G = a.G;
  const int t_tiles = a.Tpad / kTokPerWg;
  // consecutive workgroups share the weight tile (measured faster than
  // grouping whole weight tiles per XCD)
  const int b = blockIdx.x;
  const int ntile = b / t_tiles, ttile = b % t_tiles;
  const int2 heads = tile_heads(ntile, a.n_q, a.n_kv);
  // global strip of the tile's strip s (0..7: first head, 8..15: second)
  auto gstrip = [&](int s) { return (s < 8 ? heads.x * 8 : heads.y * 8 - 8) + s; };
  const int tile16_0 = ttile * kTilesPerWg;
  const int tok0 = ttile * kTokPerWg;
  const uint32_t lds0 = lds_offset(smem);

  // ---- main loop: the weight groups of d through a two-stage LDS ring ----
  // per stage and wave: 4 of the 32 A halves, 4 of the 32 B halves, and (in
  // the first token half) the scales of the wave's 4 strips
  auto issue = [&](int g, int stage) {
    const uint32_t sa = lds0 + stage * (uint32_t)kStageBytes;
    const uint32_t sb = sa + (uint32_t)kStageA;
    const uint32_t ss = sb + (uint32_t)kStageB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = wt * 4 + i, s = 4 * wn + (p >> 1), h = p & 1;
      const uint8_t* src = a.codes + ((size_t)gstrip(s) * G + g) * 2048 + lane * 32 + h * 16;
      lds_dma16(src, sa + (uint32_t)((s * 2 + h) * 1024));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = wave * 4 + i, tt = p >> 1, h = p & 1;
      const uint8_t* src = a.x8 + ((size_t)(tile16_0 + tt) * G + g) * 2048 + h * 1024 + lane * 16;
      lds_dma16(src, sb + (uint32_t)(p * 1024));
    }
    {
      const uint8_t* src = a.scales + ((size_t)gstrip(4 * wn + (lane & 3)) * G + g) * 16;
      if (wt == 0 && lane < 4) lds_dma16(src, ss + (uint32_t)(wn * 64));
    }
  };

  f32x4_t acc[kStripsPerWave][kTilesPerWave];
#pragma unroll
  for (int s = 0; s < kStripsPerWave; ++s)
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) acc[s][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int stage) {
    const unsigned char* sa = smem + (size_t)stage * kStageBytes;
    const unsigned char* sb = sa + kStageA;
    const unsigned char* ss = sb + kStageB;
    i32x8_t av[kStripsPerWave];
    int sc[kStripsPerWave];
#pragma unroll
    for (int s = 0; s < kStripsPerWave; ++s) {
      const unsigned char* pa = sa + ((4 * wn + s) * 2) * 1024 + lane * 16;
      av[s] = cat8(*reinterpret_cast<const u32x4_t*>(pa), *reinterpret_cast<const u32x4_t*>(pa + 1024));
      // the E8M0 scale of the lane's row (row r of the strip, whatever j)
      sc[s] = ss[wn * 64 + s * 16 + r];
    }
    // the group scales enter the instruction (E8M0 per row), so the
    // accumulators chain across groups with no VALU work
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const unsigned char* pb = sb + ((kTilesPerWave * wt + t) * 2) * 1024 + lane * 16;
      const i32x8_t bv = cat8(*reinterpret_cast<const u32x4_t*>(pb), *reinterpret_cast<const u32x4_t*>(pb + 1024));
#pragma unroll
      for (int s = 0; s < kStripsPerWave; ++s)
        acc[s][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[s], bv, acc[s][t], 0, 0, 0, sc[s], 0, 127);
    }
  };

  issue(0, 0);

  // token info for the epilogue, read while the first group loads
  TokInfo* tinfo = reinterpret_cast<TokInfo*>(smem + kShared);
  if (tid < kTokPerWg) {
    const int t = tok0 + tid;
    float ssum = 0.f;
    for (int c = 0; c < a.nch; ++c) ssum += a.sumsq[(size_t)c * a.Tpad + t];
    TokInfo ti;
    ti.rho = 1.0f / sqrtf(ssum / (float)a.K + a.eps);
    const int2 m = a.map[t];
    ti.row = m.x;
    ti.pos = t < a.T ? m.y : -1;
    ti.lo = 0;
    ti.hi = 0;
    ti.cap = 0;
    ti.base = 0;
    if (ti.pos >= 0) {
      ti.lo = max(a.cu[m.x], tok0) - tok0;
      ti.hi = min(min(a.cu[m.x + 1], a.T), tok0 + kTokPerWg) - tok0;
      const int64_t rb = a.kv.row_base[m.x];
      ti.cap = (int)(a.kv.row_base[m.x + 1] - rb);
      ti.base = rb * a.kv.n_kv;
    }
    tinfo[tid] = ti;
  }

  for (int g = 0; g < G; ++g) {
    // group g landed (nothing else is in flight), for every wave
    wait_vm0();
    lds_barrier();
    // the stage of group g - 1 is free again: group g + 1 goes there
    if (g + 1 < G) issue(g + 1, (g + 1) % kStages);
    compute(g % kStages);
  }
  lds_barrier();  // every wave is done with the ring; the epilogue reuses it

  // ---- epilogue ----
  float* ybuf = reinterpret_cast<float*>(smem);
  unsigned char* region = smem + kYBytes;
  float2* rope_s = reinterpret_cast<float2*>(region);
  const int hv0 = heads.x >= a.n_q + a.n_kv, hv1 = heads.y >= a.n_q + a.n_kv;  // v heads
  const int nvh = hv0 + hv1;
  const bool has_rope = nvh < 2;  // a q or k head
  uint8_t* vcodes = region + (has_rope ? kRopeBytes : 0);  // [token][v slot][128]
  // the v slot of head hl (0 for the tile's only v head)
  auto vslot = [&](int hl) { return nvh == 2 ? hl : 0; };
  // the RoPE rows of tokens [128 h, 128 h + 128) of the tile (q and k tiles)
  auto load_rope = [&](int h) {
    const uint32_t rb = lds_offset(rope_s);
    for (int tl = wave; tl < kRopeTok; tl += kWaves) {
      const float2* src = a.rope + (size_t)(tok0 + kRopeTok * h + tl) * 64 + 2 * (lane & 31);
      if (lane < 32) lds_dma16(src, rb + (uint32_t)(tl * kRopePitch * 8));
    }
  };
  if (has_rope) load_rope(0);
  const float sx = checked_scale(a.sc->x_scale, nullptr, false);
  const float sq = checked_scale(a.sc->q_scale, a.kv.err_word, blockIdx.x == 0 && tid == 0);
  const float rsq = __fdiv_rn(1.0f, sq);
  float qmax = 0.f;
  const int hl_w = wn >> 1;  // head of this wave's rows
  const int sp0 = 4 * (wn & 1);
  const int l16 = tid & 15;
#pragma unroll
  for (int c = 0; c < kTilesPerWg / 2; ++c) {
    // fp32 tile [head][token][channel] of tokens 32c .. 32c + 31, from the
    // waves of that token half (the loop is unrolled so that acc is indexed
    // by constants and stays in registers)
    if (wt == c / 4) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = 2 * (c % 4) + tt;  // the wave's tile
        const int tl = 16 * tt + r;
        const float f = sx * tinfo[32 * c + tl].rho;
#pragma unroll
        for (int s = 0; s < kStripsPerWave; ++s) {
          const int sp = sp0 + s;
          const int ch0 = (j < 2) ? 8 * sp + 4 * j : kHd / 2 + 8 * sp + 4 * (j - 2);
          const f32x4_t v = {acc[s][t][0] * f, acc[s][t][1] * f, acc[s][t][2] * f, acc[s][t][3] * f};
          *reinterpret_cast<f32x4_t*>(&ybuf[((size_t)hl_w * kChunkTok + tl) * kYPitch + ch0]) = v;
        }
      }
    }
    if (has_rope && c % 4 == 0) {
      if (c > 0) load_rope(c / 4);
      wait_vm0();  // the RoPE rows (every wave's own DMAs)
    }
    // LDS-only barriers: the chunk's global stores need not complete here
    lds_barrier();
    // one (head, token) vector per 16 lanes, 8 channels per lane
#pragma unroll 1
    for (int it = 0; it < 2 * kChunkTok / (kThreads / 16); ++it) {
      const int vec = it * (kThreads / 16) + (tid >> 4);
      const int hl = vec >> 5, tl = vec & 31;
      const int tloc = 32 * c + tl;
      const int t = tok0 + tloc;
      const int head = hl ? heads.y : heads.x;
      const bool is_q = head < a.n_q;
      const bool is_k = !is_q && head < a.n_q + a.n_kv;
      if (t >= a.T) continue;
      const TokInfo ti = tinfo[tloc];
      const float* yr = &ybuf[((size_t)hl * kChunkTok + tl) * kYPitch];
      float y[8];
      {
        const f32x4_t p0 = *reinterpret_cast<const f32x4_t*>(yr + 8 * l16);
        const f32x4_t p1 = *reinterpret_cast<const f32x4_t*>(yr + 8 * l16 + 4);
        y[0] = p0.x; y[1] = p0.y; y[2] = p0.z; y[3] = p0.w;
        y[4] = p1.x; y[5] = p1.y; y[6] = p1.z; y[7] = p1.w;
      }
      if (is_q || is_k) {
        // rotate-half RoPE: channel c pairs with c + 64 (lane l16 ^ 8)
        const int part = (8 * l16 + kHd / 2) & (kHd - 1);
        const f32x4_t p0 = *reinterpret_cast<const f32x4_t*>(yr + part);
        const f32x4_t p1 = *reinterpret_cast<const f32x4_t*>(yr + part + 4);
        const float o[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        const float2* rp = rope_s + (tloc % kRopeTok) * kRopePitch + (8 * l16 & 63);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 cs = rp[e];
          y[e] = (l16 < 8) ? y[e] * cs.x - o[e] * cs.y : y[e] * cs.x + o[e] * cs.y;
        }
      }
      if (is_q) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, fabsf(y[e]));
        const uint32_t w0 = e4m3x4(y[0] * rsq, y[1] * rsq, y[2] * rsq, y[3] * rsq);
        const uint32_t w1 = e4m3x4(y[4] * rsq, y[5] * rsq, y[6] * rsq, y[7] * rsq);
        *reinterpret_cast<u32x2_t*>(a.q8 + ((size_t)t * a.n_q + head) * kHd + 8 * l16) = u32x2_t{w0, w1};
        continue;
      }
      // keys and values: bf16, Hadamard rotation, INT4 with one fp16 scale
      const int kvh = head - a.n_q - (is_k ? 0 : a.n_kv);
      const int64_t slot = ti.base + (int64_t)kvh * ti.cap + ti.pos;
      uint16_t bf[8];
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf[e] = f32_to_bf16(y[e]);
        x[e] = bf16_to_f32(bf[e]);
      }
      uint16_t* dense = is_k ? a.k_bf16 : a.v_bf16;
      if (dense && ti.pos >= 0) {
        const u32x4_t pk = {bf[0] | ((uint32_t)bf[1] << 16), bf[2] | ((uint32_t)bf[3] << 16),
                            bf[4] | ((uint32_t)bf[5] << 16), bf[6] | ((uint32_t)bf[7] << 16)};
        *reinterpret_cast<u32x4_t*>(dense + slot * kHd + 8 * l16) = pk;
      }
#pragma unroll
      for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (!(e & h)) {
            const float lo = x[e], hi = x[e | h];
            x[e] = lo + hi;
            x[e | h] = lo - hi;
          }
      // stages h = 8 .. 64 across lanes: x' = x + p (lower lane) or p - x
      // (upper lane), both one rounded operation as fma(+-1, x, p)
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        const float sgn = (l16 & m) ? -1.0f : 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = fmaf(sgn, x[e], lane_xor(x[e], m, lane));
      }
      float am = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(x[e]));
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) am = fmaxf(am, lane_xor(am, m, lane));
      const float q7 = __fdiv_rn(am, 7.0f);
      _Float16 h16 = (_Float16)q7;
      uint16_t s16 = bitcast<uint16_t>(h16);
      if ((s16 & 0x7fffu) == 0x7c00u) s16 = (uint16_t)((s16 & 0x8000u) | 0x7bffu);
      const float sf = f16_bits_to_f32(s16);
      const float rsf = (sf != 0.f) ? __fdiv_rn(1.0f, sf) : 0.f;
      uint32_t u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = (sf != 0.f) ? int4_code(x[e], sf, rsf) : 8u;
      if (ti.pos < 0) continue;
      if (is_k) {
        // key slot dword jj * 4 + kb holds channels 32 kb + 8 jj + e: this lane's 8
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) word |= u[e] << (4 * (4 * (e & 1) + (e >> 1)));
        const int kb = l16 >> 2, jj = l16 & 3;
        reinterpret_cast<uint32_t*>(a.kv.k_codes + (size_t)slot * (kHd / 2))[jj * 4 + kb] = word;
        if (l16 == 0) a.kv.k_scales[slot] = s16;
      } else {
        uint32_t c0 = 0, c1 = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c0 |= u[e] << (8 * e);
          c1 |= u[e + 4] << (8 * e);
        }
        *reinterpret_cast<u32x2_t*>(vcodes + ((size_t)tloc * nvh + vslot(hl)) * kHd + 8 * l16) = u32x2_t{c0, c1};
        if (l16 == 0) a.kv.v_scales[slot] = s16;
      }
    }
    lds_barrier();
  }

  // Value blocks: a dword holds one channel of the 8 tokens w = 4jj + e and
  // 16 + 4jj + e (e = 0..3) of a 32-token block.  Wave 0 lists one
  // representative token per such group present in the tile (the group's
  // first token here) with the mask of its members present in the tile and
  // request; then every thread builds dwords of (representative, channel)
  // items independently: stored whole when all 8 members are present, else
  // merged nibble-wise with an atomic and/or.
  int* rep_list = reinterpret_cast<int*>(ybuf);  // [kTokPerWg] (tloc | mask << 8), then the count
  if (nvh > 0) {
    if (wave == 0) {
      int base = 0;
#pragma unroll
      for (int half = 0; half < kTokPerWg / 64; ++half) {
        const int tloc = half * 64 + lane;
        const TokInfo ti = tinfo[tloc];
        int entry = -1;
        if (ti.pos >= 0) {
          const int w = ti.pos & 31;
          const int off = (w & 3) + (w >= 16 ? 16 : 0);  // distance from the group's first position
          const int t0 = tloc - off;
          int mask = 0, first = -1;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int o = (q < 4) ? q : 12 + q;
            const bool present = t0 + o >= ti.lo && t0 + o < ti.hi;
            mask |= present ? (1 << q) : 0;
            if (present && first < 0) first = o;
          }
          if (first == off) entry = tloc | (mask << 8);
        }
        const uint64_t bal = __ballot(entry >= 0);
        const int idx = base + __popcll(bal & ((1ull << lane) - 1ull));
        if (entry >= 0) rep_list[idx] = entry;
        base += __popcll(bal);
      }
      if (lane == 0) rep_list[kTokPerWg] = base;
    }
    lds_barrier();
    const int nrep = rep_list[kTokPerWg];
    const int nitems = nrep * kHd * nvh;
#pragma unroll 4
    for (int item = tid; item < nitems; item += kThreads) {
      const int ch = item % kHd;
      const int rh = item / kHd;
      const int hl = nvh == 2 ? rh % 2 : hv1;  // the v head
      const int entry = rep_list[rh / nvh];
      const int tloc = entry & 0xFF, mask = entry >> 8;
      const TokInfo ti = tinfo[tloc];
      const int w = ti.pos & 31;
      const int jj = (w & 15) >> 2;
      const int t0 = tloc - ((w & 3) + (w >= 16 ? 16 : 0));
      const int kvh = (hl ? heads.y : heads.x) - a.n_q - a.n_kv;
      const int64_t reg = ti.base + (int64_t)kvh * ti.cap;
      uint32_t* dw = a.kv.v_codes + (size_t)(reg / 32 + ti.pos / 32) * 4 * kHd + jj * kHd + (ch % 16) * (kHd / 16) +
                     ch / 16;
      uint32_t word = 0, keep = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int o = (q < 4) ? q : 12 + q;
        const int sh = 4 * (4 * (q & 1) + (q >> 1));
        if (mask & (1 << q)) {
          word |= (uint32_t)vcodes[((size_t)(t0 + o) * nvh + vslot(hl)) * kHd + ch] << sh;
        } else {
          keep |= 0xFu << sh;
        }
      }
      if (mask == 0xFF) {
        *dw = word;
      } else {
        atomicAnd(dw, keep);
        atomicOr(dw, word);
      }
    }
  }

#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) qmax = fmaxf(qmax, lane_xor(qmax, o, lane));
  if (lane == 0 && qmax > 0.f) atomic_max_pos(&a.sc->q_amax, qmax);
}

__global__ void fp8_scales_update_kernel(i4d_fp8_scales* s) {
  if (threadIdx.x != 0) return;
  const float ax = s->x_amax, aq = s->q_amax;
  if (ax > 0.f) s->x_scale = __fdiv_rn(ax, 448.0f);
  if (aq > 0.f) s->q_scale = __fdiv_rn(aq, 448.0f);
  s->x_amax = 0.f;
  s->q_amax = 0.f;
}

struct PrefillWs {
  size_t x8, sumsq, map, rope, total;
  int Tpad, nch;
};

PrefillWs prefill_ws(const i4d_layer_shape& s, int T) {
  PrefillWs w;
  w.Tpad = ((T + kTokPerWg - 1) / kTokPerWg) * kTokPerWg;
  w.nch = (groups_of(s.d_model) + kPrepGroups - 1) / kPrepGroups;
  size_t o = 0;
  w.x8 = o;
  o = align256(o + (size_t)w.Tpad * s.d_model);
  w.sumsq = o;
  o = align256(o + (size_t)w.nch * w.Tpad * sizeof(float));
  w.map = o;
  o = align256(o + (size_t)w.Tpad * sizeof(int2));
  w.rope = o;
  o = align256(o + (size_t)w.Tpad * 64 * sizeof(float2));
  w.total = o;
  return w;
}

i4d_status check_prefill_shape(const i4d_layer_shape* s) {
  if (!s) return fail(I4D_ERR_NULL, "shape is NULL");
  i4d_status st = check_shape(s);
  if (st != I4D_OK) return st;
  if (s->head_dim != kHd) return fail(I4D_ERR_UNSUPPORTED, "the FP8 prefill takes head_dim 128 (got %d)", s->head_dim);
  if (s->n_q_heads % 2 || s->n_kv_heads % 2)
    return fail(I4D_ERR_UNSUPPORTED, "the FP8 prefill takes even numbers of q and kv heads (%d, %d)", s->n_q_heads,
                s->n_kv_heads);
  return ok();
}

}  // namespace

}  // namespace i4d

using namespace i4d;

extern "C" i4d_status i4d_prefill_workspace_bytes(const i4d_layer_shape* shape, int T, size_t* bytes) {
  i4d_status st = check_prefill_shape(shape);
  if (st != I4D_OK) return st;
  if (T < 0) return fail(I4D_ERR_RANGE, "T=%d", T);
  if (!bytes) return fail(I4D_ERR_NULL, "bytes is NULL");
  *bytes = prefill_ws(*shape, T).total;
  return ok();
}

namespace i4d {
namespace {

// host checks shared by the three entry points; fills `a` (workspace
// pointers included) and the workspace layout
i4d_status prefill_args(const i4d_prefill_weights* layer, const i4d_kv_cache* cache, const uint16_t* x, int T,
                        const int32_t* cu_seqlens, const int32_t* start_pos, int R, i4d_fp8_scales* scales,
                        void* workspace, size_t workspace_bytes, bool need_x, PrefillArgs* a, PrefillWs* w) {
  if (!layer) return fail(I4D_ERR_NULL, "layer is NULL");
  const i4d_layer_shape& s = layer->shape;
  i4d_status st = check_prefill_shape(&s);
  if (st != I4D_OK) return st;
  if ((st = need(layer->qkv_codes, "qkv_codes")) != I4D_OK) return st;
  if ((st = need(layer->qkv_scales, "qkv_scales")) != I4D_OK) return st;
  if (T < 0) return fail(I4D_ERR_RANGE, "T=%d", T);
  if (R < 1) return fail(I4D_ERR_RANGE, "R=%d requests", R);
  if ((st = check_cache(cache, &s, R)) != I4D_OK) return st;
  if (!cu_seqlens || !start_pos) return fail(I4D_ERR_NULL, "cu_seqlens / start_pos is NULL");
  if (!scales) return fail(I4D_ERR_NULL, "scales is NULL");
  if (need_x && T > 0 && (st = need(x, "x")) != I4D_OK) return st;
  *w = prefill_ws(s, T);
  if (T > 0) {
    if ((st = need(workspace, "workspace")) != I4D_OK) return st;
    if (workspace_bytes < w->total)
      return fail(I4D_ERR_WORKSPACE, "prefill workspace %zu bytes < %zu", workspace_bytes, w->total);
  }
  *a = PrefillArgs{};
  a->codes = (const uint8_t*)layer->qkv_codes;
  a->scales = layer->qkv_scales;
  a->N = (s.n_q_heads + 2 * s.n_kv_heads) * kHd;
  a->K = s.d_model;
  a->G = groups_of(s.d_model);
  a->n_q = s.n_q_heads;
  a->n_kv = s.n_kv_heads;
  a->eps = s.rms_eps;
  a->rope_ratio = pow((double)s.rope_theta, -2.0 / (double)s.head_dim);
  a->x = x;
  a->T = T;
  a->Tpad = w->Tpad;
  a->R = R;
  a->nch = w->nch;
  a->cu = cu_seqlens;
  a->start = start_pos;
  a->sc = scales;
  a->kv = kv_args(cache);
  char* ws = (char*)workspace;
  a->x8 = (uint8_t*)(ws + w->x8);
  a->sumsq = (float*)(ws + w->sumsq);
  a->map = (int2*)(ws + w->map);
  a->rope = (float2*)(ws + w->rope);
  return ok();
}

i4d_status launch_prep(const PrefillArgs& a, const PrefillWs& w, hipStream_t hs) {
  hipLaunchKernelGGL(prefill_prep_kernel, dim3(w.Tpad / 16, w.nch), dim3(256), 0, hs, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(I4D_ERR_HIP, "prefill prep launch: %s", hipGetErrorString(e));
  return ok();
}

i4d_status launch_gemm(PrefillArgs a, const PrefillWs& w, uint8_t* q_fp8, uint16_t* k_bf16, uint16_t* v_bf16,
                       hipStream_t hs) {
  i4d_status st = need(q_fp8, "q_fp8");
  if (st != I4D_OK) return st;
  if (k_bf16 && !aligned16(k_bf16)) return fail(I4D_ERR_ALIGN, "k_bf16 is not 16-byte aligned");
  if (v_bf16 && !aligned16(v_bf16)) return fail(I4D_ERR_ALIGN, "v_bf16 is not 16-byte aligned");
  a.q8 = q_fp8;
  a.k_bf16 = k_bf16;
  a.v_bf16 = v_bf16;
  const int grid = (a.N / kRowsPerWg) * (w.Tpad / kTokPerWg);
  hipLaunchKernelGGL(prefill_gemm_kernel, dim3(grid), dim3(kThreads), kGemmLds, hs, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(I4D_ERR_HIP, "prefill gemm launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace
}  // namespace i4d

extern "C" i4d_status i4d_prefill_prepare(const i4d_prefill_weights* layer, const i4d_kv_cache* cache, const uint16_t* x, int T,
                                          const int32_t* cu_seqlens, const int32_t* start_pos, int R,
                                          i4d_fp8_scales* scales, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  PrefillArgs a;
  PrefillWs w;
  i4d_status st = prefill_args(layer, cache, x, T, cu_seqlens, start_pos, R, scales, workspace, workspace_bytes,
                               true, &a, &w);
  if (st != I4D_OK || T == 0) return st;
  return launch_prep(a, w, (hipStream_t)stream);
}

extern "C" i4d_status i4d_prefill_project(const i4d_prefill_weights* layer, const i4d_kv_cache* cache, int T,
                                          const int32_t* cu_seqlens, const int32_t* start_pos, int R,
                                          i4d_fp8_scales* scales, uint8_t* q_fp8, uint16_t* k_bf16,
                                          uint16_t* v_bf16, const void* workspace, size_t workspace_bytes,
                                          void* stream) {
  PrefillArgs a;
  PrefillWs w;
  i4d_status st = prefill_args(layer, cache, nullptr, T, cu_seqlens, start_pos, R, scales, (void*)workspace,
                               workspace_bytes, false, &a, &w);
  if (st != I4D_OK || T == 0) return st;
  return launch_gemm(a, w, q_fp8, k_bf16, v_bf16, (hipStream_t)stream);
}

extern "C" i4d_status i4d_prefill_qkv_e4m3(const i4d_prefill_weights* layer, const i4d_kv_cache* cache, const uint16_t* x,
                                           int T, const int32_t* cu_seqlens, const int32_t* start_pos, int R,
                                           i4d_fp8_scales* scales, uint8_t* q_fp8, uint16_t* k_bf16,
                                           uint16_t* v_bf16, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  PrefillArgs a;
  PrefillWs w;
  i4d_status st = prefill_args(layer, cache, x, T, cu_seqlens, start_pos, R, scales, workspace, workspace_bytes,
                               true, &a, &w);
  if (st != I4D_OK || T == 0) return st;
  // the output pointers are checked before anything is enqueued
  if ((st = need(q_fp8, "q_fp8")) != I4D_OK) return st;
  if (k_bf16 && !aligned16(k_bf16)) return fail(I4D_ERR_ALIGN, "k_bf16 is not 16-byte aligned");
  if (v_bf16 && !aligned16(v_bf16)) return fail(I4D_ERR_ALIGN, "v_bf16 is not 16-byte aligned");
  hipStream_t hs = (hipStream_t)stream;
  if ((st = launch_prep(a, w, hs)) != I4D_OK) return st;
  return launch_gemm(a, w, q_fp8, k_bf16, v_bf16, hs);
}

extern "C" i4d_status i4d_fp8_scales_update(i4d_fp8_scales* scales, void* stream) {
  if (!scales) return fail(I4D_ERR_NULL, "scales is NULL");
  hipLaunchKernelGGL(fp8_scales_update_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, scales);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(I4D_ERR_HIP, "scale update launch: %s", hipGetErrorString(e));
  return ok();
}
